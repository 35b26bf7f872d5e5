"""Canary-guarded outputs: every buffer the library writes is handed over as the
head of a larger allocation whose tail holds sentinels, and the sentinels must
come back untouched (no write past out_tokens, accepted_count, the diagnostics,
the sampled tokens, the tree's node list or the workspace).  The outputs
themselves are checked against the oracle as in the parity tests."""
import numpy as np
import pytest

from rejection_sampling_verification_spec_amd import workloads as W

from ._parity import GpuResult, check_parity, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SENT_I = -123456789
SENT_B = 0x5A


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rejection_sampling_verification_spec_amd as sv
    sv.load_library()


def guarded(shape, dtype, fill, dev):
    """(buffer with one more leading row, its head view of `shape`)."""
    buf = torch.full((shape[0] + 1, *shape[1:]), fill, dtype=dtype, device=dev)
    return buf, buf[:shape[0]]


def guarded_ws(nbytes, dev):
    buf = torch.full((nbytes + 4096,), SENT_B, dtype=torch.uint8, device=dev)
    assert buf.data_ptr() % 256 == 0
    return buf, buf[:nbytes]


def tail_ok(buf, rows, fill):
    return bool(torch.all(buf[rows:] == fill).item())


# V = 1000: requests of at most 12288 logits, verified by one workgroup each
@pytest.mark.parametrize("V", [5003, 1000], ids=["two_kernels", "one_workgroup"])
@pytest.mark.parametrize("entry", ["spec_verify", "spec_verify_ex", "spec_verify_filtered", "spec_verify_noalloc"])
def test_no_write_past_the_outputs(entry, V):
    import oracle
    import rejection_sampling_verification_spec_amd as sv
    dev = torch.device("cuda:0")
    if entry in ("spec_verify", "spec_verify_noalloc"):
        w = W.make_random(501, 6, 4, V, "bf16", temps=0.9, zipf=True)
    else:
        w = W.make_random(502, 7, 5, V - 904, "bf16", temps=np.array([0, 1, 0.6, 1.3, 0, 1, 0.8], np.float32),
                          lens=np.array([5, 0, 3, 5, 2, 4, 1], np.int32), zipf=True)
        w.scalar_temperature = None
    if entry == "spec_verify_filtered":
        w.top_k = np.array([0, 5, 40, 0, 3, 100, 0], np.int32)
        w.top_p = np.array([0.9, 1.0, 0.95, 0.8, 1.0, 0.99, 0.5], np.float32)
    t = w.to_torch(dev)
    B, g = w.B, w.gamma
    cbuf, cnt = guarded((B,), torch.int32, SENT_I, dev)
    obuf, out = guarded((B, g + 1), torch.int32, SENT_I, dev)
    say(f"canary {entry} B={B} gamma={g} V={w.V}")
    if entry == "spec_verify":
        wsb, ws = guarded_ws(sv.spec_verify_workspace_bytes(B, g, w.V, sv.SV_BF16), dev)
        sv.spec_verify(t["target"], t["draft"], t["draft_tokens"], t["u_accept"], t["u_sample"],
                       float(w.scalar_temperature), accepted_count=cnt, out_tokens=out, workspace=ws)
    elif entry == "spec_verify_noalloc":
        wsb, ws = None, None
        sv.spec_verify_noalloc(t["target"], t["draft"], t["draft_tokens"], t["u_accept"], t["u_sample"],
                               float(w.scalar_temperature), accepted_count=cnt, out_tokens=out)
    else:
        rows = 2 * g + 1
        dbgbufs = {"p_draft": guarded((B, g), torch.float64, 7.5, dev), "q_draft": guarded((B, g), torch.float64, 7.5, dev),
                   "accept_prob": guarded((B, g), torch.float64, 7.5, dev),
                   "row_max": guarded((B, rows), torch.float32, 7.5, dev),
                   "row_sum": guarded((B, rows), torch.float64, 7.5, dev),
                   "row_argmax": guarded((B, g + 1), torch.int32, SENT_I, dev),
                   "residual_mass": guarded((B,), torch.float64, 7.5, dev)}
        dbg = {k: v[1] for k, v in dbgbufs.items()}
        if entry == "spec_verify_ex":
            wsb, ws = guarded_ws(sv.spec_verify_workspace_bytes(B, g, w.V, sv.SV_BF16), dev)
            sv.spec_verify_ex(t["target"], t["draft"], t["draft_tokens"], t["u_accept"], t["u_sample"],
                              t["temperature"], t["lens"], accepted_count=cnt, out_tokens=out, workspace=ws,
                              debug=dbg)
        else:
            wsb, ws = guarded_ws(sv.spec_verify_filtered_workspace_bytes(B, g, w.V, sv.SV_BF16), dev)
            sv.spec_verify_filtered(t["target"], t["draft"], t["draft_tokens"], t["u_accept"], t["u_sample"],
                                    t["temperature"], t["lens"], top_k=t["top_k"], top_p=t["top_p"],
                                    accepted_count=cnt, out_tokens=out, workspace=ws, debug=dbg)
        torch.cuda.synchronize()
        for k, (buf, _) in dbgbufs.items():
            fill = SENT_I if buf.dtype == torch.int32 else 7.5
            assert tail_ok(buf, B, fill), f"{entry}: write past debug[{k}]"
    torch.cuda.synchronize()
    assert tail_ok(cbuf, B, SENT_I), f"{entry}: write past accepted_count"
    assert tail_ok(obuf, B, SENT_I), f"{entry}: write past out_tokens"
    if wsb is not None:
        assert bool(torch.all(wsb[ws.numel():] == SENT_B).item()), f"{entry}: write past the workspace"
    o = oracle.run_workload(w)
    check_parity(w, GpuResult(cnt.cpu().numpy(), out.cpu().numpy()), o, require_no_flags=False)


def test_no_write_past_the_sampler_and_tree_outputs():
    import oracle
    import rejection_sampling_verification_spec_amd as sv
    dev = torch.device("cuda:0")
    # draft-side sampler
    R, V = 37, 4099
    rng = np.random.default_rng(503)
    z = (rng.standard_normal((R, V)) * 2.0).astype(np.float32)
    u = rng.random(R, dtype=np.float32)
    tbuf, toks = guarded((R,), torch.int32, SENT_I, dev)
    wsb, ws = guarded_ws(sv.spec_sample_workspace_bytes(R, V, sv.SV_F32), dev)
    sv.spec_sample(torch.from_numpy(z).to(dev), torch.from_numpy(u).to(dev), 0.8, tokens=toks, workspace=ws)
    torch.cuda.synchronize()
    assert tail_ok(tbuf, R, SENT_I) and bool(torch.all(wsb[ws.numel():] == SENT_B).item())
    ref, tr = oracle.sample(z, u, 0.8)
    ok = tr.flags == 0
    np.testing.assert_array_equal(toks.cpu().numpy()[ok], ref[ok])
    # tree verification
    tw = W.build_tree("canary_tree", 504, 5, 3, 2, 3001, "bf16", target_scale=3.0, zipf=True, sigma=0.6,
                      temps=np.array([1.0, 0.0, 0.7, 1.0, 0.5], np.float32))
    tt = tw.to_torch(dev)
    B, N = tw.B, tw.N
    cbuf, cnt = guarded((B,), torch.int32, SENT_I, dev)
    obuf, out = guarded((B, N + 1), torch.int32, SENT_I, dev)
    nbuf, nodes = guarded((B, N), torch.int32, SENT_I, dev)
    wsb, ws = guarded_ws(sv.spec_verify_tree_workspace_bytes(B, N, tw.V, sv.SV_BF16), dev)
    sv.spec_verify_tree(tt["target"], tt["draft"], tt["parent"], tt["tokens"], tt["u_accept"], tt["u_sample"],
                        tt["temperature"], num_nodes=tt["num_nodes"], accepted_count=cnt, out_tokens=out,
                        out_nodes=nodes, workspace=ws)
    torch.cuda.synchronize()
    for buf, rows, name in ((cbuf, B, "accepted_count"), (obuf, B, "out_tokens"), (nbuf, B, "out_nodes")):
        assert tail_ok(buf, rows, SENT_I), f"tree: write past {name}"
    assert bool(torch.all(wsb[ws.numel():] == SENT_B).item()), "tree: write past the workspace"
    o = oracle.spec_verify_tree(tw.target, tw.draft, tw.parent, tw.tokens, tw.u_accept, tw.u_sample, tw.temperature,
                                num_nodes=tw.num_nodes, dtype=tw.dtype)
    ok = o.flags == 0
    np.testing.assert_array_equal(cnt.cpu().numpy()[ok], o.accepted_count[ok])
    np.testing.assert_array_equal(out.cpu().numpy()[ok], o.out_tokens[ok])
