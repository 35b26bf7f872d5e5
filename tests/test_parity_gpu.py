"""GPU parity: libspecverify (HIP, through the C ABI) against the CPU oracle.

Bar: accepted counts and tokens bit-exact on every request the oracle does not
flag as near-boundary: |u - a| < 1e-6 at a decided position (bit 0), u_sample
within 1e-6 of the sampled token's interval ends on the normalised CDF (bit 1),
the zero-mass fallback (bit 2), or the same CDF distance below 1e-6 in
probability units, i.e. multiplied by the residual's mass Z (bit 4).  The
number of flagged requests must be 0 on the five workloads; no case may excuse
more than half of its requests; greedy requests fully bit-exact; probabilities
within 1e-5 (fp32 logits) / 2e-3 (bf16 logits).
"""
import json
import os
import zlib

import numpy as np
import pytest

from rejection_sampling_verification_spec_amd import workloads as W

from ._parity import check_parity, gpu_run, run_and_check, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rejection_sampling_verification_spec_amd as sv
    sv.load_library()


# ------------------------------------------------------------------ the five workloads
@pytest.mark.parametrize("cfg,greedy", [(0, False), (1, False), (2, False), (3, False), (3, True), (4, False)])
def test_workload_parity(cfg, greedy):
    w = W.make_config(cfg, greedy=greedy)
    rep = run_and_check(w, debug=True)
    assert rep["flagged"] == 0
    if w.lens is None:
        # the uniform entry point (what the benchmark times) gives the same outputs
        say(f"{w.name} via spec_verify")
        g = gpu_run(w, debug=False)
        import oracle
        check_parity(w, g, oracle.run_workload(w))


def test_workload3_deterministic():
    w = W.make_config(3)
    a = gpu_run(w, debug=True)
    b = gpu_run(w, debug=True)
    np.testing.assert_array_equal(a.count, b.count)
    np.testing.assert_array_equal(a.out, b.out)
    for k in a.dbg:
        np.testing.assert_array_equal(a.dbg[k], b.dbg[k])


# ------------------------------------------------------------------ random shapes
SHAPES = [
    # (B, gamma, V, dtype)
    (1, 0, 1, "f32"), (3, 1, 1, "bf16"), (2, 1, 7, "f32"), (5, 8, 7, "bf16"), (4, 3, 64, "f32"),
    (3, 31, 64, "bf16"), (2, 32, 1000, "f32"), (5, 8, 1000, "bf16"), (4, 1, 4099, "f32"),
    (3, 5, 4099, "bf16"), (2, 4, 16384, "bf16"), (2, 4, 16385, "f32"), (3, 2, 40000, "bf16"),
    (2, 3, 70001, "f32"), (6, 0, 3000, "bf16"),
    # sub-chunk boundaries: one whole 2048-token sub-chunk, one plus a single
    # token, three whole ones
    (3, 3, 2048, "bf16"), (3, 3, 2049, "bf16"), (2, 2, 6144, "f32"),
]


@pytest.mark.parametrize("B,gamma,V,dtype", SHAPES)
@pytest.mark.parametrize("mode", ["uniform", "mixed"])
def test_random_shapes(B, gamma, V, dtype, mode):
    seed = zlib.crc32(repr((B, gamma, V, dtype, mode)).encode()) % 100000
    rng = np.random.default_rng(seed)
    if mode == "uniform":
        w = W.make_random(seed, B, gamma, V, dtype, temps=0.8, target_scale=3.0, sigma=0.7,
                          zipf=V > 100)
    else:
        temps = rng.choice(np.array([0.0, 0.6, 1.0, 1.7], np.float32), size=B)
        lens = rng.integers(0, gamma + 1, size=B).astype(np.int32)
        w = W.make_random(seed, B, gamma, V, dtype, temps=temps, lens=lens, target_scale=4.0,
                          sigma=1.0, zipf=V > 100)
    run_and_check(w, debug=True, require_no_flags=False)
    run_and_check(w, debug=False, require_no_flags=False)


# The draw runs inside the decision kernel when a request has at most 512
# sub-chunks: drawn by the workgroup that computed the chosen sub-chunk's mass
# while the decision kernel's grid (B times the workgroups per request) fits
# the chip at once (1024 workgroups for bf16 rows, 512 for fp32), by
# workgroup 0 of the request beyond that; V = 2^20 (512 sub-chunks) is the
# largest fused case.  The three-kernel path (more sub-chunks) is covered by
# test_large_vocabulary.
DRAW_PATHS = [
    # (B, gamma, V, dtype): workgroups of the decision kernel
    (64, 2, 128256, "bf16"),   # 1024: every workgroup of a request waits
    (65, 2, 128256, "bf16"),   # 1040: workgroup 0 draws
    (128, 2, 32000, "f32"),    # 512
    (129, 2, 32000, "f32"),    # 516
    (2, 2, 1 << 20, "bf16"),   # 512 sub-chunks in workgroup 0's list
]


@pytest.mark.parametrize("B,gamma,V,dtype", DRAW_PATHS)
def test_draw_paths(B, gamma, V, dtype):
    seed = zlib.crc32(repr((B, gamma, V, dtype, "draw")).encode()) % 100000
    rng = np.random.default_rng(seed)
    temps = rng.choice(np.array([0.0, 0.7, 1.0], np.float32), size=B)
    lens = rng.integers(0, gamma + 1, size=B).astype(np.int32)
    w = W.make_random(seed, B, gamma, V, dtype, temps=temps, lens=lens, target_scale=4.0, sigma=0.8,
                      zipf=True)
    say(f"draw path B={B} gamma={gamma} V={V} {dtype}")
    run_and_check(w, debug=True, require_no_flags=False)
    w = W.make_random(seed + 1, B, gamma, V, dtype, temps=1.0, target_scale=3.0, sigma=0.7, zipf=True)
    run_and_check(w, debug=False, require_no_flags=False)


@pytest.mark.parametrize("dtype,mode", [("bf16", "uniform"), ("f32", "mixed")])
def test_large_vocabulary(dtype, mode):
    """V = 2^20 + 3: 513 sub-chunks per row (the selection scans the sub-chunk masses
    in nine batches of 64; the last sub-chunk holds three tokens) and many K1 chunks
    per row."""
    V = (1 << 20) + 3
    seed = 4100 + (mode == "mixed")
    if mode == "uniform":
        w = W.make_random(seed, 3, 3, V, dtype, temps=1.0, target_scale=4.0, sigma=0.5, zipf=True)
    else:
        w = W.make_random(seed, 4, 3, V, dtype, temps=np.array([0.0, 0.7, 1.0, 1.3], np.float32),
                          lens=np.array([3, 1, 3, 2], np.int32), target_scale=4.0, sigma=0.8, zipf=True)
    say(f"large vocabulary {dtype} {mode} V={V}")
    run_and_check(w, debug=True, require_no_flags=False)


@pytest.mark.parametrize("B,gamma,V", [(16, 4, 5000), (6, 3, 128256), (5, 2, 100003)])
def test_greedy_ties_lowest_index(B, gamma, V):
    """Greedy rows with many exact ties (the lowest index wins), across several
    chunks and whole tiles at the larger sizes (V = 100003 rows are not 16-byte
    aligned); one target row is -inf throughout (its arg-max is token 0) and one
    is -inf except for a tie of two finite logits late in the row."""
    rng = np.random.default_rng(V)
    zp = rng.integers(-2, 3, size=(B, gamma + 1, V)).astype(np.float32)  # many exact ties
    zp[1, 1] = -np.inf
    zp[2, 0] = -np.inf
    zp[2, 0, V - 5] = zp[2, 0, V - 2] = -7.0
    zq = zp[:, :gamma] + rng.integers(-1, 2, size=(B, gamma, V)).astype(np.float32)
    zq[1, 1] = 0.0
    zq[2, 0] = 0.0
    tok = np.argmax(zq, axis=2)
    tok[1, 1] = 0
    tok[2, 0] = V - 5
    for dtype in ("f32", "bf16"):
        say(f"greedy ties {dtype} B={B} gamma={gamma} V={V}")
        w = W.from_logits(zp, zq, tok, np.zeros((B, gamma)), np.zeros(B), 0.0, dtype=dtype)
        rep = run_and_check(w, debug=True)
        assert rep["flagged"] == 0


# ------------------------------------------------------------------ one workgroup per request
# A request whose (2 gamma + 1) V logits fit 12288 (48 KB of LDS) is verified by
# one workgroup, in one kernel; one logit more takes the two-kernel path.
SMALL = [
    # (B, gamma, V, dtype)
    (1, 4, 1000, "f32"),     # the B = 1, gamma = 4, V = 1000 fp32 shape
    (3, 5, 1117, "bf16"),    # 11 * 1117 = 12287
    (2, 0, 12288, "f32"),    # one row of 12288 logits: the limit
    (2, 0, 12289, "f32"),    # one logit more: the two-kernel path
    (4, 1, 4096, "bf16"),    # 3 * 4096 = 12288
    (200, 2, 512, "bf16"),   # many requests
    (5, 32, 100, "f32"),     # the longest drafts
    (7, 6, 511, "bf16"),     # rows that are not 16-byte aligned
]


@pytest.mark.parametrize("B,gamma,V,dtype", SMALL)
@pytest.mark.parametrize("mode", ["uniform", "mixed", "greedy"])
def test_small_problems(B, gamma, V, dtype, mode):
    seed = zlib.crc32(repr((B, gamma, V, dtype, mode, "small")).encode()) % 100000
    rng = np.random.default_rng(seed)
    if mode == "uniform":
        w = W.make_random(seed, B, gamma, V, dtype, temps=0.9, target_scale=3.0, sigma=0.7, zipf=V > 100)
    elif mode == "greedy":
        w = W.make_random(seed, B, gamma, V, dtype, temps=0.0, target_scale=3.0, sigma=0.7, zipf=V > 100)
    else:
        temps = rng.choice(np.array([0.0, 0.6, 1.0, 1.7], np.float32), size=B)
        lens = rng.integers(0, gamma + 1, size=B).astype(np.int32)
        w = W.make_random(seed, B, gamma, V, dtype, temps=temps, lens=lens, target_scale=4.0, sigma=1.0,
                          zipf=V > 100)
    say(f"small problem B={B} gamma={gamma} V={V} {dtype} {mode}")
    run_and_check(w, debug=True, require_no_flags=False)
    run_and_check(w, debug=False, require_no_flags=False)


def test_small_problem_misaligned_rows():
    """The one-workgroup path reads element by element: rows only 2-byte aligned."""
    w = W.make_random(9, 6, 4, 1000, "bf16", temps=np.array([1.0, 0.0, 0.7, 1.3, 0.0, 2.0], np.float32),
                      zipf=True)
    import oracle
    import rejection_sampling_verification_spec_amd as sv
    o = oracle.run_workload(w)
    dev = torch.device("cuda:0")
    t = w.to_torch(dev)

    def shifted(x):
        buf = torch.empty(x.numel() + 1, dtype=x.dtype, device=dev)
        v = buf[1:].view(x.shape)
        v.copy_(x)
        return v
    count, out = sv.spec_verify_ex(shifted(t["target"]), shifted(t["draft"]), t["draft_tokens"], t["u_accept"],
                                   t["u_sample"], t["temperature"])
    torch.cuda.synchronize()
    ok = o.flags == 0
    assert ok.sum() >= w.B // 2
    np.testing.assert_array_equal(count.cpu().numpy()[ok], o.accepted_count[ok])
    np.testing.assert_array_equal(out.cpu().numpy()[ok], o.out_tokens[ok])


# ------------------------------------------------------------------ the pins' inputs through the library
def _lnp(p):
    p = np.asarray(p, dtype=np.float64)
    z = np.full(p.shape, -1000.0)
    z[p > 0] = np.log(p[p > 0])
    return z.astype(np.float32)


def test_t1_enumeration_through_library():
    p, q = np.array([1, 2, 3, 2]) / 8, np.array([2, 1, 1, 4]) / 8
    grid = (2 * np.arange(6) + 1) / 12.0
    xs, ua, us = (a.ravel() for a in np.meshgrid(np.arange(4), grid, grid, indexing="ij"))
    B = xs.size
    target = np.stack([np.broadcast_to(_lnp(p), (B, 4)), np.broadcast_to(_lnp([.2, .2, .2, .4]), (B, 4))], 1)
    draft = np.broadcast_to(_lnp(q), (B, 1, 4)).copy()
    for dtype in ("f32", "bf16"):
        w = W.from_logits(target, draft, xs[:, None], ua[:, None], us, 1.0, dtype=dtype, name=f"T1_{dtype}")
        run_and_check(w, debug=True)
        g = gpu_run(w)
        marg = np.zeros(4)
        np.add.at(marg, g.out[:, 0], q[xs] / 36.0)
        if dtype == "f32":
            np.testing.assert_allclose(marg, p, atol=1e-14)


def test_t2_grid_through_library():
    gamma = 3
    grid10 = (2 * np.arange(10) + 1) / 20.0
    idx = np.indices((10,) * gamma).reshape(gamma, -1).T
    B = idx.shape[0]
    w = W.from_logits(np.broadcast_to(_lnp([0.63, 0.37]), (B, gamma + 1, 2)),
                      np.broadcast_to(_lnp([0.9, 0.1]), (B, gamma, 2)), np.zeros((B, gamma), int),
                      grid10[idx], np.full(B, 0.5), 1.0, name="T2_grid")
    run_and_check(w, debug=True)
    g = gpu_run(w)
    assert abs((g.count + 1).mean() - (1 - 0.7 ** (gamma + 1)) / 0.3) < 1e-12


def test_t3_greedy_worked_example_through_library():
    gd = json.load(open(os.path.join(GOLDEN, "greedy_worked_example.json")))
    V, gamma = gd["V"], gd["gamma"]
    cases = gd["cases"]
    B = len(cases)
    target = np.zeros((B, gamma + 1, V), np.float32)
    for i, t in enumerate(gd["target_argmax"]):
        target[:, i, t] = 5.0
    tokens = np.array([c["drafts"] for c in cases])
    for dtype in ("f32", "bf16"):
        w = W.from_logits(target, np.zeros((B, gamma, V), np.float32), tokens, np.zeros((B, gamma)),
                          np.zeros(B), 0.0, dtype=dtype, name=f"T3_{dtype}")
        g = gpu_run(w)
        np.testing.assert_array_equal(g.count, [c["accepted_count"] for c in cases])
        np.testing.assert_array_equal(g.out, [c["out_tokens"] for c in cases])


# ------------------------------------------------------------------ edge cases
def test_zero_residual_mass_fallback():
    rng = np.random.default_rng(1)
    V = 3000
    z = rng.standard_normal(V).astype(np.float32)
    B = 7
    us = ((np.arange(B) + 0.5) / B).astype(np.float32)
    w = W.from_logits(np.broadcast_to(z, (B, 2, V)), np.broadcast_to(z, (B, 1, V)),
                      np.full((B, 1), 3), np.ones((B, 1)), us, 1.0, name="zero_mass")
    import oracle
    o = oracle.run_workload(w)
    assert np.all(o.flags & 4)
    g = gpu_run(w)
    np.testing.assert_array_equal(g.count, o.accepted_count)
    np.testing.assert_array_equal(g.out, o.out_tokens)


@pytest.mark.parametrize("dtype,temps,scale", [
    ("f32", 1e-3, 3.0),                                              # nearly one-hot rows
    ("bf16", 1e-2, 40.0),                                            # logits up to about +-150
    ("f32", 50.0, 3.0),                                              # nearly uniform rows
    ("bf16", np.array([1e-3, 0.05, 1.0, 20.0, 0.0, 3.0, 0.2, 7.0], np.float32), 8.0),
], ids=["T1e-3_f32", "T1e-2_bf16_large_logits", "T50_f32", "mixed_extremes_bf16"])
def test_extreme_temperatures(dtype, temps, scale):
    """Temperatures from 1e-3 to 50 (and greedy rows among them), with logits up to
    about 150 in magnitude: y = z log2(e) / T - M reaches -1e5 and the integer M 1e5."""
    w = W.make_random(4242, 8, 4, 5003, dtype, temps=temps, target_scale=scale, sigma=0.5, zipf=True)
    rep = run_and_check(w, debug=True, require_no_flags=False)
    assert rep["flagged"] <= 1


def test_identical_rows_accept_all():
    w = W.make_random(77, 8, 6, 20000, "bf16", temps=0.9, zipf=True)
    w.draft[:] = w.target[:, :6]
    g = gpu_run(w)
    assert np.all(g.count == 6)
    run_and_check(w, debug=True, require_no_flags=False)


def test_greedy_requests_never_read_draft_rows():
    w = W.make_random(31, 12, 5, 9000, "bf16", temps=np.array([0.0, 1.0] * 6, np.float32), zipf=True)
    import oracle
    o = oracle.run_workload(w)
    w.draft[w.temperature == 0] = W.BF16_NAN      # poison what greedy requests must not read
    w.u_accept[w.temperature == 0] = np.nan
    check_parity(w, gpu_run(w, debug=True), o, require_no_flags=False)


def test_misaligned_rows_and_workspace_garbage():
    w = W.make_random(5, 3, 4, 3001, "bf16", temps=1.0, zipf=True)
    import oracle
    o = oracle.run_workload(w)
    dev = torch.device("cuda:0")
    t = w.to_torch(dev)
    # shift every logit tensor by one element so rows are only 2-byte aligned
    def shifted(x):
        buf = torch.empty(x.numel() + 1, dtype=x.dtype, device=dev)
        v = buf[1:].view(x.shape)
        v.copy_(x)
        return v
    import rejection_sampling_verification_spec_amd as sv
    need = sv.spec_verify_workspace_bytes(w.B, w.gamma, w.V, sv.SV_BF16)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=dev)   # contents on entry must not matter
    say("misaligned bf16 rows")
    count, out = sv.spec_verify(shifted(t["target"]), shifted(t["draft"]), t["draft_tokens"], t["u_accept"],
                                t["u_sample"], 1.0, workspace=ws)
    torch.cuda.synchronize()
    ok = o.flags == 0
    np.testing.assert_array_equal(count.cpu().numpy()[ok], o.accepted_count[ok])
    np.testing.assert_array_equal(out.cpu().numpy()[ok], o.out_tokens[ok])


def test_large_batch_with_the_queried_workspace():
    """B = 1300 requests, 9100 row slots: the unfiltered verify grid takes two chunks
    per row where the default plan takes one, so the size spec_verify_workspace_bytes
    reports must cover the larger plan.  Exactly that many bytes are passed, and a
    sample of the requests (they are independent) is checked against the oracle."""
    import dataclasses

    import oracle
    import rejection_sampling_verification_spec_amd as sv
    w = W.make_random(4242, 1300, 3, 16400, "bf16", temps=1.0)
    nbytes = sv.spec_verify_workspace_bytes(w.B, w.gamma, w.V, sv.SV_BF16)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    g = gpu_run(w, workspace=ws)
    idx = np.array([0, 1, 2, 3, 647, 648, 649, 1296, 1297, 1298, 1299])
    sub = dataclasses.replace(w, name=w.name + "_sample", B=idx.size, target=w.target[idx], draft=w.draft[idx],
                              draft_tokens=w.draft_tokens[idx], u_accept=w.u_accept[idx],
                              u_sample=w.u_sample[idx], temperature=w.temperature[idx])
    gs = type(g)(count=g.count[idx], out=g.out[idx])
    check_parity(sub, gs, oracle.run_workload(sub), require_no_flags=False)


def test_side_stream():
    w = W.make_config(2)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = gpu_run(w, stream=s)
    import oracle
    check_parity(w, g, oracle.run_workload(w))


@pytest.mark.parametrize("cfg", [2, 0], ids=["two_kernels", "one_workgroup"])
def test_graph_replay_matches_eager(cfg):
    """The step captured in a HIP graph (as the benchmark replays it) equals the eager call on every replay."""
    import oracle
    import rejection_sampling_verification_spec_amd as sv
    w = W.make_config(cfg)
    dev = torch.device("cuda:0")
    t = w.to_torch(dev)
    count = torch.empty(w.B, dtype=torch.int32, device=dev)
    out = torch.empty((w.B, w.gamma + 1), dtype=torch.int32, device=dev)
    dt = sv.SV_BF16 if w.dtype == "bf16" else sv.SV_F32
    ws = sv.new_workspace(sv.spec_verify_workspace_bytes(w.B, w.gamma, w.V, dt), dev)
    s = torch.cuda.Stream()

    def call():
        return sv.spec_verify(t["target"], t["draft"], t["draft_tokens"], t["u_accept"], t["u_sample"],
                              float(w.scalar_temperature), accepted_count=count, out_tokens=out,
                              workspace=ws, stream=s)

    with torch.cuda.stream(s):
        call()
    torch.cuda.synchronize()
    ref = (count.cpu().clone(), out.cpu().clone())
    o = oracle.run_workload(w)
    np.testing.assert_array_equal(ref[0].numpy(), o.accepted_count)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    for rep in range(4):
        count.fill_(-5)
        out.fill_(-5)
        ws.fill_(0xAB)                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"graph replay {rep}")
        assert torch.equal(count.cpu(), ref[0]) and torch.equal(out.cpu(), ref[1])


def _verify_fuzz_case(seed, V=None):
    """A small random batch of spec_verify_ex: shape, dtype, ragged lengths, per-request T
    (greedy included) and the logit law (Gaussian, integer ties, one dominant token,
    nearly flat) all drawn; draft tokens half from the draft arg-max, half at random."""
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 9))
    gamma = int(rng.integers(0, 9))
    V = int(rng.choice([1, 2, 5, 64, 999, 4099])) if V is None else V
    dtype = str(rng.choice(["f32", "bf16"]))
    law = str(rng.choice(["normal", "ties", "dominant", "flat"]))
    shape = (B, gamma + 1, V)
    if law == "normal":
        z = rng.standard_normal(shape) * rng.uniform(0.5, 4.0)
    elif law == "ties":
        z = rng.integers(0, 4, size=shape).astype(np.float64)
    elif law == "dominant":
        z = rng.standard_normal(shape) * 2.0
        z[..., int(rng.integers(0, V))] += rng.uniform(5.0, 30.0)
    else:
        z = rng.standard_normal(shape) * 0.05
    z = z.astype(np.float32)
    draft = z[:, :gamma] + rng.standard_normal((B, gamma, V)).astype(np.float32) * np.float32(rng.uniform(0.0, 1.5))
    tokens = rng.integers(0, V, size=(B, gamma)).astype(np.int32)
    am = np.argmax(draft, axis=2) if gamma > 0 else np.zeros((B, 0), np.int64)
    pick = rng.random((B, gamma)) < 0.5
    tokens[pick] = am[pick]
    T = rng.choice(np.array([0.0, 0.4, 1.0, 1.7], np.float32), size=B)
    lens = rng.integers(0, gamma + 1, size=B).astype(np.int32) if gamma > 0 and rng.random() < 0.5 else None
    w = W.from_logits(z, draft, tokens, rng.random((B, gamma)), rng.random(B), T, dtype=dtype, lens=lens,
                      name=f"vfuzz{seed}_{law}")
    w.scalar_temperature = None
    return w


@pytest.mark.parametrize("seed", range(30))
def test_verify_fuzz(seed):
    w = _verify_fuzz_case(3000 + seed)
    rep = run_and_check(w, debug=True, require_no_flags=False)
    assert rep["flagged"] <= w.B // 2


def test_non_current_stream_without_workspace():
    """``stream`` other than the current stream, no workspace and no outputs passed:
    the binding makes its allocations and fills on that stream."""
    import oracle
    import rejection_sampling_verification_spec_amd as sv
    w = W.make_config(2)
    dev = torch.device("cuda:0")
    t = w.to_torch(dev)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    assert torch.cuda.current_stream() != s
    count, out = sv.spec_verify(t["target"], t["draft"], t["draft_tokens"], t["u_accept"], t["u_sample"],
                                float(w.scalar_temperature), stream=s)
    tok = sv.spec_sample(t["target"][:, 0].contiguous(), t["u_sample"], 0.7, stream=s,
                         top_p=torch.full((w.B,), 0.9, dtype=torch.float32, device=dev))
    s.synchronize()
    o = oracle.run_workload(w)
    ok = o.flags == 0
    np.testing.assert_array_equal(count.cpu().numpy()[ok], o.accepted_count[ok])
    np.testing.assert_array_equal(out.cpu().numpy()[ok], o.out_tokens[ok])
    ref, tr = oracle.sample(w.target[:, 0], w.u_sample, 0.7, dtype=w.dtype, top_p=0.9)
    okr = tr.flags == 0
    np.testing.assert_array_equal(tok.cpu().numpy()[okr], ref[okr])


@pytest.mark.parametrize("cfg,greedy", [(2, False), (3, True), (0, False)])
def test_uniform_entry_with_diagnostics(cfg, greedy):
    """spec_verify_dbg (spec_verify's kernels, with diagnostics and the row-statistics events) gives
    the outputs and diagnostics of spec_verify_ex on the same uniform batch."""
    import rejection_sampling_verification_spec_amd as sv
    w = W.make_config(cfg, greedy=greedy)
    dev = torch.device("cuda:0")
    t = w.to_torch(dev)
    B, gamma = w.B, w.gamma
    rows = 2 * gamma + 1

    def dbg():
        f64 = dict(dtype=torch.float64, device=dev)
        return dict(p_draft=torch.full((B, gamma), float("nan"), **f64),
                    q_draft=torch.full((B, gamma), float("nan"), **f64),
                    accept_prob=torch.full((B, gamma), float("nan"), **f64),
                    row_max=torch.full((B, rows), float("nan"), dtype=torch.float32, device=dev),
                    row_sum=torch.full((B, rows), float("nan"), **f64),
                    row_argmax=torch.full((B, gamma + 1), -1, dtype=torch.int32, device=dev),
                    residual_mass=torch.full((B,), float("nan"), **f64))
    d1, d2 = dbg(), dbg()
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for e in ev:
        e.record()   # torch's own bookkeeping: elapsed_time needs events it has recorded once
    T = float(w.scalar_temperature)
    say(f"{w.name} via spec_verify_dbg")
    c1, o1 = sv.spec_verify(t["target"], None if greedy else t["draft"], t["draft_tokens"],
                            None if greedy else t["u_accept"], t["u_sample"], T, debug=d1, k1_events=ev)
    c2, o2 = sv.spec_verify_ex(t["target"], t["draft"], t["draft_tokens"], t["u_accept"], t["u_sample"],
                               t["temperature"], debug=d2)
    torch.cuda.synchronize()
    assert ev[0].elapsed_time(ev[1]) > 0.0
    assert torch.equal(c1, c2) and torch.equal(o1, o2)
    for k in d1:
        np.testing.assert_array_equal(d1[k].cpu().numpy(), d2[k].cpu().numpy(), err_msg=k)
