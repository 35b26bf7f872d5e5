"""GPU parity of top-k / top-p filtered verification (spec_verify_filtered) against the oracle.

Bar: as for the unfiltered path (counts and tokens bit-exact on every request
the oracle does not flag, probabilities within 1e-5 / 2e-3, kept mass within
1e-6 relative), with one more flag: a top-p cut whose crossing lies within
1e-6 of the kept mass of a value group's boundary (bit 3).

Draft tokens are drawn from the filtered draft distribution (the sampler a
serving system runs before verification) with numpy, except where a test
wants drafts outside the kept set.
"""
import zlib

import numpy as np
import pytest

from rejection_sampling_verification_spec_amd import workloads as W

from ._parity import check_parity, gpu_run, run_and_check, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rejection_sampling_verification_spec_amd as sv
    sv.load_library()


def filtered_probs(z, T, k, p):
    """Filtered softmax of rows z [n, V] (numpy, sort-based; k <= 0 or >= V and p >= 1 mean off)."""
    z = np.asarray(z, np.float64)
    m = z.max(axis=1, keepdims=True)
    e = np.exp((z - m) / T)
    n, V = z.shape
    zs = -np.sort(-z, axis=1)
    tau = np.full(n, -np.inf)
    if 0 < k < V:
        tau = zs[:, k - 1]
    if p < 1.0:
        for r in range(n):
            keep = z[r] >= tau[r]
            Fk = e[r][keep].sum()
            vals, inv = np.unique(z[r][keep], return_inverse=True)
            mass = np.bincount(inv, weights=e[r][keep])[::-1]
            cum = np.cumsum(mass)
            j = int(np.argmax(cum >= p * Fk))
            tau[r] = max(tau[r], vals[::-1][j])
    out = np.where(z >= tau[:, None], e, 0.0)
    return out / out.sum(axis=1, keepdims=True)


def redraw_filtered_drafts(w, seed):
    """Replace the draft tokens by draws from the filtered draft rows (stochastic requests)."""
    rng = np.random.default_rng(seed)
    for b in range(w.B):
        T = float(w.temperature[b])
        g = int(w.draft_lens[b])
        if T == 0 or g == 0:
            continue
        k = int(w.top_k[b]) if w.top_k is not None else 0
        p = float(w.top_p[b]) if w.top_p is not None else 1.0
        q = filtered_probs(W._as_f64(w.draft[b, :g], w.dtype), T, k, p)
        u = rng.random(g)
        for i in range(g):
            c = np.cumsum(q[i])
            w.draft_tokens[b, i] = min(int(np.searchsorted(c, u[i] * c[-1], side="right")), w.V - 1)
    return w


def with_filter(w, top_k=None, top_p=None):
    if top_k is not None:
        w.top_k = np.ascontiguousarray(np.broadcast_to(np.asarray(top_k, np.int32), (w.B,)))
    if top_p is not None:
        w.top_p = np.ascontiguousarray(np.broadcast_to(np.asarray(top_p, np.float32), (w.B,)))
    w.name += f"_k{'' if top_k is None else 'x'}_p{'' if top_p is None else 'x'}"
    return w


# ------------------------------------------------------------------ small shapes
CASES = [
    # (B, gamma, V, dtype, T, top_k, top_p)
    (16, 4, 1000, "f32", 1.0, 20, None),
    (16, 4, 1000, "f32", 0.7, None, 0.9),
    (16, 4, 1000, "bf16", 0.7, 50, 0.9),
    (8, 3, 5000, "f32", 1.3, 1, None),
    (8, 3, 5000, "bf16", 0.5, None, 0.5),
    (8, 5, 32000, "f32", 0.7, 40, 0.95),
    (4, 2, 32003, "bf16", 1.0, 4000, 0.8),     # ragged tail, unaligned rows, k beyond one bin
    (8, 2, 70001, "bf16", 1.0, None, 0.99),    # deep cut: thousands of tokens kept
    (8, 2, 70001, "f32", 1.0, None, 0.999),    # deep cut among fp32 values on a 1/16 grid
    (12, 0, 4096, "f32", 0.9, 10, 0.7),        # gamma = 0: filtered plain sampling
]
# requests the oracle may flag: a deep top-p cut among many distinct logits of
# small mass can lie within 1e-6 of a group boundary.  A cut among tens of
# thousands of distinct fp32 logits of mass ~1e-6 each always does, so the fp32
# deep-cut case puts its logits on a 1/16 grid (387 distinct values per row):
# value groups then hold many tokens and most cuts are decided.
MAX_FLAGGED = {(8, 2, 70001, "f32", 1.0, None, 0.999): 2, (8, 2, 70001, "bf16", 1.0, None, 0.99): 3}
GRID = {(8, 2, 70001, "f32", 1.0, None, 0.999): 16}


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}_g{c[1]}_V{c[2]}_{c[3]}_T{c[4]}_k{c[5]}_p{c[6]}"
                                             for c in CASES])
def test_filtered_parity_shapes(case):
    B, gamma, V, dtype, T, k, p = case
    seed = zlib.crc32(repr(case).encode()) & 0xffff
    w = with_filter(W.make_random(seed, B, gamma, V, dtype, temps=T, target_scale=3.0, sigma=0.6, zipf=True),
                    top_k=k, top_p=p)
    if case in GRID:
        q = np.float32(GRID[case])
        w.target = (np.round(w.target * q) / q).astype(np.float32)
        w.draft = (np.round(w.draft * q) / q).astype(np.float32)
    redraw_filtered_drafts(w, seed + 1)
    rep = run_and_check(w, debug=True, require_no_flags=False)
    assert rep["flagged"] <= MAX_FLAGGED.get(case, B // 8)


def test_filtered_per_request_parameters_mixed_batch():
    """Every request its own k, p (including off values), T (including greedy) and draft length."""
    rng = np.random.default_rng(77)
    B, gmax, V = 48, 5, 20000
    lens = rng.integers(0, gmax + 1, size=B).astype(np.int32)
    temps = rng.choice(np.array([0.0, 0.6, 1.0, 1.5], np.float32), size=B)
    w = W.make_random(78, B, gmax, V, "bf16", temps=temps, lens=lens, target_scale=3.5, zipf=True)
    w.top_k = rng.choice(np.array([0, 1, 5, 100, 3000, V, V + 9, -4], np.int32), size=B)
    w.top_p = rng.choice(np.array([1.0, 0.95, 0.9, 0.6, 0.2, 1.5, 0.0], np.float32), size=B)
    # the oracle rejects out-of-range filter values; the library treats them as "off"
    w_or = W.Workload(**{**w.__dict__})
    w_or.top_k = np.where((w.top_k > 0) & (w.top_k < V), w.top_k, 0).astype(np.int32)
    w_or.top_p = np.where((w.top_p > 0) & (w.top_p < 1), w.top_p, 1.0).astype(np.float32)
    redraw_filtered_drafts(w_or, 79)
    w.draft_tokens = w_or.draft_tokens
    import oracle
    say(f"mixed filtered batch B={B} V={V}")
    g = gpu_run(w, debug=True)
    rep = check_parity(w_or, g, oracle.run_workload(w_or), require_no_flags=False)
    say(f"ok {rep}")
    assert rep["flagged"] <= 4


def test_filtered_drafts_outside_the_kept_set():
    """Drafts drawn from the unfiltered q: some have q'(x) = 0 (accepted iff p'(x) > 0)."""
    w = with_filter(W.make_random(91, 24, 4, 3000, "f32", temps=1.0, target_scale=2.0, sigma=1.2),
                    top_k=8, top_p=0.6)
    import oracle
    o = oracle.run_workload(w)
    assert np.any(o.q_draft == 0.0)
    g = gpu_run(w, debug=True)
    rep = check_parity(w, g, o, require_no_flags=False)
    say(f"ok {rep}")


def test_crowded_bins_force_key_refinement():
    """Logits on a fine grid around one value put > 2048 tokens into one y bin, and
    repeated values put large tie groups on the cuts."""
    rng = np.random.default_rng(5)
    B, gamma, V = 6, 2, 60000
    base = rng.integers(0, 40, size=(B, gamma + 1, V)).astype(np.float32) * np.float32(1e-4)
    base[:, :, :50] += 3.0                                   # a handful of leaders
    draft = base[:, :gamma] + rng.integers(0, 3, size=(B, gamma, V)).astype(np.float32) * np.float32(1e-4)
    tokens = np.zeros((B, gamma), np.int32)
    w = W.from_logits(base, draft, tokens, rng.random((B, gamma)), rng.random(B), 1.0, dtype="f32",
                      name="crowded")
    w.scalar_temperature = None
    w.top_k = np.array([100, 5000, 0, 30000, 59999, 7], np.int32)
    w.top_p = np.array([1.0, 1.0, 0.5, 0.9, 0.99, 0.3], np.float32)
    redraw_filtered_drafts(w, 6)
    rep = run_and_check(w, debug=True, require_no_flags=False)
    assert rep["flagged"] <= 1


@pytest.mark.parametrize("V,dtype,ragged", [(50000, "bf16", False), (32003, "f32", False), (20001, "bf16", True)],
                         ids=["V50000_bf16", "V32003_f32_unaligned", "V20001_bf16_unaligned_ragged"])
def test_cut_below_the_capture_window(V, dtype, ragged):
    """One dominant logit per row puts every other logit more than 16 binary orders of
    magnitude below the maximum: the captured list holds one logit, so the k-th logit
    or the top-p crossing lies below it.  Rows resolve through a deeper window
    (the band counts and a second capture) or, when that floor would hold more than
    4096 logits, through the general path.  Odd V makes every row after the first
    start off a 16-byte boundary (the one-by-one paths); ragged draft lengths leave
    padding rows that must not be read."""
    rng = np.random.default_rng(8 + V)
    B, gamma = 8, 3
    z = (rng.standard_normal((B, gamma + 1, V)) * 2.0 - 10.0).astype(np.float32)
    for b in range(B):  # a tier of 60 logits 11.2 to 12.8 nats below the top, outside the window
        for i in range(gamma + 1):
            tier = rng.choice(V, 60, replace=False)
            z[b, i, tier] = (12.0 - rng.uniform(11.2, 12.8, 60)).astype(np.float32)
    z[:, :, 4321] = 12.0
    draft = z[:, :gamma] + (rng.standard_normal((B, gamma, V)) * 0.3).astype(np.float32)
    tokens = np.zeros((B, gamma), np.int32)
    lens = np.array([3, 1, 0, 2, 3, 3, 2, 1], np.int32) if ragged else None
    # the token at the end is drawn in the last 4e-4 of the CDF: one of the kept tier
    u_s = np.minimum(1.0 - rng.random(B) * 4e-4, 1.0 - 2.0 ** -24).astype(np.float32)
    w = W.from_logits(z, draft, tokens, rng.random((B, gamma)), u_s, 1.0, dtype=dtype,
                      name="dominant", lens=lens)
    w.scalar_temperature = None
    if ragged:  # padding rows poisoned
        nan = W.BF16_NAN if dtype == "bf16" else np.float32(np.nan)
        for b in range(B):
            w.target[b, lens[b] + 1:] = nan
            w.draft[b, lens[b]:] = nan
    #              deeper window by count ...... general  top-p below the window ...... both
    w.top_k = np.array([50, 200, 1000, 3000, 6000, 0, 0, 40], np.int32)
    w.top_p = np.array([1.0, 1.0, 1.0, 0.95, 1.0, 0.99999, 0.9999999, 0.99], np.float32)
    redraw_filtered_drafts(w, 9)
    rep = run_and_check(w, debug=True, require_no_flags=False)
    # the top-p rows' cuts and some tail draws sit within the rounding bands
    assert rep["flagged"] <= 4


def test_filters_off_equal_unfiltered_entry_point():
    w = W.make_random(33, 16, 3, 9000, "bf16", temps=0.8, zipf=True)
    base = gpu_run(w, debug=True, force_ex=True)
    w.top_k = np.array([0, 9000, 100000, -1] * 4, np.int32)
    w.top_p = np.array([1.0, 2.0, 0.0, float("nan")] * 4, np.float32)
    f = gpu_run(w, debug=True)
    np.testing.assert_array_equal(f.count, base.count)
    np.testing.assert_array_equal(f.out, base.out)
    for k in base.dbg:
        np.testing.assert_array_equal(f.dbg[k], base.dbg[k])


def test_top1_equals_greedy_verification():
    w = W.make_random(34, 32, 4, 12000, "f32", temps=0.9, target_scale=2.0)
    w.draft_tokens[:] = np.argmax(w.draft, axis=2)
    wg = W.Workload(**{**w.__dict__})
    wg.temperature = np.zeros(w.B, np.float32)
    wg.scalar_temperature = None
    greedy = gpu_run(wg, force_ex=True)
    w.top_k = np.ones(w.B, np.int32)
    f = gpu_run(w)
    np.testing.assert_array_equal(f.count, greedy.count)
    np.testing.assert_array_equal(f.out, greedy.out)


@pytest.mark.parametrize("top_k,top_p", [(None, 0.9), (50, 0.9)])
def test_filtered_serving_shape(top_k, top_p):
    """B = 64, gamma = 5, V = 128256 bf16 at T = 0.7 with top_p = 0.9 (the pages' vLLM example)."""
    w = with_filter(W.build("B64_g5_V128256_bf16_T0.7_zipf", 2000, 64, 5, 128256, "bf16", target_scale=4.0,
                            zipf=True, sigma=0.5, temps=0.7), top_k=top_k, top_p=top_p)
    redraw_filtered_drafts(w, 2001)
    rep = run_and_check(w, debug=True, require_no_flags=False)
    assert rep["flagged"] <= 2


def test_filtered_largest_vocabulary():
    """V = 2^20, the largest the filtered entry point accepts (fixed-point masses with
    41 fractional bits), top_k = 100 and top_p = 0.9."""
    w = with_filter(W.build("B2_g2_V1048576_bf16_T0.7_zipf", 2200, 2, 2, 1 << 20, "bf16", target_scale=4.0,
                            zipf=True, sigma=0.5, temps=0.7), top_k=100, top_p=0.9)
    redraw_filtered_drafts(w, 2201)
    rep = run_and_check(w, debug=True, require_no_flags=False)
    assert rep["flagged"] <= 1


@pytest.mark.parametrize("T", [1.2, 2.5])
def test_filtered_flat_rows(T):
    """Serving-size rows at a high temperature: at T = 1.2 the capture window holds up to
    about 25000 logits (the long list), at T = 2.5 nearly the whole row (the general path)."""
    w = with_filter(W.build(f"B4_g2_V128256_bf16_T{T}_zipf", 2100, 4, 2, 128256, "bf16", target_scale=4.0,
                            zipf=True, sigma=0.5, temps=T), top_p=0.9)
    redraw_filtered_drafts(w, 2101)
    rep = run_and_check(w, debug=True, require_no_flags=False)
    assert rep["flagged"] <= 1


def test_filtered_deterministic():
    w = with_filter(W.make_random(35, 16, 4, 30000, "bf16", temps=0.7, zipf=True), top_k=200, top_p=0.9)
    a = gpu_run(w, debug=True)
    b = gpu_run(w, debug=True)
    np.testing.assert_array_equal(a.count, b.count)
    np.testing.assert_array_equal(a.out, b.out)
    for k in a.dbg:
        np.testing.assert_array_equal(a.dbg[k], b.dbg[k])


def test_filtered_graph_replay_and_side_stream():
    """Filtered verification captured in a HIP graph equals the eager call on every replay, with the
    workspace scribbled between replays (the filter kernels clear what they need themselves)."""
    import rejection_sampling_verification_spec_amd as sv
    w = with_filter(W.make_random(36, 12, 4, 20000, "bf16", temps=0.7, zipf=True), top_k=40, top_p=0.9)
    redraw_filtered_drafts(w, 37)
    dev = torch.device("cuda:0")
    t = w.to_torch(dev)
    count = torch.empty(w.B, dtype=torch.int32, device=dev)
    out = torch.empty((w.B, w.gamma + 1), dtype=torch.int32, device=dev)
    ws = torch.empty(sv.spec_verify_filtered_workspace_bytes(w.B, w.gamma, w.V, sv.SV_BF16), dtype=torch.uint8,
                     device=dev)
    s = torch.cuda.Stream()

    def call():
        sv.spec_verify_filtered(t["target"], t["draft"], t["draft_tokens"], t["u_accept"], t["u_sample"],
                                t["temperature"], None, top_k=t["top_k"], top_p=t["top_p"], accepted_count=count,
                                out_tokens=out, workspace=ws, stream=s)

    with torch.cuda.stream(s):
        call()
    torch.cuda.synchronize()
    ref = (count.cpu().clone(), out.cpu().clone())
    g0 = gpu_run(w)
    np.testing.assert_array_equal(ref[0].numpy(), g0.count)
    np.testing.assert_array_equal(ref[1].numpy(), g0.out)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    for rep in range(3):
        count.fill_(-5)
        out.fill_(-5)
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"filtered graph replay {rep}")
        assert torch.equal(count.cpu(), ref[0]) and torch.equal(out.cpu(), ref[1])


def _fuzz_case(seed, V=None):
    """A small random filtered batch: shape, dtype, temperature, filter values and the
    logit law (Gaussian, integer ties, one dominant token, nearly flat) all drawn."""
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 9))
    gamma = int(rng.integers(0, 7))
    V = int(rng.choice([1, 2, 3, 17, 64, 257, 1000, 4099, 5000])) if V is None else V
    dtype = str(rng.choice(["f32", "bf16"]))
    law = str(rng.choice(["normal", "ties", "dominant", "flat"]))
    shape = (B, gamma + 1, V)
    if law == "normal":
        z = rng.standard_normal(shape) * rng.uniform(0.5, 4.0)
    elif law == "ties":
        z = rng.integers(0, 5, size=shape).astype(np.float64)
    elif law == "dominant":
        z = rng.standard_normal(shape) * 2.0
        z[..., int(rng.integers(0, V))] += rng.uniform(8.0, 30.0)
    else:
        z = rng.standard_normal(shape) * 0.1
    z = z.astype(np.float32)
    noise = rng.standard_normal((B, gamma, V)).astype(np.float32) * np.float32(rng.uniform(0.0, 1.0))
    draft = z[:, :gamma] + noise
    T = rng.choice(np.array([0.0, 0.3, 1.0, 2.0], np.float32), size=B)
    lens = rng.integers(0, gamma + 1, size=B).astype(np.int32) if gamma > 0 and rng.random() < 0.5 else None
    w = W.from_logits(z, draft, np.zeros((B, gamma), np.int32), rng.random((B, gamma)), rng.random(B), T,
                      dtype=dtype, lens=lens, name=f"fuzz{seed}_{law}")
    w.scalar_temperature = None
    w.top_k = rng.choice(np.array([0, 1, 2, 5, max(V - 1, 0), V, int(rng.integers(1, V + 1))], np.int32), size=B)
    w.top_p = rng.choice(np.array([1.0, 0.5, 0.9, 0.99, 0.999], np.float32), size=B)
    redraw_filtered_drafts(w, seed + 1)
    return w


@pytest.mark.parametrize("seed", range(40))
def test_filtered_fuzz(seed):
    w = _fuzz_case(1000 + seed)
    rep = run_and_check(w, debug=True, require_no_flags=False)
    assert rep["flagged"] <= w.B // 2
