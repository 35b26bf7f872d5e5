"""Adaptive draft length closed on the device: each step the policy picks gamma, a
ragged batch is verified by spec_verify_ex on the GPU, and the accepted counts it
returns are fed back to the policy.

The policies are those of the pages (the batch-size table and the moving
average of the accepted length: page "投機的デコーディングとは：同時リクエストが多い
と遅くなる理由", section vLLM は利用者が書く表で、SGLang は実行中に観測した受理の長さ
で先読み数を変える; the windowed acceptance rate: page "LLM推測デコーディング最適化
實踐", section 動的推測戦略).  In lockstep the same loop runs on the CPU with the
plain restatement of the policies (oracle/gamma_policy.py), fed the same counts,
and the CPU oracle of the verify step checks every step on the same inputs.
Required: identical gamma trajectories, counts and tokens bit-exact at every
step outside the near-boundary band (no step excusing more than half of its
requests), and a trajectory that moves.
"""
import numpy as np
import pytest

from oracle import gamma_policy as ref
from rejection_sampling_verification_spec_amd import workloads as W

from ._parity import GpuResult, check_parity, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

STEPS = 60


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rejection_sampling_verification_spec_amd as sv
    sv.load_library()


def _policies(kind):
    import rejection_sampling_verification_spec_amd as sv
    if kind == "by_batch":
        return sv.GammaPolicy(sv.SV_GAMMA_BY_BATCH), ref.ByBatch()
    if kind == "ema":
        return sv.GammaPolicy(sv.SV_GAMMA_EMA), ref.Ema()
    # a 10-step window (the pages use 100) so that 60 steps move the rate across both thresholds
    return sv.GammaPolicy(sv.SV_GAMMA_RATE_WINDOW, window=10), ref.RateWindow(window=10)


def _batch_size(kind, step, rng):
    if kind == "by_batch":      # across the table's ranges: 1-64 -> 3, 65-128 -> 1, 129-512 -> 0
        return int(rng.choice([4, 30, 64, 65, 90, 128, 129, 140]))
    if kind == "ema":           # the moving-average buckets (1, 2, 3-4, 5-8, 9-16, 17-31) and the fixed >= 32
        return int(rng.choice([1, 2, 3, 6, 12, 20, 31, 33]))
    return 12


def _sigma(kind, step):
    """Draft noise per step: phases of close drafts (high acceptance) and far drafts (low)."""
    if kind == "rate_window":
        return 0.0 if (step // 15) % 2 == 0 else 2.5
    return 0.3 + 1.2 * ((step // 7) % 3) / 2


def _lens(kind, g, B, rng):
    """Ragged draft lengths at stride g: some requests hold fewer drafts than the policy allows."""
    if g == 0:
        return None
    if kind == "rate_window":   # mostly full, so that an all-accepting phase reads as a high rate
        return np.where(rng.random(B) < 0.1, g - 1, g).astype(np.int32)
    return rng.integers(max(0, g - 1), g + 1, size=B).astype(np.int32)


@pytest.mark.parametrize("kind", ["by_batch", "ema", "rate_window"])
def test_policy_loop_through_the_library(kind):
    import oracle
    import rejection_sampling_verification_spec_amd as sv
    dev = torch.device("cuda:0")
    rng = np.random.default_rng({"by_batch": 1, "ema": 2, "rate_window": 3}[kind])
    pol, ora = _policies(kind)
    gammas = []
    flagged = 0
    for step in range(STEPS):
        B = _batch_size(kind, step, rng)
        g = pol.next(B)
        assert g == ora.next(B), f"{kind} step {step}: library gamma {g}, restatement {ora.next(B)}"
        gammas.append(g)
        # a ragged batch at stride g: requests may hold fewer drafts than the policy allows
        lens = _lens(kind, g, B, rng)
        temps = rng.choice(np.array([0.0, 0.7, 1.0], np.float32), size=B)
        w = W.build(f"{kind}_s{step}", 7000 + 97 * step + {"by_batch": 0, "ema": 1, "rate_window": 2}[kind],
                    B, g, 3001, "bf16", target_scale=3.0, zipf=True, sigma=_sigma(kind, step), temps=temps,
                    lens=lens)
        t = w.to_torch(dev)
        count, out = sv.spec_verify_ex(t["target"], t["draft"] if g > 0 else None,
                                       t["draft_tokens"] if g > 0 else None, t["u_accept"] if g > 0 else None,
                                       t["u_sample"], t["temperature"], t["lens"])
        torch.cuda.synchronize()
        gc, go = count.cpu().numpy(), out.cpu().numpy()
        o = oracle.run_workload(w)
        check_parity(w, GpuResult(gc, go), o, require_no_flags=False)   # bit-exact outside the band
        flagged += int((o.flags != 0).sum())
        pol.observe(count, g)          # the device tensor, as a serving loop would hand it over
        ora.observe(gc, g)             # the same counts into the restatement
    say(f"{kind}: gamma trajectory {gammas}; near-boundary requests {flagged}")
    assert len(set(gammas)) > 1, f"{kind}: the trajectory never moved"
    if kind == "ema":
        for k, v in ora.avg.items():
            assert abs(pol.state.ema[k] - v) < 1e-12
    if kind == "rate_window":
        assert max(gammas) > 5 and min(gammas) < 5, gammas
