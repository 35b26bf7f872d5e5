"""spec_verify_noalloc (the entry point for callers that cannot allocate) against
spec_verify, through the C ABI: identical counts and tokens on two calls in a
row on the built-in scratch array, the second with a smaller problem, so that
whatever the first call left in the array does not leak into the second."""
import numpy as np
import pytest

from rejection_sampling_verification_spec_amd import workloads as W

from ._parity import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rejection_sampling_verification_spec_amd as sv
    sv.load_library()


def _both(w):
    import rejection_sampling_verification_spec_amd as sv
    dev = torch.device("cuda:0")
    t = w.to_torch(dev)
    T = float(w.scalar_temperature)
    greedy = T == 0.0
    args = (t["target"], None if greedy else t["draft"], t["draft_tokens"] if w.gamma > 0 else None,
            None if greedy or w.gamma == 0 else t["u_accept"], t["u_sample"], T)
    ref_c, ref_o = sv.spec_verify(*args)
    cnt = torch.full((w.B,), -9, dtype=torch.int32, device=dev)
    out = torch.full((w.B, w.gamma + 1), -9, dtype=torch.int32, device=dev)
    sv.spec_verify_noalloc(*args, accepted_count=cnt, out_tokens=out)
    torch.cuda.synchronize()
    return ref_c.cpu().numpy(), ref_o.cpu().numpy(), cnt.cpu().numpy(), out.cpu().numpy()


@pytest.mark.parametrize("first,second", [
    ((3, False), (0, False)),                                     # B=64 V=128256 bf16, then B=1 V=1000 fp32
    ((2, False), (1, False)),
    ((3, True), ("small_greedy", None)),
])
def test_noalloc_matches_spec_verify_twice(first, second):
    for spec in (first, second):
        if spec[0] == "small_greedy":
            w = W.make_random(11, 3, 2, 777, "bf16", temps=0.0, zipf=True)
        else:
            w = W.make_config(spec[0], greedy=spec[1])
        say(f"noalloc {w.name} B={w.B} gamma={w.gamma} V={w.V}")
        rc, ro, nc, no = _both(w)
        np.testing.assert_array_equal(nc, rc)
        np.testing.assert_array_equal(no, ro)


def test_noalloc_rejects_problems_beyond_the_scratch():
    import rejection_sampling_verification_spec_amd as sv
    from rejection_sampling_verification_spec_amd import binding
    dev = torch.device("cuda:0")
    B, gamma, V = 4096, 8, 70000            # needs far more than the built-in array
    assert sv.spec_verify_workspace_bytes(B, gamma, V, sv.SV_BF16) > binding.SV_NOALLOC_SCRATCH_BYTES
    lib = binding.load_library()
    cnt = torch.empty(B, dtype=torch.int32, device=dev)
    out = torch.empty((B, gamma + 1), dtype=torch.int32, device=dev)
    # the size check fails on the host before any pointer is used
    rc = lib.spec_verify_noalloc(None, None, None, None, None, 1.0, B, gamma, V, sv.SV_BF16, cnt.data_ptr(),
                                 out.data_ptr(), None)
    assert rc == binding.SV_ESCRATCH
    assert "scratch" in sv.spec_verify_strerror(rc)
