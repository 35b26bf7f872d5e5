"""The parity helpers' failure path (CPU only): a mismatch planted in a copy of the
oracle's own result makes check_parity fail, write the case to an .npz file, and
the replay helper finds the planted request again."""
import numpy as np
import pytest

from rejection_sampling_verification_spec_amd import workloads as W

from . import _parity


def test_failing_case_is_dumped_and_replayed(tmp_path, monkeypatch, oracle_mod):
    monkeypatch.setenv("SPECVERIFY_DUMP_DIR", str(tmp_path))
    w = W.make_random(17, 5, 3, 300, "bf16", temps=np.array([1, 0, 0.7, 1, 1], np.float32),
                      lens=np.array([3, 2, 0, 1, 3], np.int32), zipf=True)
    w.scalar_temperature = None
    o = oracle_mod.run_workload(w)
    g = _parity.GpuResult(o.accepted_count.copy(), o.out_tokens.copy())
    _parity.check_parity(w, g, o, require_no_flags=False)          # identical results pass
    g.out[3, 0] = (g.out[3, 0] + 1) % w.V                          # plant one wrong token (stochastic request)
    assert o.flags[3] == 0
    with pytest.raises(AssertionError, match="case written to"):
        _parity.check_parity(w, g, o, require_no_flags=False)
    path = tmp_path / f"{w.name}.npz"
    assert path.exists()
    z = np.load(path, allow_pickle=False)
    np.testing.assert_array_equal(z["target"], w.target)
    np.testing.assert_array_equal(z["lens"], w.lens)
    assert _parity.replay(str(path)) == 1
