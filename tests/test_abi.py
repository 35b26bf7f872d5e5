"""The C-ABI library loads and exports every entry point include/specverify.h declares.

No compute call is made here: argument checks run on the host before anything
is enqueued.  The argument-check cases pass small integers as device pointers,
so they run only where no GPU is visible: were a host check ever to regress,
nothing could be enqueued on such an address.
"""
import ctypes
import os
import re

import pytest

import rejection_sampling_verification_spec_amd as sv
from rejection_sampling_verification_spec_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0     # counts devices without initialising HIP
    except Exception:
        return os.path.exists("/dev/kfd")


fake_pointers = pytest.mark.skipif(_gpu_visible(), reason="passes fake device pointers; CPU-only check")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from rejection_sampling_verification_spec_amd import build_lib
        build_lib.build()
    return binding.load_library()


def test_header_declares_the_binding_surface():
    assert declared_functions() == sorted(binding.EXPORTED_SYMBOLS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_constants_match_header():
    text = open(HEADER).read()
    assert re.search(r"SV_F32\s*=\s*0", text) and re.search(r"SV_BF16\s*=\s*1", text)
    assert int(re.search(r"#define SV_GAMMA_MAX (\d+)", text).group(1)) == binding.SV_GAMMA_MAX
    assert re.search(r"#define SV_FILTER_MAX_V \(1 << (\d+)\)", text).group(1) == "20"
    assert binding.SV_FILTER_MAX_V == 1 << 20
    assert int(re.search(r"#define SV_TREE_MAX_NODES (\d+)", text).group(1)) == binding.SV_TREE_MAX_NODES
    assert re.search(r"#define SV_TREE_MAX_V \(1 << (\d+)\)", text).group(1) == "20"
    for name in ("SV_OK", "SV_EINVAL", "SV_EWORKSPACE", "SV_EHIP"):
        assert int(re.search(name + r"\s*=\s*(-?\d+)", text).group(1)) == getattr(binding, name)


def test_workspace_bytes(lib):
    assert sv.spec_verify_workspace_bytes(64, 5, 128256, sv.SV_BF16) > 0
    assert sv.spec_verify_workspace_bytes(64, 5, 128256, sv.SV_BF16) % 256 == 0
    assert sv.spec_verify_workspace_bytes(0, 5, 100, sv.SV_F32) == 0
    assert sv.spec_verify_workspace_bytes(1, -1, 100, sv.SV_F32) == 0
    assert sv.spec_verify_workspace_bytes(1, 33, 100, sv.SV_F32) == 0
    assert sv.spec_verify_workspace_bytes(1, 32, 100, sv.SV_F32) > 0
    assert sv.spec_verify_workspace_bytes(1, 3, 0, sv.SV_F32) == 0
    assert sv.spec_verify_workspace_bytes(1, 3, 10, 7) == 0


def test_strerror(lib):
    for code in (0, -1, -2, -3, 99):
        assert isinstance(sv.spec_verify_strerror(code), str) and sv.spec_verify_strerror(code)


def _call(lib, **kw):
    a = dict(t=1, d=1, tok=1, ua=1, us=1, T=1.0, B=2, g=3, V=10, dt=sv.SV_F32, cnt=1, out=1,
             ws=256, wsb=1 << 20)
    a.update(kw)
    return lib.spec_verify(a["t"], a["d"], a["tok"], a["ua"], a["us"], a["T"], a["B"], a["g"], a["V"],
                           a["dt"], a["cnt"], a["out"], a["ws"], a["wsb"], None)


@fake_pointers
def test_host_argument_checks(lib):
    # every case fails on the host before anything is enqueued
    assert _call(lib, B=0) == sv.binding.SV_EINVAL
    assert _call(lib, g=-1) == sv.binding.SV_EINVAL
    assert _call(lib, g=33) == sv.binding.SV_EINVAL
    assert _call(lib, V=0) == sv.binding.SV_EINVAL
    assert _call(lib, dt=5) == sv.binding.SV_EINVAL
    assert _call(lib, T=-1.0) == sv.binding.SV_EINVAL
    assert _call(lib, T=float("nan")) == sv.binding.SV_EINVAL
    assert _call(lib, T=float("inf")) == sv.binding.SV_EINVAL
    assert _call(lib, t=None) == sv.binding.SV_EINVAL
    assert _call(lib, us=None) == sv.binding.SV_EINVAL
    assert _call(lib, cnt=None) == sv.binding.SV_EINVAL
    assert _call(lib, tok=None) == sv.binding.SV_EINVAL
    assert _call(lib, d=None) == sv.binding.SV_EINVAL          # stochastic needs draft logits
    assert _call(lib, ua=None) == sv.binding.SV_EINVAL
    assert _call(lib, ws=None) == sv.binding.SV_EWORKSPACE
    assert _call(lib, ws=128) == sv.binding.SV_EWORKSPACE      # not 256-byte aligned
    assert _call(lib, wsb=16) == sv.binding.SV_EWORKSPACE      # too small
    ex = lib.spec_verify_ex(1, 1, 1, 1, 1, None, None, 2, 3, 10, sv.SV_F32, 1, 1, 256, 1 << 20, None, None)
    assert ex == sv.binding.SV_EINVAL                           # device temperature array is required


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(binding.LibraryMissing):
        binding.load_library(str(tmp_path / "nope.so"))


@fake_pointers
def test_sample_host_argument_checks(lib):
    f = lib.spec_sample
    ok = dict(l=1, u=1, T=1.0, Ts=None, R=4, V=10, dt=sv.SV_F32, tok=1, ws=256, wsb=1 << 20)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["l"], a["u"], a["T"], a["Ts"], a["R"], a["V"], a["dt"], a["tok"], a["ws"], a["wsb"], None)

    assert call(R=0) == sv.binding.SV_EINVAL
    assert call(V=0) == sv.binding.SV_EINVAL
    assert call(T=-0.5) == sv.binding.SV_EINVAL
    assert call(T=float("nan")) == sv.binding.SV_EINVAL
    assert call(l=None) == sv.binding.SV_EINVAL
    assert call(tok=None) == sv.binding.SV_EINVAL
    assert call(ws=None) == sv.binding.SV_EWORKSPACE
    assert call(wsb=8) == sv.binding.SV_EWORKSPACE
    assert sv.spec_sample_workspace_bytes(4, 10, sv.SV_F32) > sv.spec_verify_workspace_bytes(4, 0, 10, sv.SV_F32)


@fake_pointers
def test_filtered_host_argument_checks(lib):
    f = lib.spec_verify_filtered

    def call(V=10, T=1, k=1, p=None, B=2):
        return f(1, 1, 1, 1, 1, T, None, k, p, B, 3, V, sv.SV_F32, 1, 1, 256, 1 << 30, None, None)

    assert call(T=None) == sv.binding.SV_EINVAL                 # device temperature array is required
    assert call(V=(1 << 20) + 1) == sv.binding.SV_EINVAL        # beyond the fixed-point range
    assert call(V=(1 << 20) + 1, k=None, p=1) == sv.binding.SV_EINVAL
    assert call(B=0) == sv.binding.SV_EINVAL
    ws = f(1, 1, 1, 1, 1, 1, None, 1, None, 2, 3, 10, sv.SV_F32, 1, 1, 256, 16, None, None)
    assert ws == sv.binding.SV_EWORKSPACE
    # a workspace sized for the unfiltered call is too small for a filtered one
    plain = sv.spec_verify_workspace_bytes(2, 3, 10, sv.SV_F32)
    assert sv.spec_verify_filtered_workspace_bytes(2, 3, 10, sv.SV_F32) > plain
    assert f(1, 1, 1, 1, 1, 1, None, 1, None, 2, 3, 10, sv.SV_F32, 1, 1, 256, plain, None, None) == \
        sv.binding.SV_EWORKSPACE
    assert sv.spec_verify_filtered_workspace_bytes(2, 3, (1 << 20) + 1, sv.SV_F32) == 0


@fake_pointers
def test_tree_host_argument_checks(lib):
    f = lib.spec_verify_tree

    def call(B=2, N=3, V=10, dt=sv.SV_F32, wsb=1 << 20, **kw):
        a = dict(t=1, d=1, par=1, tok=1, nn=None, ua=1, us=1, T=1, cnt=1, out=1, nodes=1, ws=256)
        a.update(kw)
        return f(a["t"], a["d"], a["par"], a["tok"], a["nn"], a["ua"], a["us"], a["T"], B, N, V, dt, a["cnt"],
                 a["out"], a["nodes"], a["ws"], wsb, None)

    E = sv.binding.SV_EINVAL
    assert call(B=0) == E
    assert call(N=-1) == E
    assert call(N=sv.binding.SV_TREE_MAX_NODES + 1) == E
    assert call(V=sv.binding.SV_TREE_MAX_V + 1) == E
    assert call(dt=3) == E
    for name in ("t", "us", "T", "cnt", "out", "d", "par", "tok", "ua", "nodes"):
        assert call(**{name: None}) == E, name
    assert call(ws=None) == sv.binding.SV_EWORKSPACE
    assert call(ws=100) == sv.binding.SV_EWORKSPACE
    assert call(wsb=8) == sv.binding.SV_EWORKSPACE
    assert sv.spec_verify_tree_workspace_bytes(8, 84, 128256, sv.SV_BF16) > 0
    assert sv.spec_verify_tree_workspace_bytes(8, sv.binding.SV_TREE_MAX_NODES + 1, 100, sv.SV_BF16) == 0


@fake_pointers
def test_sample_filtered_host_argument_checks(lib):
    f = lib.spec_sample_filtered
    E = sv.binding.SV_EINVAL
    assert f(1, 1, None, 1, None, 4, 10, sv.SV_F32, 1, 256, 1 << 20, None) == E      # temperatures required
    assert f(1, 1, 1, 1, None, 4, (1 << 20) + 1, sv.SV_F32, 1, 256, 1 << 30, None) == E
    assert f(None, 1, 1, 1, None, 4, 10, sv.SV_F32, 1, 256, 1 << 20, None) == E
    assert f(1, 1, 1, 1, None, 4, 10, sv.SV_F32, 1, 256, 16, None) == sv.binding.SV_EWORKSPACE
    assert sv.spec_sample_filtered_workspace_bytes(4, 10, sv.SV_F32) > sv.spec_sample_workspace_bytes(4, 10, sv.SV_F32)
