"""Thin ctypes binding of libspecverify (include/specverify.h).

Argument marshalling only: shapes and dtypes are read off torch tensors, their
device pointers and the HIP stream (the ``stream`` argument, else torch's
current stream) are handed to the C ABI, and
every step of the verify path runs in the library's HIP kernels.  There is no
fallback: if the compiled library is missing the calls raise ``LibraryMissing``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspecverify.so")

SV_F32 = 0
SV_BF16 = 1
SV_GAMMA_MAX = 32
SV_FILTER_MAX_V = 1 << 20
SV_TREE_MAX_NODES = 256
SV_TREE_MAX_V = 1 << 20

SV_OK = 0
SV_EINVAL = -1
SV_EWORKSPACE = -2
SV_EHIP = -3
SV_ESCRATCH = -4
SV_NOALLOC_SCRATCH_BYTES = 4 << 20

EXPORTED_SYMBOLS = (
    "spec_verify_workspace_bytes",
    "spec_verify",
    "spec_verify_dbg",
    "spec_verify_ex",
    "spec_verify_filtered",
    "spec_verify_filtered_workspace_bytes",
    "spec_verify_tree",
    "spec_verify_tree_workspace_bytes",
    "spec_sample_filtered",
    "spec_sample_filtered_workspace_bytes",
    "spec_sample_workspace_bytes",
    "spec_sample",
    "spec_gamma_policy_init",
    "spec_gamma_next",
    "spec_gamma_observe",
    "spec_verify_strerror",
    "spec_verify_noalloc",
)

SV_GAMMA_BY_BATCH = 0
SV_GAMMA_EMA = 1
SV_GAMMA_RATE_WINDOW = 2
SV_GAMMA_POLICY_SLOTS = 16
SV_GAMMA_WINDOW_MAX = 256


class LibraryMissing(RuntimeError):
    """The compiled HIP library is not there (run ``__graft_entry__.build()``)."""


class SpecVerifyError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where} failed: {spec_verify_strerror(code)} (code {code})")


class SvDebug(ctypes.Structure):
    _fields_ = [
        ("p_draft", ctypes.c_void_p),
        ("q_draft", ctypes.c_void_p),
        ("accept_prob", ctypes.c_void_p),
        ("row_max", ctypes.c_void_p),
        ("row_sum", ctypes.c_void_p),
        ("row_argmax", ctypes.c_void_p),
        ("residual_mass", ctypes.c_void_p),
        ("k1_events", ctypes.c_void_p * 2),
    ]


class SvGammaPolicy(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int),
        ("n_ranges", ctypes.c_int),
        ("range_max_batch", ctypes.c_int * SV_GAMMA_POLICY_SLOTS),
        ("range_gamma", ctypes.c_int * SV_GAMMA_POLICY_SLOTS),
        ("n_buckets", ctypes.c_int),
        ("bucket_max_batch", ctypes.c_int * SV_GAMMA_POLICY_SLOTS),
        ("ema", ctypes.c_double * SV_GAMMA_POLICY_SLOTS),
        ("ema_count", ctypes.c_int * SV_GAMMA_POLICY_SLOTS),
        ("ema_weight", ctypes.c_double),
        ("steps_min", ctypes.c_int), ("steps_max", ctypes.c_int),
        ("fixed_from_batch", ctypes.c_int), ("fixed_steps", ctypes.c_int),
        ("window", ctypes.c_int), ("hist_len", ctypes.c_int), ("hist_pos", ctypes.c_int),
        ("history", ctypes.c_double * SV_GAMMA_WINDOW_MAX),
        ("raise_above", ctypes.c_double), ("lower_below", ctypes.c_double),
        ("gamma_min", ctypes.c_int), ("gamma_max", ctypes.c_int), ("gamma_current", ctypes.c_int),
    ]


_lib: Optional[ctypes.CDLL] = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libspecverify.so; raises ``LibraryMissing`` if it has not been built.

    ``path`` (or the SPECVERIFY_LIB environment variable) selects another build
    of the same library."""
    global _lib
    if _lib is not None:
        return _lib
    if path is None:
        path = os.environ.get("SPECVERIFY_LIB", LIB_PATH)
    if not os.path.exists(path):
        raise LibraryMissing(f"{path} not found: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.spec_verify_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.spec_verify_workspace_bytes.restype = sz
    lib.spec_verify.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, i32, i32, i32, i32,
                                vp, vp, vp, sz, vp]
    lib.spec_verify.restype = i32
    lib.spec_verify_dbg.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, i32, i32, i32, i32,
                                    vp, vp, vp, sz, vp, ctypes.POINTER(SvDebug)]
    lib.spec_verify_dbg.restype = i32
    lib.spec_verify_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                   vp, vp, vp, sz, vp, ctypes.POINTER(SvDebug)]
    lib.spec_verify_ex.restype = i32
    lib.spec_verify_filtered.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                         vp, vp, vp, sz, vp, ctypes.POINTER(SvDebug)]
    lib.spec_verify_filtered.restype = i32
    lib.spec_verify_filtered_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.spec_verify_filtered_workspace_bytes.restype = sz
    lib.spec_verify_tree.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.spec_verify_tree.restype = i32
    lib.spec_verify_tree_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.spec_verify_tree_workspace_bytes.restype = sz
    lib.spec_sample_filtered.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, sz, vp]
    lib.spec_sample_filtered.restype = i32
    lib.spec_sample_filtered_workspace_bytes.argtypes = [i32, i32, i32]
    lib.spec_sample_filtered_workspace_bytes.restype = sz
    lib.spec_sample_workspace_bytes.argtypes = [i32, i32, i32]
    lib.spec_sample_workspace_bytes.restype = sz
    lib.spec_sample.argtypes = [vp, vp, ctypes.c_float, vp, i32, i32, i32, vp, vp, sz, vp]
    lib.spec_sample.restype = i32
    lib.spec_gamma_policy_init.argtypes = [ctypes.POINTER(SvGammaPolicy), i32]
    lib.spec_gamma_policy_init.restype = i32
    lib.spec_gamma_next.argtypes = [ctypes.POINTER(SvGammaPolicy), i32]
    lib.spec_gamma_next.restype = i32
    lib.spec_gamma_observe.argtypes = [ctypes.POINTER(SvGammaPolicy), vp, i32, i32]
    lib.spec_gamma_observe.restype = i32
    lib.spec_verify_noalloc.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, i32, i32, i32, i32, vp, vp, vp]
    lib.spec_verify_noalloc.restype = i32
    lib.spec_verify_strerror.argtypes = [i32]
    lib.spec_verify_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def spec_verify_strerror(code: int) -> str:
    return load_library().spec_verify_strerror(int(code)).decode()


def spec_verify_workspace_bytes(B: int, gamma: int, V: int, dtype: int) -> int:
    return int(load_library().spec_verify_workspace_bytes(B, gamma, V, dtype))


def spec_verify_filtered_workspace_bytes(B: int, gamma: int, V: int, dtype: int) -> int:
    return int(load_library().spec_verify_filtered_workspace_bytes(B, gamma, V, dtype))


# --------------------------------------------------------------------------- torch marshalling
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return SV_BF16
    if t.dtype == torch.float32:
        return SV_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libspecverify must be contiguous")
    return t.data_ptr()


def _check_device(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libspecverify takes device tensors")


def _shapes(target_logits):
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, gamma+1, V]")
    B, g1, V = target_logits.shape
    return int(B), int(g1) - 1, int(V)


def _expect(t, shape, dtype, name, optional=False):
    """Host-side shape / dtype check before anything reaches the kernels."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_all(target_logits, draft_logits, draft_tokens, u_accept, u_sample, accepted_count,
               out_tokens, greedy_only: bool):
    import torch
    B, gamma, V = _shapes(target_logits)
    need_draft = gamma > 0 and not greedy_only
    _expect(draft_logits, (B, gamma, V), target_logits.dtype, "draft_logits", optional=not need_draft)
    _expect(draft_tokens, (B, gamma), torch.int32, "draft_tokens", optional=gamma == 0)
    _expect(u_accept, (B, gamma), torch.float32, "u_accept", optional=not need_draft)
    _expect(u_sample, (B,), torch.float32, "u_sample")
    _expect(accepted_count, (B,), torch.int32, "accepted_count")
    _expect(out_tokens, (B, gamma + 1), torch.int32, "out_tokens")


def _outputs(B, gamma, device, accepted_count, out_tokens):
    import torch
    if accepted_count is None:
        accepted_count = torch.empty(B, dtype=torch.int32, device=device)
    if out_tokens is None:
        out_tokens = torch.empty((B, gamma + 1), dtype=torch.int32, device=device)
    return accepted_count, out_tokens


def new_workspace(nbytes: int, device):
    """Device workspace of ``nbytes`` bytes (its contents on entry do not matter)."""
    import torch
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _workspace(B, gamma, V, dt, device, workspace, filtered=False):
    need = (spec_verify_filtered_workspace_bytes if filtered else spec_verify_workspace_bytes)(B, gamma, V, dt)
    if workspace is None:
        workspace = new_workspace(need, device)
    return workspace, need


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on(stream):
    """Context for the binding's own allocations and fills: with a ``stream``,
    they are made on that stream (torch's allocator then ties the blocks to it,
    and a fill is ordered before the kernels that read it); otherwise on the
    current stream, which is where the kernels run."""
    import contextlib

    import torch
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def spec_verify(target_logits, draft_logits, draft_tokens, u_accept, u_sample, temperature: float,
                accepted_count=None, out_tokens=None, workspace=None, stream=None, debug: Optional[dict] = None,
                k1_events=None):
    """Uniform batch (one temperature, gamma drafts per request).  Returns (accepted_count, out_tokens).

    ``debug`` / ``k1_events``: as for ``spec_verify_ex`` (the call then goes through spec_verify_dbg,
    which runs the same kernels as spec_verify)."""
    lib = load_library()
    B, gamma, V = _shapes(target_logits)
    dt = _dtype_code(target_logits)
    _check_device(target_logits, draft_logits, draft_tokens, u_accept, u_sample)
    with _on(stream):
        accepted_count, out_tokens = _outputs(B, gamma, target_logits.device, accepted_count, out_tokens)
        _check_all(target_logits, draft_logits, draft_tokens, u_accept, u_sample, accepted_count, out_tokens,
                   greedy_only=float(temperature) == 0.0)
        workspace, need = _workspace(B, gamma, V, dt, target_logits.device, workspace)
    args = (_ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), _ptr(u_accept), _ptr(u_sample),
            float(temperature), B, gamma, V, dt, _ptr(accepted_count), _ptr(out_tokens), _ptr(workspace),
            workspace.numel(), _stream(stream))
    if debug or k1_events:
        rc = lib.spec_verify_dbg(*args, _debug_struct(B, gamma, debug, k1_events))
    else:
        rc = lib.spec_verify(*args)
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify")
    return accepted_count, out_tokens


def spec_verify_noalloc(target_logits, draft_logits, draft_tokens, u_accept, u_sample, temperature: float,
                        accepted_count, out_tokens, stream=None):
    """``spec_verify`` on the library's built-in scratch array: no workspace, and
    nothing is allocated (the caller passes the outputs).  Calls that overlap on
    one GPU race; a problem whose workspace would exceed SV_NOALLOC_SCRATCH_BYTES
    raises SpecVerifyError(SV_ESCRATCH)."""
    lib = load_library()
    B, gamma, V = _shapes(target_logits)
    dt = _dtype_code(target_logits)
    _check_device(target_logits, draft_logits, draft_tokens, u_accept, u_sample, accepted_count, out_tokens)
    _check_all(target_logits, draft_logits, draft_tokens, u_accept, u_sample, accepted_count, out_tokens,
               greedy_only=float(temperature) == 0.0)
    rc = lib.spec_verify_noalloc(_ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), _ptr(u_accept),
                                 _ptr(u_sample), float(temperature), B, gamma, V, dt, _ptr(accepted_count),
                                 _ptr(out_tokens), _stream(stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_noalloc")
    return accepted_count, out_tokens


def spec_verify_ex(target_logits, draft_logits, draft_tokens, u_accept, u_sample, temperature,
                   draft_lens=None, accepted_count=None, out_tokens=None, workspace=None,
                   stream=None, debug: Optional[dict] = None, k1_events=None):
    """Ragged / mixed batch: ``temperature`` and ``draft_lens`` are device tensors [B].

    ``debug``: optional dict of preallocated device tensors keyed like ``sv_debug``.
    ``k1_events``: optional pair of recorded ``torch.cuda.Event(enable_timing=True)``
    that the library records around its row-statistics kernel.
    """
    return _verify_device_params("spec_verify_ex", target_logits, draft_logits, draft_tokens, u_accept,
                                 u_sample, temperature, draft_lens, None, None, accepted_count, out_tokens,
                                 workspace, stream, debug, k1_events)


def spec_verify_filtered(target_logits, draft_logits, draft_tokens, u_accept, u_sample, temperature,
                         draft_lens=None, top_k=None, top_p=None, accepted_count=None, out_tokens=None,
                         workspace=None, stream=None, debug: Optional[dict] = None, k1_events=None):
    """``spec_verify_ex`` with per-request top-k / top-p filtering.

    ``top_k``: device int32 [B] or None (k in [1, V-1] filters, other values leave it off);
    ``top_p``: device float32 [B] or None (p in (0, 1) filters, other values leave it off).
    """
    return _verify_device_params("spec_verify_filtered", target_logits, draft_logits, draft_tokens, u_accept,
                                 u_sample, temperature, draft_lens, top_k, top_p, accepted_count, out_tokens,
                                 workspace, stream, debug, k1_events)


def _debug_struct(B, gamma, debug, k1_events):
    """An sv_debug pointing at the caller's preallocated diagnostic tensors and event pair."""
    import torch
    d = SvDebug()
    rows = 2 * gamma + 1
    dshapes = {"p_draft": ((B, gamma), torch.float64), "q_draft": ((B, gamma), torch.float64),
               "accept_prob": ((B, gamma), torch.float64), "row_max": ((B, rows), torch.float32),
               "row_sum": ((B, rows), torch.float64), "row_argmax": ((B, gamma + 1), torch.int32),
               "residual_mass": ((B,), torch.float64)}
    for name, (shape, dtype) in dshapes.items():
        t = (debug or {}).get(name)
        _expect(t, shape, dtype, f"debug[{name}]", optional=True)
        setattr(d, name, _ptr(t))
    if k1_events:
        d.k1_events[0] = k1_events[0].cuda_event
        d.k1_events[1] = k1_events[1].cuda_event
    return ctypes.pointer(d)


def _verify_device_params(entry, target_logits, draft_logits, draft_tokens, u_accept, u_sample, temperature,
                          draft_lens, top_k, top_p, accepted_count, out_tokens, workspace, stream, debug,
                          k1_events):
    lib = load_library()
    B, gamma, V = _shapes(target_logits)
    dt = _dtype_code(target_logits)
    _check_device(target_logits, draft_logits, draft_tokens, u_accept, u_sample, temperature, draft_lens,
                  top_k, top_p)
    with _on(stream):
        accepted_count, out_tokens = _outputs(B, gamma, target_logits.device, accepted_count, out_tokens)
    _check_all(target_logits, draft_logits, draft_tokens, u_accept, u_sample, accepted_count, out_tokens,
               greedy_only=False)
    import torch
    _expect(temperature, (B,), torch.float32, "temperature")
    _expect(draft_lens, (B,), torch.int32, "draft_lens", optional=True)
    _expect(top_k, (B,), torch.int32, "top_k", optional=True)
    _expect(top_p, (B,), torch.float32, "top_p", optional=True)
    with _on(stream):
        workspace, need = _workspace(B, gamma, V, dt, target_logits.device, workspace,
                                     filtered=entry == "spec_verify_filtered")
    if workspace.numel() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, {need} needed")
    dbg = _debug_struct(B, gamma, debug, k1_events) if (debug or k1_events) else None
    head = (_ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), _ptr(u_accept), _ptr(u_sample),
            _ptr(temperature), _ptr(draft_lens))
    tail = (B, gamma, V, dt, _ptr(accepted_count), _ptr(out_tokens), _ptr(workspace), workspace.numel(),
            _stream(stream), dbg)
    if entry == "spec_verify_filtered":
        rc = lib.spec_verify_filtered(*head, _ptr(top_k), _ptr(top_p), *tail)
    else:
        rc = lib.spec_verify_ex(*head, *tail)
    if rc != SV_OK:
        raise SpecVerifyError(rc, entry)
    return accepted_count, out_tokens


def spec_verify_tree_workspace_bytes(B: int, max_nodes: int, V: int, dtype: int) -> int:
    return int(load_library().spec_verify_tree_workspace_bytes(B, max_nodes, V, dtype))


def spec_verify_tree(target_logits, draft_logits, node_parent, node_tokens, u_accept, u_sample, temperature,
                     num_nodes=None, accepted_count=None, out_tokens=None, out_nodes=None, workspace=None,
                     stream=None):
    """Tree verification (see ``spec_verify_tree`` in include/specverify.h).

    target_logits [B, N+1, V], draft_logits [B, N, V] (bf16 or fp32); node_parent,
    node_tokens [B, N] int32; u_accept [B, N], u_sample [B], temperature [B] float32;
    num_nodes [B] int32 or None.  Returns (accepted_count [B], out_tokens [B, N+1],
    out_nodes [B, N]).
    """
    import torch
    lib = load_library()
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, max_nodes + 1, V]")
    B, n1, V = target_logits.shape
    N = n1 - 1
    dt = _dtype_code(target_logits)
    _check_device(target_logits, draft_logits, node_parent, node_tokens, u_accept, u_sample, temperature,
                  num_nodes)
    dev = target_logits.device
    _expect(target_logits, (B, N + 1, V), target_logits.dtype, "target_logits")
    _expect(draft_logits, (B, N, V), target_logits.dtype, "draft_logits", optional=N == 0)
    _expect(node_parent, (B, N), torch.int32, "node_parent", optional=N == 0)
    _expect(node_tokens, (B, N), torch.int32, "node_tokens", optional=N == 0)
    _expect(u_accept, (B, N), torch.float32, "u_accept", optional=N == 0)
    _expect(u_sample, (B,), torch.float32, "u_sample")
    _expect(temperature, (B,), torch.float32, "temperature")
    _expect(num_nodes, (B,), torch.int32, "num_nodes", optional=True)
    with _on(stream):
        if accepted_count is None:
            accepted_count = torch.empty(B, dtype=torch.int32, device=dev)
        if out_tokens is None:
            out_tokens = torch.empty((B, N + 1), dtype=torch.int32, device=dev)
        if out_nodes is None:
            out_nodes = torch.empty((B, max(N, 1)), dtype=torch.int32, device=dev)
    _expect(accepted_count, (B,), torch.int32, "accepted_count")
    _expect(out_tokens, (B, N + 1), torch.int32, "out_tokens")
    need = spec_verify_tree_workspace_bytes(B, N, V, dt)
    if need == 0:
        raise SpecVerifyError(SV_EINVAL, "spec_verify_tree_workspace_bytes")
    if workspace is None:
        with _on(stream):
            workspace = new_workspace(need, dev)
    if workspace.numel() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, {need} needed")
    rc = lib.spec_verify_tree(_ptr(target_logits), _ptr(draft_logits), _ptr(node_parent), _ptr(node_tokens),
                              _ptr(num_nodes), _ptr(u_accept), _ptr(u_sample), _ptr(temperature), B, N, V, dt,
                              _ptr(accepted_count), _ptr(out_tokens), _ptr(out_nodes), _ptr(workspace),
                              workspace.numel(), _stream(stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_tree")
    return accepted_count, out_tokens, out_nodes[:, :N]


def spec_sample_workspace_bytes(R: int, V: int, dtype: int) -> int:
    return int(load_library().spec_sample_workspace_bytes(R, V, dtype))


def spec_sample_filtered_workspace_bytes(R: int, V: int, dtype: int) -> int:
    return int(load_library().spec_sample_filtered_workspace_bytes(R, V, dtype))


def spec_sample(logits, u, temperature, tokens=None, workspace=None, stream=None, top_k=None, top_p=None):
    """One token per row of softmax(logits / T) by inverse CDF with the uniforms ``u``.

    logits: device [R, V] bf16/fp32; u: device [R] fp32; temperature: float, or a
    device fp32 tensor [R] of per-row temperatures (0 = arg-max).  ``top_k`` /
    ``top_p``: optional device tensors [R] (int32 / fp32) that truncate each row
    first (spec_sample_filtered).  Returns tokens [R] int32.
    """
    import torch
    lib = load_library()
    if logits.dim() != 2:
        raise ValueError("logits must be [R, V]")
    R, V = int(logits.shape[0]), int(logits.shape[1])
    dt = _dtype_code(logits)
    if top_k is not None or top_p is not None:
        with _on(stream):        # the fill is ordered before the kernels that read it
            temps = temperature if isinstance(temperature, torch.Tensor) else \
                torch.full((R,), float(temperature), dtype=torch.float32, device=logits.device)
        _check_device(logits, u, temps, top_k, top_p)
        _expect(logits, (R, V), None, "logits")
        _expect(u, (R,), torch.float32, "u")
        _expect(temps, (R,), torch.float32, "temperature")
        _expect(top_k, (R,), torch.int32, "top_k", optional=True)
        _expect(top_p, (R,), torch.float32, "top_p", optional=True)
        need = spec_sample_filtered_workspace_bytes(R, V, dt)
        with _on(stream):
            if tokens is None:
                tokens = torch.empty(R, dtype=torch.int32, device=logits.device)
            if workspace is None:
                workspace = new_workspace(need, logits.device)
        _expect(tokens, (R,), torch.int32, "tokens")
        rc = lib.spec_sample_filtered(_ptr(logits), _ptr(u), _ptr(temps), _ptr(top_k), _ptr(top_p), R, V, dt,
                                      _ptr(tokens), _ptr(workspace), workspace.numel(), _stream(stream))
        if rc != SV_OK:
            raise SpecVerifyError(rc, "spec_sample_filtered")
        return tokens
    per_row = isinstance(temperature, torch.Tensor)
    _check_device(logits, u, temperature if per_row else None)
    _expect(logits, (R, V), None, "logits")
    _expect(u, (R,), torch.float32, "u")
    if per_row:
        _expect(temperature, (R,), torch.float32, "temperature")
    need = spec_sample_workspace_bytes(R, V, dt)
    with _on(stream):
        if tokens is None:
            tokens = torch.empty(R, dtype=torch.int32, device=logits.device)
        if workspace is None:
            workspace = new_workspace(need, logits.device)
    _expect(tokens, (R,), torch.int32, "tokens")
    rc = lib.spec_sample(_ptr(logits), _ptr(u), 0.0 if per_row else float(temperature),
                         _ptr(temperature) if per_row else None, R, V, dt, _ptr(tokens), _ptr(workspace),
                         workspace.numel(), _stream(stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_sample")
    return tokens


class GammaPolicy:
    """Adaptive draft length (host-side state owned here; the arithmetic is in the C library).

    kind: SV_GAMMA_BY_BATCH, SV_GAMMA_EMA or SV_GAMMA_RATE_WINDOW.  ``next(batch)``
    returns the draft length for the next step; ``observe(accepted_count, gamma)``
    feeds back a step's accepted counts (host array or CPU/GPU tensor).
    """

    def __init__(self, kind: int, **fields):
        self._lib = load_library()
        self.state = SvGammaPolicy()
        rc = self._lib.spec_gamma_policy_init(ctypes.byref(self.state), int(kind))
        if rc != SV_OK:
            raise SpecVerifyError(rc, "spec_gamma_policy_init")
        for k, v in fields.items():
            cur = getattr(self.state, k)
            if isinstance(cur, ctypes.Array):
                for i, x in enumerate(v):
                    cur[i] = x
            else:
                setattr(self.state, k, v)

    def next(self, batch_size: int) -> int:
        g = self._lib.spec_gamma_next(ctypes.byref(self.state), int(batch_size))
        if g < 0:
            raise SpecVerifyError(g, "spec_gamma_next")
        return g

    def observe(self, accepted_count, gamma_used: int) -> None:
        import numpy as np
        if hasattr(accepted_count, "detach"):
            accepted_count = accepted_count.detach().cpu().numpy()
        a = np.ascontiguousarray(accepted_count, dtype=np.int32).reshape(-1)
        rc = self._lib.spec_gamma_observe(ctypes.byref(self.state), a.ctypes.data_as(ctypes.c_void_p),
                                          int(a.size), int(gamma_used))
        if rc != SV_OK:
            raise SpecVerifyError(rc, "spec_gamma_observe")
