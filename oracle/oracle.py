"""ctypes marshalling for the C oracle (test infrastructure only; no arithmetic here)."""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "spec_verify_oracle.c")
LIB = os.path.join(HERE, "libspecverify_oracle.so")

ORACLE_F32 = 0
ORACLE_BF16 = 1
GAMMA_MAX = 32


def build(extra_flags=(), src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math, no contraction)."""
    tmp = f"{out}.tmp{os.getpid()}"
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
           "-shared", "-fPIC", "-I", HERE, *extra_flags, "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True, cwd=HERE)
    os.replace(tmp, out)   # atomic: a concurrent loader sees the old or the new library, whole
    return out


class _Trace(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "p_draft", "q_draft", "accept_prob", "row_max", "row_sum", "row_argmax",
        "residual_mass", "flags", "accept_margin", "cdf_margin")]


class _Args(ctypes.Structure):
    _fields_ = [
        ("target", ctypes.c_void_p), ("draft", ctypes.c_void_p), ("dtype", ctypes.c_int),
        ("draft_tokens", ctypes.c_void_p), ("u_accept", ctypes.c_void_p), ("u_sample", ctypes.c_void_p),
        ("temperature", ctypes.c_void_p), ("lens", ctypes.c_void_p),
        ("top_k", ctypes.c_void_p), ("top_p", ctypes.c_void_p),
        ("B", ctypes.c_int), ("gamma", ctypes.c_int), ("V", ctypes.c_int),
        ("accepted_count", ctypes.c_void_p), ("out_tokens", ctypes.c_void_p),
        ("trace", ctypes.POINTER(_Trace)),
    ]


class _TreeArgs(ctypes.Structure):
    _fields_ = [
        ("target", ctypes.c_void_p), ("draft", ctypes.c_void_p), ("dtype", ctypes.c_int),
        ("parent", ctypes.c_void_p), ("tokens", ctypes.c_void_p), ("num_nodes", ctypes.c_void_p),
        ("u_accept", ctypes.c_void_p), ("u_sample", ctypes.c_void_p), ("temperature", ctypes.c_void_p),
        ("B", ctypes.c_int), ("max_nodes", ctypes.c_int), ("V", ctypes.c_int),
        ("accepted_count", ctypes.c_void_p), ("out_tokens", ctypes.c_void_p), ("out_nodes", ctypes.c_void_p),
        ("flags", ctypes.c_void_p),
    ]


_lib = None


def _open(path: str) -> ctypes.CDLL:
    lib = ctypes.CDLL(path)
    lib.oracle_spec_verify.argtypes = [ctypes.POINTER(_Args)]
    lib.oracle_spec_verify.restype = ctypes.c_int
    lib.oracle_spec_verify_tree.argtypes = [ctypes.POINTER(_TreeArgs)]
    lib.oracle_spec_verify_tree.restype = ctypes.c_int
    return lib


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the compiled oracle (compiling it first if no build exists).

    ``path`` opens another build of the same interface (used by the tests that
    plant mistakes in a copy of the oracle)."""
    global _lib
    if path is not None:
        return _open(path)
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _lib = _open(LIB)
    return _lib


@dataclass
class OracleResult:
    accepted_count: np.ndarray  # [B] int32
    out_tokens: np.ndarray      # [B, gamma+1] int32
    p_draft: Optional[np.ndarray] = None
    q_draft: Optional[np.ndarray] = None
    accept_prob: Optional[np.ndarray] = None
    row_max: Optional[np.ndarray] = None
    row_sum: Optional[np.ndarray] = None
    row_argmax: Optional[np.ndarray] = None
    residual_mass: Optional[np.ndarray] = None
    flags: Optional[np.ndarray] = None
    accept_margin: Optional[np.ndarray] = None
    cdf_margin: Optional[np.ndarray] = None


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def spec_verify(target, draft, draft_tokens, u_accept, u_sample, temperature, lens=None,
                dtype: Optional[str] = None, trace: bool = True, lib: Optional[ctypes.CDLL] = None,
                top_k=None, top_p=None) -> OracleResult:
    """Run the oracle on host arrays.

    target: [B, gamma+1, V] float32, or uint16 holding bf16 bits (dtype="bf16").
    draft:  [B, gamma, V] same storage.  temperature: scalar or [B].
    """
    if dtype is None:
        dtype = "bf16" if np.asarray(target).dtype == np.uint16 else "f32"
    store = np.uint16 if dtype == "bf16" else np.float32
    target = np.ascontiguousarray(target, dtype=store)
    B, g1, V = target.shape
    gamma = g1 - 1
    draft = np.ascontiguousarray(draft, dtype=store).reshape(B, gamma, V) if gamma > 0 else None
    tokens = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(B, gamma)
    ua = np.ascontiguousarray(u_accept, dtype=np.float32).reshape(B, gamma)
    us = np.ascontiguousarray(u_sample, dtype=np.float32).reshape(B)
    if np.isscalar(temperature):
        temperature = np.full(B, temperature, dtype=np.float32)
    temps = np.ascontiguousarray(temperature, dtype=np.float32).reshape(B)
    lens_a = None if lens is None else np.ascontiguousarray(lens, dtype=np.int32).reshape(B)
    if top_k is not None and np.isscalar(top_k):
        top_k = np.full(B, top_k, dtype=np.int32)
    if top_p is not None and np.isscalar(top_p):
        top_p = np.full(B, top_p, dtype=np.float32)
    tk_a = None if top_k is None else np.ascontiguousarray(top_k, dtype=np.int32).reshape(B)
    tp_a = None if top_p is None else np.ascontiguousarray(top_p, dtype=np.float32).reshape(B)

    count = np.zeros(B, dtype=np.int32)
    out = np.full((B, gamma + 1), -7, dtype=np.int32)
    res = OracleResult(accepted_count=count, out_tokens=out)
    tr = None
    if trace:
        nrows = 2 * gamma + 1
        res.p_draft = np.full((B, gamma), np.nan)
        res.q_draft = np.full((B, gamma), np.nan)
        res.accept_prob = np.full((B, gamma), np.nan)
        res.row_max = np.full((B, nrows), np.nan)
        res.row_sum = np.full((B, nrows), np.nan)
        res.row_argmax = np.full((B, gamma + 1), -1, dtype=np.int32)
        res.residual_mass = np.full(B, np.nan)
        res.flags = np.zeros(B, dtype=np.int32)
        res.accept_margin = np.full(B, np.inf)
        res.cdf_margin = np.full(B, np.inf)
        tr = _Trace(*[_ptr(getattr(res, n)) for n, _ in _Trace._fields_])
    args = _Args(_ptr(target), _ptr(draft), ORACLE_BF16 if dtype == "bf16" else ORACLE_F32,
                 _ptr(tokens), _ptr(ua), _ptr(us), _ptr(temps), _ptr(lens_a), _ptr(tk_a), _ptr(tp_a), B, gamma, V,
                 _ptr(count), _ptr(out), ctypes.pointer(tr) if tr is not None else None)
    rc = (lib or load()).oracle_spec_verify(ctypes.byref(args))
    if rc != 0:
        raise ValueError(f"oracle_spec_verify rejected its arguments (code {rc})")
    return res


def run_workload(w, trace: bool = True, lib: Optional[ctypes.CDLL] = None) -> OracleResult:
    """Convenience: run the oracle on a ``workloads.Workload``."""
    return spec_verify(w.target, w.draft, w.draft_tokens, w.u_accept, w.u_sample, w.temperature,
                       lens=w.lens, dtype=w.dtype, trace=trace, lib=lib,
                       top_k=getattr(w, "top_k", None), top_p=getattr(w, "top_p", None))


def sample(logits, u, temperature, dtype: Optional[str] = None, lib: Optional[ctypes.CDLL] = None,
           top_k=None, top_p=None) -> np.ndarray:
    """One token per row of softmax(logits / T) (optionally top-k / top-p filtered)
    by inverse CDF with the uniforms u.

    This is the oracle's verify step with no drafts (every row is a bonus row)."""
    logits = np.asarray(logits)
    R, V = logits.shape
    res = spec_verify(logits.reshape(R, 1, V), np.zeros((R, 0, V), dtype=logits.dtype), np.zeros((R, 0)),
                      np.zeros((R, 0)), u, temperature, dtype=dtype, trace=True, lib=lib, top_k=top_k, top_p=top_p)
    return res.out_tokens[:, 0].copy(), res


@dataclass
class TreeResult:
    accepted_count: np.ndarray  # [B] int32: nodes on the accepted path
    out_tokens: np.ndarray      # [B, max_nodes+1] int32: path tokens, then the drawn token, -1 after
    out_nodes: np.ndarray       # [B, max_nodes] int32: path node indices, -1 after
    flags: np.ndarray           # [B] int32: bit0 accept band, bit1 CDF band, bit2 zero-mass fallback,
                                #   bit4 a band in units of the current target's unnormalised mass only


def spec_verify_tree(target, draft, parent, tokens, u_accept, u_sample, temperature, num_nodes=None,
                     dtype: Optional[str] = None, lib: Optional[ctypes.CDLL] = None) -> TreeResult:
    """Tree verification on host arrays.

    target: [B, max_nodes+1, V] (row j = target at position j; position 0 is the
    verified prefix, position n+1 is node n); draft: [B, max_nodes, V] (row j = q
    at position j); parent, tokens, u_accept: [B, max_nodes]; u_sample: [B].
    """
    if dtype is None:
        dtype = "bf16" if np.asarray(target).dtype == np.uint16 else "f32"
    store = np.uint16 if dtype == "bf16" else np.float32
    target = np.ascontiguousarray(target, dtype=store)
    B, n1, V = target.shape
    Nmax = n1 - 1
    draft = np.ascontiguousarray(draft, dtype=store).reshape(B, Nmax, V) if Nmax > 0 else None
    par = np.ascontiguousarray(parent, dtype=np.int32).reshape(B, Nmax)
    tok = np.ascontiguousarray(tokens, dtype=np.int32).reshape(B, Nmax)
    ua = np.ascontiguousarray(u_accept, dtype=np.float32).reshape(B, Nmax)
    us = np.ascontiguousarray(u_sample, dtype=np.float32).reshape(B)
    if np.isscalar(temperature):
        temperature = np.full(B, temperature, dtype=np.float32)
    temps = np.ascontiguousarray(temperature, dtype=np.float32).reshape(B)
    nn = None if num_nodes is None else np.ascontiguousarray(num_nodes, dtype=np.int32).reshape(B)
    res = TreeResult(accepted_count=np.zeros(B, np.int32), out_tokens=np.full((B, Nmax + 1), -7, np.int32),
                     out_nodes=np.full((B, Nmax), -7, np.int32), flags=np.zeros(B, np.int32))
    args = _TreeArgs(_ptr(target), _ptr(draft), 1 if dtype == "bf16" else 0, _ptr(par), _ptr(tok), _ptr(nn),
                     _ptr(ua), _ptr(us), _ptr(temps), B, Nmax, V, _ptr(res.accepted_count), _ptr(res.out_tokens),
                     _ptr(res.out_nodes), _ptr(res.flags))
    rc = (lib or load()).oracle_spec_verify_tree(ctypes.byref(args))
    if rc != 0:
        raise ValueError(f"oracle_spec_verify_tree rejected its arguments (code {rc})")
    return res
