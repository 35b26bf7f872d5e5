"""Seeded synthetic inputs for the verify step (shared by tests, smoke check and benchmark).

This module draws random numbers and lays out arrays.  It holds none of the
verify step's arithmetic: no softmax, no acceptance ratio, no residual, no
inverse-CDF sampling.  Draft tokens, which in a real system come from the
drafting step *before* verification, are drawn here with the Gumbel-max trick
(argmax of z/T plus Gumbel noise is an exact sample from softmax(z/T)); at
T = 0 the draft is the arg-max of the draft logits.

The five workload shapes stand in for the logits that a target / draft model
pair would produce on the pages' serving workloads (batch 1 to 128, up to 7
draft tokens, vocabularies of 32k to 152k entries).  No dataset item is used.

Draw order for one workload (one ``numpy.random.Generator(PCG64(seed))``):
  1. per-request parameters (ragged draft lengths, temperatures, draft noise);
  2. target noise, float32 normal, shape (B, gamma_max+1, V);
  3. a Zipf-like bias per target row: a random permutation pi of the vocabulary
     and bias[pi[j]] = -1.1 * ln(j + 1) (rank 1 gets bias 0);
  4. target logits = scale * noise + bias; draft logits = target logits of the
     first gamma_max positions + sigma * normal noise;
  5. one cast to the storage dtype (bf16 by round-to-nearest-even);
  6. draft tokens from the cast draft logits (Gumbel-max at T, arg-max at T=0);
  7. u_accept (B, gamma_max) and u_sample (B,) uniform in [0, 1), float32.
Rows that a ragged request does not own are filled with NaN.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"

BF16_NAN = np.uint16(0x7FC0)


# --------------------------------------------------------------------------- bf16 storage
def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns the uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> 16) & np.uint32(1)
    lsb += np.uint32(0x7FFF)
    lsb += bits            # no wrap for non-NaN inputs: the largest is 0xFF800000 + 0x8000
    lsb >>= 16
    out = lsb.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def f32_from_bf16_bits(h: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to float32."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------- workload container
@dataclass
class Workload:
    name: str
    B: int
    gamma: int            # gamma_max: the padding stride of the draft dimension
    V: int
    dtype: str            # "f32" or "bf16"
    target: np.ndarray    # [B, gamma+1, V] float32, or uint16 bf16 bits
    draft: np.ndarray     # [B, gamma, V]
    draft_tokens: np.ndarray  # [B, gamma] int32 (padding entries 0)
    u_accept: np.ndarray      # [B, gamma] float32
    u_sample: np.ndarray      # [B] float32
    temperature: np.ndarray   # [B] float32, 0 = greedy request
    lens: Optional[np.ndarray] = None  # [B] int32 draft lengths, None = all gamma
    scalar_temperature: Optional[float] = None  # set when every request shares T
    top_k: Optional[np.ndarray] = None  # [B] int32 per-request top-k (0: off), None = no filter
    top_p: Optional[np.ndarray] = None  # [B] float32 per-request top-p (1: off), None = no filter
    meta: dict = field(default_factory=dict)

    @property
    def filtered(self) -> bool:
        return self.top_k is not None or self.top_p is not None

    @property
    def draft_lens(self) -> np.ndarray:
        if self.lens is None:
            return np.full(self.B, self.gamma, dtype=np.int32)
        return self.lens

    def positions(self) -> int:
        """Number of draft positions verified in one call (sum of draft lengths)."""
        return int(self.draft_lens.sum())

    def rows_read(self) -> int:
        """Logit rows the method must read: gamma_b+1 target rows, plus gamma_b draft rows when T_b > 0."""
        g = self.draft_lens.astype(np.int64)
        stoch = (self.temperature > 0).astype(np.int64)
        return int(((g + 1) + stoch * g).sum())

    def elt_bytes(self) -> int:
        return 2 if self.dtype == BF16 else 4

    def bytes_alg(self) -> int:
        """Algorithmic logit bytes of one call (rows the method must read x V x element size)."""
        return self.rows_read() * self.V * self.elt_bytes()

    def to_torch(self, device):
        """Copy the arrays into torch tensors on ``device`` (bf16 bits become torch.bfloat16)."""
        import torch

        def logits(a):
            if self.dtype == BF16:
                return torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).to(device)
            return torch.from_numpy(np.ascontiguousarray(a)).to(device)

        def plain(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(device)

        d = dict(
            target=logits(self.target),
            draft=logits(self.draft),
            draft_tokens=plain(self.draft_tokens),
            u_accept=plain(self.u_accept),
            u_sample=plain(self.u_sample),
            temperature=plain(self.temperature),
            lens=None if self.lens is None else plain(self.lens),
            top_k=None if self.top_k is None else plain(self.top_k),
            top_p=None if self.top_p is None else plain(self.top_p),
        )
        return d


# --------------------------------------------------------------------------- pieces
def _zipf_bias_rows(rng: np.random.Generator, nrows: int, V: int) -> np.ndarray:
    """One Zipf-like bias row per target row: token pi[j] gets -1.1 ln(j+1)."""
    ranks = (-1.1 * np.log(np.arange(1, V + 1, dtype=np.float64))).astype(np.float32)
    out = np.empty((nrows, V), dtype=np.float32)
    for r in range(nrows):
        perm = rng.permutation(V)
        out[r, perm] = ranks
    return out


def _cast(z: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return bf16_bits_from_f32(z)
    return np.ascontiguousarray(z, dtype=np.float32)


def _as_f64(stored: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return f32_from_bf16_bits(stored).astype(np.float64)
    return stored.astype(np.float64)


def _draw_drafts(rng, draft_stored, dtype, temps, lens, gamma, block_elems: int = 1 << 23) -> np.ndarray:
    """Draft tokens: Gumbel-max sample of softmax(z_q / T) (exact), arg-max at T = 0.

    Rows are visited in (request, position) order, in blocks of at most
    ``block_elems`` logits, drawing one uniform per logit of every stochastic row.
    """
    B, _, V = draft_stored.shape
    tokens = np.zeros((B, gamma), dtype=np.int32)
    rows = [(b, i) for b in range(B) for i in range(int(lens[b]))]
    per = max(1, block_elems // V)
    for start in range(0, len(rows), per):
        blk = rows[start:start + per]
        bi = np.array([r[0] for r in blk])
        ii = np.array([r[1] for r in blk])
        z = _as_f64(draft_stored[bi, ii], dtype)          # [n, V]
        T = temps[bi].astype(np.float64)
        stoch = T > 0
        pick = np.argmax(z, axis=1)
        if stoch.any():
            u = rng.random((int(stoch.sum()), V))
            with np.errstate(divide="ignore"):
                gumbel = -np.log(-np.log(u))
            pick[stoch] = np.argmax(z[stoch] / T[stoch, None] + gumbel, axis=1)
        tokens[bi, ii] = pick
    return tokens


def build(name: str, seed: int, B: int, gamma: int, V: int, dtype: str, *,
          target_scale: float, zipf: bool, sigma, temps, lens=None,
          rng: Optional[np.random.Generator] = None) -> Workload:
    """Generic generator following the draw order in the module docstring.

    ``sigma``: scalar or per-request array of draft-noise scales.
    ``temps``: scalar or per-request array (0 = greedy request).
    ``lens``: None (every request has gamma drafts) or per-request draft lengths.
    ``rng``: a generator that already drew the per-request parameters (step 1).
    """
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    scalar_T = None
    if np.isscalar(temps):
        scalar_T = float(temps)
        temps = np.full(B, temps, dtype=np.float32)
    temps = np.asarray(temps, dtype=np.float32)
    sig = np.full(B, sigma, dtype=np.float32) if np.isscalar(sigma) else np.asarray(sigma, np.float32)
    glens = np.full(B, gamma, dtype=np.int32) if lens is None else np.asarray(lens, dtype=np.int32)

    # 2. target noise, 3. bias, 4. logits
    zp = rng.standard_normal((B, gamma + 1, V), dtype=np.float32)
    zp *= np.float32(target_scale)
    if zipf:
        zp += _zipf_bias_rows(rng, B * (gamma + 1), V).reshape(B, gamma + 1, V)
    zq = rng.standard_normal((B, gamma, V), dtype=np.float32)
    zq *= sig[:, None, None]
    zq += zp[:, :gamma, :]
    # 5. cast
    target = _cast(zp, dtype)
    del zp
    draft = _cast(zq, dtype)
    del zq
    # 6. drafts
    tokens = _draw_drafts(rng, draft, dtype, temps, glens, gamma)
    # 7. uniforms
    u_accept = rng.random((B, gamma), dtype=np.float32)
    u_sample = rng.random(B, dtype=np.float32)
    # padding rows of ragged requests are poisoned
    if lens is not None:
        nan = BF16_NAN if dtype == BF16 else np.float32(np.nan)
        for b in range(B):
            g = int(glens[b])
            target[b, g + 1:, :] = nan
            draft[b, g:, :] = nan
    return Workload(name=name, B=B, gamma=gamma, V=V, dtype=dtype, target=target, draft=draft,
                    draft_tokens=tokens, u_accept=u_accept, u_sample=u_sample,
                    temperature=temps, lens=None if lens is None else glens,
                    scalar_temperature=scalar_T,
                    meta=dict(seed=seed, target_scale=target_scale, zipf=zipf))


# --------------------------------------------------------------------------- the five workloads
CONFIG_NAMES = {
    0: "B1_g4_V1000_f32_T1",
    1: "B1_g5_V32000_f32_T1_zipf",
    2: "B8_g3_V128256_bf16_T0.7_zipf",
    3: "B64_g5_V128256_bf16_T1_zipf",
    4: "B128_gragged1-7_V152064_bf16_mixedT_zipf",
}


def make_config(i: int, seed: Optional[int] = None, greedy: bool = False) -> Workload:
    """Workload ``i`` (0..4).  ``greedy=True`` is the T = 0 mode of workload 3."""
    if seed is None:
        seed = 1000 + i
    if i == 0:
        w = build(CONFIG_NAMES[0], seed, 1, 4, 1000, F32, target_scale=3.0, zipf=False, sigma=0.7, temps=1.0)
    elif i == 1:
        w = build(CONFIG_NAMES[1], seed, 1, 5, 32000, F32, target_scale=4.0, zipf=True, sigma=0.5, temps=1.0)
    elif i == 2:
        w = build(CONFIG_NAMES[2], seed, 8, 3, 128256, BF16, target_scale=4.0, zipf=True, sigma=1.0, temps=0.7)
    elif i == 3:
        T = 0.0 if greedy else 1.0
        name = CONFIG_NAMES[3] + ("_greedy" if greedy else "")
        w = build(name, seed, 64, 5, 128256, BF16, target_scale=4.0, zipf=True, sigma=0.5, temps=T)
    elif i == 4:
        B, gmax = 128, 7
        rng = np.random.Generator(np.random.PCG64(seed))
        lens = rng.integers(1, gmax + 1, size=B).astype(np.int32)
        temps = rng.choice(np.array([0.0, 0.6, 1.0], dtype=np.float32), size=B)
        sigma = rng.uniform(0.2, 1.5, size=B).astype(np.float32)
        w = build(CONFIG_NAMES[4], seed, B, gmax, 152064, BF16, target_scale=5.0, zipf=True,
                  sigma=sigma, temps=temps, lens=lens, rng=rng)
    else:
        raise ValueError(f"no workload {i}")
    w.meta["config"] = i
    w.meta["greedy"] = greedy
    return w


def make_random(seed: int, B: int, gamma: int, V: int, dtype: str = F32, *, temps=1.0, lens=None,
                target_scale: float = 3.0, sigma=0.7, zipf: bool = False) -> Workload:
    """Small random case for parity sweeps (same recipe, arbitrary shape)."""
    return build(f"rand_s{seed}_B{B}_g{gamma}_V{V}_{dtype}", seed, B, gamma, V, dtype,
                 target_scale=target_scale, zipf=zipf, sigma=sigma, temps=temps, lens=lens)


def from_logits(target_f32: np.ndarray, draft_f32: np.ndarray, draft_tokens, u_accept, u_sample,
                temps, dtype: str = F32, lens=None, name: str = "explicit") -> Workload:
    """Wrap explicit arrays (used by the hand-built pin cases)."""
    target_f32 = np.asarray(target_f32, dtype=np.float32)
    B, g1, V = target_f32.shape
    gamma = g1 - 1
    draft_f32 = np.asarray(draft_f32, dtype=np.float32).reshape(B, gamma, V)
    scalar_T = None
    if np.isscalar(temps):
        scalar_T = float(temps)
        temps = np.full(B, temps, dtype=np.float32)
    return Workload(name=name, B=B, gamma=gamma, V=V, dtype=dtype,
                    target=_cast(target_f32, dtype), draft=_cast(draft_f32, dtype),
                    draft_tokens=np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(B, gamma),
                    u_accept=np.ascontiguousarray(u_accept, dtype=np.float32).reshape(B, gamma),
                    u_sample=np.ascontiguousarray(u_sample, dtype=np.float32).reshape(B),
                    temperature=np.ascontiguousarray(temps, dtype=np.float32).reshape(B),
                    lens=None if lens is None else np.ascontiguousarray(lens, dtype=np.int32),
                    scalar_temperature=scalar_T)


# --------------------------------------------------------------------------- trees of drafts
def tree_parents(width: int, depth: int) -> np.ndarray:
    """Parent of each node of a full tree with `width` children per node and `depth` levels, nodes
    numbered level by level (-1: the verified prefix).  Parents precede their children."""
    parents, level = [], [-1]
    for _ in range(depth):
        nxt = []
        for pa in level:
            for _ in range(width):
                parents.append(pa)
                nxt.append(len(parents) - 1)
        level = nxt
    return np.array(parents, dtype=np.int32)


@dataclass
class TreeWorkload:
    name: str
    B: int
    N: int                     # max_nodes: the padding stride of the node dimension
    V: int
    dtype: str
    target: np.ndarray         # [B, N+1, V]: row j = target at position j (0: prefix, n+1: node n)
    draft: np.ndarray          # [B, N, V]: row j = the draft distribution at position j
    parent: np.ndarray         # [B, N] int32
    tokens: np.ndarray         # [B, N] int32
    u_accept: np.ndarray       # [B, N] float32
    u_sample: np.ndarray       # [B] float32
    temperature: np.ndarray    # [B] float32
    num_nodes: Optional[np.ndarray] = None  # [B] int32, None = N
    meta: dict = field(default_factory=dict)

    def node_counts(self) -> np.ndarray:
        return np.full(self.B, self.N, np.int32) if self.num_nodes is None else self.num_nodes

    def bytes_alg(self) -> int:
        """Logit bytes of every row a tree could need: every target row of a used position and,
        for stochastic requests, every draft row of a position that can have children."""
        n = self.node_counts().astype(np.int64)
        stoch = (self.temperature > 0).astype(np.int64)
        return int(((n + 1) + stoch * n).sum()) * self.V * (2 if self.dtype == BF16 else 4)

    def bytes_walked(self, out_nodes: np.ndarray, accepted_count: np.ndarray) -> int:
        """Logit bytes of the rows a walk needs, given its accepted paths: the target row of
        every position it visits and, for stochastic requests, the draft row of each visited
        position that has children."""
        n = self.node_counts()
        rows = 0
        for b in range(self.B):
            par = self.parent[b, :n[b]]
            visited = [0] + [int(x) + 1 for x in out_nodes[b, :int(accepted_count[b])]]
            for p in visited:
                rows += 1
                if self.temperature[b] > 0 and np.any(par == p - 1):
                    rows += 1
        return rows * self.V * (2 if self.dtype == BF16 else 4)

    def to_torch(self, device):
        import torch

        def logits(a):
            t = torch.from_numpy(np.ascontiguousarray(a))
            return (t.view(torch.bfloat16) if self.dtype == BF16 else t).to(device)

        def plain(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(device)

        return dict(target=logits(self.target), draft=logits(self.draft), parent=plain(self.parent),
                    tokens=plain(self.tokens), u_accept=plain(self.u_accept), u_sample=plain(self.u_sample),
                    temperature=plain(self.temperature),
                    num_nodes=None if self.num_nodes is None else plain(self.num_nodes))


def build_tree(name: str, seed: int, B: int, width: int, depth: int, V: int, dtype: str, *,
               target_scale: float, zipf: bool, sigma: float, temps, num_nodes=None,
               block_elems: int = 1 << 23) -> TreeWorkload:
    """Seeded tree workload.  Draw order: target noise (+ Zipf bias), draft noise, node tokens
    (children of a position drawn independently from softmax(z_q / T) by Gumbel-max; at T = 0 the
    children are the draft row's largest logits, in order), then u_accept and u_sample."""
    rng = np.random.Generator(np.random.PCG64(seed))
    par1 = tree_parents(width, depth)
    N = par1.size
    temps = np.full(B, temps, np.float32) if np.isscalar(temps) else np.asarray(temps, np.float32)
    zp = rng.standard_normal((B, N + 1, V), dtype=np.float32)
    zp *= np.float32(target_scale)
    if zipf:
        zp += _zipf_bias_rows(rng, B * (N + 1), V).reshape(B, N + 1, V)
    zq = rng.standard_normal((B, N, V), dtype=np.float32)
    zq *= np.float32(sigma)
    zq += zp[:, :N, :]
    target = _cast(zp, dtype)
    del zp
    draft = _cast(zq, dtype)
    del zq
    parent = np.tile(par1, (B, 1))
    tokens = np.zeros((B, N), np.int32)
    # greedy requests: the children of a position are its draft row's largest logits
    for b in np.nonzero(temps == 0)[0]:
        for j in range(N):
            kids = np.nonzero(par1 == j - 1)[0]
            if kids.size:
                z = _as_f64(draft[b, j], dtype)
                top = np.argsort(-z, kind="stable")[:kids.size]
                tokens[b, kids] = top
    # stochastic requests: independent draws, rows visited in (request, node) order
    rows = [(b, n) for b in np.nonzero(temps > 0)[0] for n in range(N)]
    per = max(1, block_elems // V)
    for s0 in range(0, len(rows), per):
        blk = rows[s0:s0 + per]
        bi = np.array([r[0] for r in blk])
        ni = np.array([r[1] for r in blk])
        z = _as_f64(draft[bi, par1[ni] + 1], dtype)
        u = rng.random((len(blk), V))
        with np.errstate(divide="ignore"):
            g = -np.log(-np.log(u))
        tokens[bi, ni] = np.argmax(z / temps[bi].astype(np.float64)[:, None] + g, axis=1)
    u_accept = rng.random((B, N), dtype=np.float32)
    u_sample = rng.random(B, dtype=np.float32)
    nn = None if num_nodes is None else np.asarray(num_nodes, np.int32)
    return TreeWorkload(name=name, B=B, N=N, V=V, dtype=dtype, target=target, draft=draft, parent=parent,
                        tokens=tokens, u_accept=u_accept, u_sample=u_sample, temperature=temps, num_nodes=nn,
                        meta=dict(seed=seed, width=width, depth=depth))
