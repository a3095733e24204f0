"""Seeded synthetic workloads for exact tiled attention.

This module only *generates inputs*: random matrices, allowed-key sets and
their packed bit representation, and round-to-nearest-even conversion of the
generated float32 values to bfloat16.  It holds none of the attention
arithmetic, so that both the float64 oracle (``oracle/``) and the HIP path
can consume the same inputs without sharing any code that computes a result.

Problem statement followed (exact tiled softmax attention, alphabetamath
page, "Inputs"): positive integers n, d, v; Q, K in R^{n x d}; V in
R^{n x v}; a real scale c; nonempty allowed-key sets A_1..A_n read on demand
from caller-owned storage.  Batched, multi-head use applies the same problem
per (batch, head) unit (HarshvardhanJ/FlashAttention README, list of
extensions: multi-head and batched inputs).

Recipe (the pages fix no inputs; these are the synthetic stand-ins):

* ``numpy.random.default_rng(seed)`` (PCG64); Q, K, V, G drawn in that order
  with ``standard_normal(shape, dtype=float32)``, each multiplied in float32
  by its workload factor; bf16 workloads then round to bfloat16 (RNE).
* The bitmask workload draws, after G and head by head, one
  ``rng.random((n, n), dtype=float32) < n_global / n`` Bernoulli matrix and
  ORs it with a sliding window j - i in [-window/2, window/2), clipped to
  [0, n).  The window holds j = i, so every row is nonempty.
* Masks are packed LSB-first into uint32 words, row-major
  ``[head][i][ceil(n/32)]``; pad bits past n are zero.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

MASK_NONE = "none"
MASK_CAUSAL = "causal"
MASK_BITMASK = "bitmask"


@dataclass(frozen=True)
class Workload:
    """One synthetic problem: shapes, value recipe, mask recipe and seed."""

    name: str
    B: int
    H: int
    n: int
    d: int
    v: int
    dtype: str  # "f32" or "bf16": element type of Q, K, V, O, dO, dQ, dK, dV
    mask: str  # MASK_NONE / MASK_CAUSAL / MASK_BITMASK
    seed: int
    scale: float  # the real scale c applied to <Q_i, K_j>
    qk_std: float = 1.0
    vg_std: float = 1.0
    oracle_blocks: tuple = (32,)  # key-block sizes b the oracle's tiled route uses
    window: int = 0  # bitmask only: sliding-window width
    n_global: int = 0  # bitmask only: expected random global keys per row
    note: str = ""

    def with_(self, **kw) -> "Workload":
        fields = dict(self.__dict__)
        fields.update(kw)
        return Workload(**fields)


WORKLOADS = {
    w.name: w
    for w in [
        Workload(
            name="f32_n256_d64",
            B=1, H=1, n=256, d=64, v=64, dtype="f32", mask=MASK_NONE, seed=0,
            scale=1.0 / math.sqrt(64), oracle_blocks=(1, 32, 256),
            note="single head, non-causal, fp32",
        ),
        Workload(
            name="f32_causal_n1000_d80",
            B=1, H=1, n=1000, d=80, v=80, dtype="f32", mask=MASK_CAUSAL, seed=1,
            scale=1.0 / math.sqrt(80), oracle_blocks=(1, 17, 64, 1000),
            note="causal, n not a power of two, d=80 not a multiple of 64, fp32",
        ),
        Workload(
            name="bf16_b4h16_n4096_d128",
            B=4, H=16, n=4096, d=128, v=128, dtype="bf16", mask=MASK_NONE, seed=2,
            scale=1.0 / math.sqrt(128), qk_std=0.5, oracle_blocks=(128,),
            note="batch 4 x 16 heads, non-causal, bf16, Q,K ~ 0.5 N(0,1)",
        ),
        Workload(
            name="bf16_causal_h32_n16384_d128",
            B=1, H=32, n=16384, d=128, v=128, dtype="bf16", mask=MASK_CAUSAL, seed=3,
            scale=1.0 / math.sqrt(128), oracle_blocks=(128,),
            note="1 x 32 heads, causal, n=16384, bf16: long-sequence throughput case",
        ),
        Workload(
            name="bf16_bitmask_b2h8_n8192_d64v128",
            B=2, H=8, n=8192, d=64, v=128, dtype="bf16", mask=MASK_BITMASK, seed=4,
            scale=1.0 / math.sqrt(64), qk_std=2.0, oracle_blocks=(128,),
            window=1024, n_global=64,
            note="2 x 8 heads, explicit per-head bitmask: window 1024 + Bernoulli(64/n)",
        ),
    ]
}

# Short workload order used by tests and the benchmark (small first).
ORDER = list(WORKLOADS)


# ---------------------------------------------------------------------------
# bfloat16 conversion (round to nearest, ties to even) on float32 bit patterns
# ---------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bfloat16 bit patterns, round-to-nearest-even.

    Inputs are finite by construction; NaN handling is not needed here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float32 values (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 value, returned as float32."""
    return bf16_bits_to_f32(bf16_bits(x))


# ---------------------------------------------------------------------------
# Masks
# ---------------------------------------------------------------------------

def causal_allowed(n: int, rows=None, nk: int | None = None, offset: int = 0) -> np.ndarray:
    """A_i = {j <= i + offset} (0-based) over nk keys (default n), as bool [len(rows), nk]."""
    nk = n if nk is None else nk
    rows = np.arange(n) if rows is None else np.asarray(rows)
    return np.arange(nk)[None, :] <= rows[:, None] + offset


def window_allowed(n: int, window: int, rows=None) -> np.ndarray:
    """j - i in [-window/2, window/2), clipped to [0, n)."""
    rows = np.arange(n) if rows is None else np.asarray(rows)
    off = np.arange(n)[None, :] - rows[:, None]
    half = window // 2
    return (off >= -half) & (off < half)


def pack_bits(allowed: np.ndarray) -> np.ndarray:
    """bool [..., n] -> uint32 [..., ceil(n/32)], bit (j & 31) of word j >> 5."""
    allowed = np.asarray(allowed, dtype=bool)
    n = allowed.shape[-1]
    words = (n + 31) // 32
    pad = words * 32 - n
    if pad:
        allowed = np.concatenate(
            [allowed, np.zeros(allowed.shape[:-1] + (pad,), dtype=bool)], axis=-1)
    by = np.packbits(allowed, axis=-1, bitorder="little")  # [..., words*4] uint8
    return np.ascontiguousarray(by).view("<u4").astype(np.uint32)


def unpack_bits(words: np.ndarray, n: int) -> np.ndarray:
    """Inverse of pack_bits (used only to check the packing itself)."""
    by = np.ascontiguousarray(words.astype("<u4")).view(np.uint8)
    return np.unpackbits(by, axis=-1, bitorder="little")[..., :n].astype(bool)


# ---------------------------------------------------------------------------
# Generated problem
# ---------------------------------------------------------------------------

@dataclass
class Problem:
    """Generated inputs of one workload.

    ``Q, K, V, G`` are float32 arrays holding exactly the values the device
    receives (already bf16-rounded for bf16 workloads).  For bf16 workloads
    ``*_bits`` hold the uint16 patterns.  ``mask_bool[h]`` is the boolean
    allowed matrix of head h (bitmask workloads only; shared across the
    batch) and ``mask_words`` its packed form ``[H, n, ceil(n/32)]``.
    """

    w: Workload
    Q: np.ndarray
    K: np.ndarray
    V: np.ndarray
    G: np.ndarray
    bits: dict = field(default_factory=dict)
    mask_bool: np.ndarray | None = None
    mask_words: np.ndarray | None = None

    def allowed(self, h: int, rows=None) -> np.ndarray | None:
        """Boolean allowed matrix rows for head h; None means 'all keys'."""
        n = self.w.n
        if self.w.mask == MASK_NONE:
            if rows is None:
                return np.ones((n, n), dtype=bool)
            return np.ones((len(rows), n), dtype=bool)
        if self.w.mask == MASK_CAUSAL:
            return causal_allowed(n, rows)
        m = self.mask_bool[h]
        return m if rows is None else m[np.asarray(rows)]


def generate(w: Workload | str, *, heads: int | None = None, n: int | None = None) -> Problem:
    """Generate a workload's inputs from its seed.

    ``heads``/``n`` optionally shrink the problem (same recipe, same seed)
    for quick tests; the full workload is generated when both are None.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    if heads is not None or n is not None:
        w = w.with_(H=heads if heads is not None else w.H, n=n if n is not None else w.n)
    rng = np.random.default_rng(w.seed)
    B, H, n_, d, v = w.B, w.H, w.n, w.d, w.v

    def draw(shape, std):
        x = rng.standard_normal(shape, dtype=np.float32)
        if std != 1.0:
            x = x * np.float32(std)
        return x

    Q = draw((B, H, n_, d), w.qk_std)
    K = draw((B, H, n_, d), w.qk_std)
    V = draw((B, H, n_, v), w.vg_std)
    G = draw((B, H, n_, v), w.vg_std)
    prob = Problem(w=w, Q=Q, K=K, V=V, G=G)
    if w.dtype == "bf16":
        for name in ("Q", "K", "V", "G"):
            b = bf16_bits(getattr(prob, name))
            prob.bits[name] = b
            setattr(prob, name, bf16_bits_to_f32(b))
    if w.mask == MASK_BITMASK:
        masks = np.empty((H, n_, n_), dtype=bool)
        win = window_allowed(n_, w.window)
        p = np.float32(w.n_global / n_)
        for h in range(H):
            bern = rng.random((n_, n_), dtype=np.float32) < p
            masks[h] = bern | win
        prob.mask_bool = masks
        prob.mask_words = pack_bits(masks)
    return prob


def custom(Q, K, V, G, *, scale: float, mask: str = MASK_NONE, allowed=None,
           dtype: str = "f32", name: str = "custom") -> Problem:
    """Wrap caller-made arrays ([B,H,n,.] float32) as a Problem.

    For ``mask == MASK_BITMASK`` pass ``allowed`` as bool [H, n, n].
    bf16 problems expect values that are already bf16-representable.
    """
    Q, K, V, G = (np.ascontiguousarray(a, dtype=np.float32) for a in (Q, K, V, G))
    B, H, n, d = Q.shape
    w = Workload(name=name, B=B, H=H, n=n, d=d, v=V.shape[-1], dtype=dtype, mask=mask,
                 seed=-1, scale=float(scale))
    prob = Problem(w=w, Q=Q, K=K, V=V, G=G)
    if dtype == "bf16":
        for nm in ("Q", "K", "V", "G"):
            b = bf16_bits(getattr(prob, nm))
            prob.bits[nm] = b
            setattr(prob, nm, bf16_bits_to_f32(b))
    if mask == MASK_BITMASK:
        allowed = np.asarray(allowed, dtype=bool)
        prob.mask_bool = allowed
        prob.mask_words = pack_bits(allowed)
    return prob


def allowed_pairs(w: Workload, prob: Problem | None = None) -> int:
    """#A summed over all (batch, head) units: n^2, n(n+1)/2 or the popcount."""
    n = w.n
    if w.mask == MASK_NONE:
        per = [n * n] * w.H
    elif w.mask == MASK_CAUSAL:
        per = [n * (n + 1) // 2] * w.H
    else:
        per = [int(prob.mask_bool[h].sum()) for h in range(w.H)]
    return w.B * sum(per)


def flops(w: Workload, pairs: int) -> tuple[float, float]:
    """Algorithmic FLOPs: forward 2#A(d+v) (QK^T + PV); backward 2#A(3d+2v)."""
    return 2.0 * pairs * (w.d + w.v), 2.0 * pairs * (3 * w.d + 2 * w.v)
