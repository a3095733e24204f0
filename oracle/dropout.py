"""Attention with dropout on the probabilities, in float64 (test infrastructure only).

The alphabetamath page ("Reverse procedure", closing remark) has no dropout
in the base method and requires any dropout extension to replay, in the
reverse pass, the same realised mask as the forward pass.  The reading
taken here:

* Keep decisions Z_ij in {0, 1} are drawn per allowed pair (i, j) of unit
  u = b H + h from a counter-based generator, so the reverse pass regenerates
  them from (seed, u, i, j) instead of storing them.
* The drop probability is used in units of 1/256: p8 = round(256 p), and
  pair (i, j) is kept iff its 8-bit draw is >= p8, so P(keep) = 1 - p8 / 256
  exactly; kept weights are scaled by 256 / (256 - p8).
* The generator is Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
  random numbers: as easy as 1, 2, 3", SC 2011): counter (j // 4, i // 4,
  u, 0), key (seed mod 2^32, seed div 2^32).  Its four output words cover
  the 4 x 4 block of pairs with i // 4, j // 4: pair (i, j) takes byte
  j % 4 (least significant first) of word i % 4.
* The row statistics m, l, L are those of the undropped softmax; the output
  is Y = (P o Z) V / keep with P = softmax over A_i.

Gradients of <G, Y> with Z fixed: dV = (P o Z)^T G / keep,
dPd = (G V^T) o Z / keep, dS = P o (dPd - rowsum(P o dPd)),
dQ = c dS K, dK = c dS^T Q.
"""

from __future__ import annotations

import numpy as np

from . import dense

_M0, _M1 = 0xD2511F53, 0xCD9E8D57  # Philox4x32 round multipliers
_W0, _W1 = 0x9E3779B9, 0xBB67AE85  # Weyl key increments
_MASK32 = 0xFFFFFFFF


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32 with 10 rounds on arrays of uint32 counters; returns 4 uint32 arrays."""
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) & _MASK32 for x in (c0, c1, c2, c3))
    k0 = np.uint64(int(k0) & _MASK32)
    k1 = np.uint64(int(k1) & _MASK32)
    for r in range(10):
        p0 = np.uint64(_M0) * c0
        p1 = np.uint64(_M1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(_MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(_MASK32)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        k0 = np.uint64((int(k0) + _W0) & _MASK32)
        k1 = np.uint64((int(k1) + _W1) & _MASK32)
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))


def p8_of(p: float) -> int:
    """The drop probability in units of 1/256 (0 <= p8 <= 255)."""
    if not 0.0 <= p < 1.0:
        raise ValueError("dropout probability must be in [0, 1)")
    return min(255, int(np.floor(p * 256.0 + 0.5)))


def keep_mask(seed: int, unit: int, n: int, nk: int, p8: int) -> np.ndarray:
    """Z [n, nk] (bool) of one unit."""
    i = np.arange(n)[:, None]
    j = np.arange(nk)[None, :]
    words = philox4x32_10(j // 4, i // 4, np.full((n, nk), unit), 0, seed & _MASK32, seed >> 32)
    w = np.select([i % 4 == 0, i % 4 == 1, i % 4 == 2], words[:3], words[3])
    byte = (w >> (8 * (j % 4)).astype(np.uint32)) & np.uint32(0xFF)
    return byte >= p8


def forward(Q, K, V, c, allowed, Z, p8):
    """Y, L of one unit with keep mask Z (L of the undropped softmax)."""
    Y0, m, ell, L = dense.forward(Q, K, V, c, allowed)
    A = np.ones(Z.shape, bool) if allowed is None else allowed
    S = np.where(A, c * (np.asarray(Q, np.float64) @ np.asarray(K, np.float64).T), -np.inf)
    P = np.exp(S - L[:, None])
    keep = (256 - p8) / 256.0
    Y = ((P * Z) @ np.asarray(V, np.float64)) / keep
    return Y, L


def vjp(Q, K, V, c, allowed, Z, p8, G, Y=None):
    """dQ, dK, dV of <G, Y> with the keep mask Z held fixed.

    The row term D_i = sum_j P_ij dPd_ij equals <G_i, Y_i>.  By default it
    is taken in the first form (exact); given ``Y``, in the second, from that
    forward output: the reverse procedure consumes the output of a forward
    run (alphabetamath page, "Reverse procedure", delta_i), which a
    comparison with a bf16 device run passes as stored.
    """
    Q, K, V, G = (np.asarray(x, np.float64) for x in (Q, K, V, G))
    A = np.ones(Z.shape, bool) if allowed is None else allowed
    S = np.where(A, c * (Q @ K.T), -np.inf)
    E = np.exp(S - S.max(axis=1, keepdims=True))
    P = E / E.sum(axis=1, keepdims=True)
    keep = (256 - p8) / 256.0
    dV = (P * Z).T @ G / keep
    dPd = (G @ V.T) * Z / keep
    if Y is None:
        D = (P * dPd).sum(axis=1, keepdims=True)
    else:
        D = np.sum(G * np.asarray(Y, np.float64), axis=1, keepdims=True)
    dS = P * (dPd - D)
    return c * (dS @ K), c * (dS.T @ Q), dV
