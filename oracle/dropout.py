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


def keep_mask_at(seed: int, unit: int, rows, cols, p8: int) -> np.ndarray:
    """Z at the pairs rows x cols of one unit (bool [len(rows), len(cols)]).

    The decisions of ``keep_mask``, with one generator call per 4 x 4 block
    of pairs the index sets touch instead of one per pair, for units too
    large to draw pair by pair: block (a, b)'s word r holds the draws of row
    4 a + r, byte e (least significant first) that of column 4 b + e.
    """
    rows = np.asarray(rows, np.int64)
    cols = np.asarray(cols, np.int64)
    bi, at_i = np.unique(rows // 4, return_inverse=True)
    bj, at_j = np.unique(cols // 4, return_inverse=True)
    words = np.stack(philox4x32_10(bj[None, :], bi[:, None], np.full((len(bi), len(bj)), unit), 0,
                                   seed & _MASK32, seed >> 32))  # [word r, row block a, column block b]
    draws = (words[:, :, :, None] >> (8 * np.arange(4, dtype=np.uint32))) & np.uint32(0xFF)  # [r, a, b, e]
    kept = (draws >= p8).transpose(1, 0, 2, 3).reshape(4 * len(bi), 4 * len(bj))  # [4 a + r, 4 b + e]
    ri, ci = 4 * at_i + rows % 4, 4 * at_j + cols % 4
    if np.array_equal(ri, np.arange(kept.shape[0])) and np.array_equal(ci, np.arange(kept.shape[1])):
        return kept
    return kept[np.ix_(ri, ci)]


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


def output_rows(Q, K, V, c, allowed_rows, L, Z_rows, p8, rows):
    """Rows of Y = (P o Z) V / keep, with P_ij = exp(c q_i.k_j - L_i) on A_i
    and L the undropped softmax's logsumexp (from ``dense.forward``), for
    units too large for ``forward``.  allowed_rows(r) and Z_rows(r) give
    bool [len(r), nk]."""
    Q, K, V, L = (np.asarray(x, np.float64) for x in (Q, K, V, L))
    rows = np.asarray(rows)
    A = allowed_rows(rows)
    S = np.where(A, c * (Q[rows] @ K.T), -np.inf)
    P = np.exp(S - L[rows, None])
    keep = (256 - p8) / 256.0
    return ((P * Z_rows(rows)) @ V) / keep


def grads_sampled(Q, K, V, c, allowed_rows, G, L, Y, rows, cols, Z_r, Z_c, p8):
    """dQ for sampled query rows and dK, dV for sampled key columns of <G, Y>
    with the keep mask held fixed (the formulas of ``vjp``: dPd = (G V^T) o
    Z / keep, dS = P o (dPd - D), D_i = <G_i, Y_i> from the given output of
    every row), one output row or column at a time.  Z_r: Z[rows] (bool
    [len(rows), nk]); Z_c: Z[:, cols] (bool [n, len(cols)])."""
    Q, K, V, G, L, Y = (np.asarray(x, np.float64) for x in (Q, K, V, G, L, Y))
    n = Q.shape[0]
    rows, cols = np.asarray(rows), np.asarray(cols)
    keep = (256 - p8) / 256.0
    D = np.sum(G * Y, axis=1)
    A = allowed_rows(rows)
    P = np.exp(np.where(A, c * (Q[rows] @ K.T), -np.inf) - L[rows, None])
    dS = P * ((G[rows] @ V.T) * Z_r / keep - D[rows, None])
    dQ = c * (dS @ K)
    Ac = allowed_rows(np.arange(n))[:, cols]
    Pc = np.exp(np.where(Ac, c * (Q @ K[cols].T), -np.inf) - L[:, None])
    dSc = Pc * ((G @ V[cols].T) * Z_c / keep - D[:, None])
    dK = c * (dSc.T @ Q)
    dV = (Pc * Z_c).T @ G / keep
    return dQ, dK, dV
