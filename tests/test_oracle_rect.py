"""Pins of the oracle on rectangular problems (n query rows, nk key rows).

The maitreyasuin page's tiled forward takes Tq query rows against Tk key
rows; the definition of every output is row-wise and does not depend on
nk = n.  A causal mask with an offset allows key j for query i iff
j <= i + offset.  These tests pin the oracle there against:

* the textbook softmax (scipy) on each row's allowed keys;
* the second route (key-block procedure) for the forward and the reverse;
* central finite differences of the forward for the VJP;
* the exact merge of results over disjoint key ranges (the merge * of the
  row summaries, read as in oracle/tiled.py): L = ln sum_s e^{L_s},
  O = sum_s e^{L_s - L} O_s, and per-shard gradients taken with the global
  statistics, which add up (dQ) or concatenate (dK, dV) to the full VJP.
"""

from __future__ import annotations

import numpy as np
import pytest
from scipy.special import softmax

import workloads as W
from oracle import dense, tiled

CASES = [(7, 19, 0), (19, 7, 0), (12, 30, 18), (30, 12, -5), (1, 33, 32), (25, 1, 0)]


def _problem(n, nk, d=5, v=4, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.normal(size=(n, d)), rng.normal(size=(nk, d)), rng.normal(size=(nk, v)),
            rng.normal(size=(n, v)))


def _rows(A):
    return np.nonzero(A.any(axis=1))[0]


@pytest.mark.parametrize("n,nk,off", CASES)
def test_rectangular_forward_is_the_textbook_softmax(n, nk, off):
    Q, K, V, _ = _problem(n, nk, seed=n + nk)
    for A in (None, W.causal_allowed(n, nk=nk, offset=off)):
        rows = np.arange(n) if A is None else _rows(A)
        Ar = None if A is None else A[rows]
        Y, _, _, L = dense.forward(Q[rows], K, V, 0.7, Ar)
        for k, i in enumerate(rows):
            keys = np.arange(nk) if A is None else np.nonzero(A[i])[0]
            s = 0.7 * (K[keys] @ Q[i])
            assert np.abs(Y[k] - softmax(s) @ V[keys]).max() < 1e-13
            assert abs(L[k] - (s.max() + np.log(np.exp(s - s.max()).sum()))) < 1e-13


@pytest.mark.parametrize("n,nk,off", CASES)
def test_rectangular_routes_agree(n, nk, off):
    Q, K, V, G = _problem(n, nk, seed=3 * n + nk)
    A = W.causal_allowed(n, nk=nk, offset=off)
    rows = _rows(A)
    Q, G, A = Q[rows], G[rows], A[rows]
    Y, m, ell, L = dense.forward(Q, K, V, 1.3, A)
    for b in (1, 4, nk):
        Yt, mt, lt, Lt = tiled.forward(Q, K, V, 1.3, A, b)
        assert np.abs(Yt - Y).max() < 1e-12 and np.abs(Lt - L).max() < 1e-12
        dQ, dK, dV = tiled.reverse(Q, K, V, 1.3, A, b, Yt, mt, lt, G)
        rQ, rK, rV = dense.vjp(Q, K, V, 1.3, A, G)
        for x, r in ((dQ, rQ), (dK, rK), (dV, rV)):
            assert np.abs(x - r).max() <= 1e-10 * max(1.0, np.abs(r).max())


def test_rectangular_vjp_finite_differences():
    n, nk, off, c = 3, 5, 1, 0.9
    Q, K, V, G = _problem(n, nk, d=2, v=3, seed=11)
    A = W.causal_allowed(n, nk=nk, offset=off)
    dQ, dK, dV = dense.vjp(Q, K, V, c, A, G)
    h = 1e-6
    for X, dX, which in ((Q, dQ, 0), (K, dK, 1), (V, dV, 2)):
        ref = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            args_p = [Q.copy(), K.copy(), V.copy()]
            args_m = [Q.copy(), K.copy(), V.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            fp = (G * dense.forward(*args_p, c, A)[0]).sum()
            fm = (G * dense.forward(*args_m, c, A)[0]).sum()
            ref[idx] = (fp - fm) / (2 * h)
        assert np.abs(dX - ref).max() <= 1e-7 * max(1.0, np.abs(ref).max()), which


def _shard_forward(Q, K, V, c, A):
    """O, L over one key range; rows with no allowed key there: O = 0, L = -inf."""
    n = Q.shape[0]
    O, L = np.zeros((n, V.shape[1])), np.full(n, -np.inf)
    rows = _rows(A)
    if rows.size:
        Y, _, _, Lr = dense.forward(Q[rows], K, V, c, A[rows])
        O[rows], L[rows] = Y, Lr
    return O, L


@pytest.mark.parametrize("splits", [[0, 40, 97], [0, 1, 50, 96, 97], [0, 60, 97]])
def test_key_range_results_merge_exactly(splits):
    n, c = 97, 0.8
    Q, K, V, G = _problem(n, n, d=6, v=5, seed=len(splits))
    A = W.causal_allowed(n)
    Y, m, ell, L = dense.forward(Q, K, V, c, A)
    parts = []
    for k0, k1 in zip(splits, splits[1:]):
        As = W.causal_allowed(n, nk=k1 - k0, offset=-k0)  # absolute key k0 + j <= i
        assert np.array_equal(As, A[:, k0:k1])
        parts.append(_shard_forward(Q, K[k0:k1], V[k0:k1], c, As))
    Ls = np.stack([p[1] for p in parts])
    Lm = np.logaddexp.reduce(Ls, axis=0)
    Om = sum(np.exp(Ls[s] - Lm)[:, None] * parts[s][0] for s in range(len(parts)))
    assert np.abs(Lm - L).max() < 1e-13 and np.abs(Om - Y).max() < 1e-13
    # Gradients per key range with the global statistics.
    rQ, rK, rV = dense.vjp(Q, K, V, c, A, G)
    dQ = np.zeros_like(Q)
    for k0, k1 in zip(splits, splits[1:]):
        dq, dk, dv = tiled.reverse(Q, K[k0:k1], V[k0:k1], c, A[:, k0:k1], 8, Y, m, ell, G)
        dQ += dq
        assert np.abs(dk - rK[k0:k1]).max() < 1e-12 and np.abs(dv - rV[k0:k1]).max() < 1e-12
    assert np.abs(dQ - rQ).max() < 1e-12
