"""Pins that tie the float64 oracle to facts other than itself.

Each ``check_*`` takes the oracle modules (``dense``, ``tiled``, ``tilemap``)
as arguments and raises AssertionError on failure, so that
``test_oracle_pins.py`` runs them on the real oracle and
``test_oracle_mutants.py`` runs them on copies of the oracle with one
planted mistake each (every mutant must fail at least one check).

Facts used (none of them re-types the oracle's own formulas):

* closed forms of softmax attention: c = 0 or equal keys give the mean of
  the allowed V_j and L_i = ln |A_i| (+ c<Q_i, k>); a one-key-per-row mask
  selects V_pi(i); n = 1 gives Y = V; two keys give a sigmoid mix;
* hand-derived numbers in ``tests/golden/closed_forms.json``;
* a library softmax / logsumexp (scipy.special) on masked rows;
* invariants: key shift, permutation equivariance, convex hull,
  sum_j exp(s_ij - L_i) = 1;
* block-size independence b in {1, ..., n} of the key-block route
  (trentorch exercise constraint: identical output for every block size),
  also with score ranges wide enough to overflow an unguarded rescale;
* central finite differences of <G, Y> in float64 (ob1 page: backward
  checked against central differences);
* gradient identities: sum_j dK_j = 0, sum_j dV_j = sum_i G_i,
  <dQ, Q> = <dK, K>, <dV, V> = <G, Y>, and the zero cases.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.special

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = max(np.abs(b).max(initial=0.0), 1e-300)
    return float(np.abs(a - b).max(initial=0.0) / den)


def rand_mask(rng, n, nk=None, p=0.4):
    nk = n if nk is None else nk
    A = rng.random((n, nk)) < p
    A[np.arange(n), rng.integers(0, nk, n)] = True  # every row nonempty
    return A


def masks_for(rng, n):
    return {
        "none": None,
        "causal": workloads.causal_allowed(n),
        "bitmask": rand_mask(rng, n),
    }


def full(A, n):
    return np.ones((n, n), bool) if A is None else A


# ---------------------------------------------------------------------------
# Forward pins
# ---------------------------------------------------------------------------

def check_closed_forms(dense):
    rng = np.random.default_rng(11)
    n, d, v = 13, 5, 3
    Q, K, V = rng.normal(size=(n, d)), rng.normal(size=(n, d)), rng.normal(size=(n, v))
    for name, A in masks_for(rng, n).items():
        Af = full(A, n)
        cnt = Af.sum(1)
        mean = (Af.astype(float) @ V) / cnt[:, None]
        # c = 0: uniform weights over A_i.
        Y, m, ell, L = dense.forward(Q, K, V, 0.0, A)
        assert rel(Y, mean) < 1e-13, name
        assert np.abs(L - np.log(cnt)).max() < 1e-13, name
        # Q = 0: same.
        Y, _, _, L = dense.forward(np.zeros_like(Q), K, V, 0.7, A)
        assert rel(Y, mean) < 1e-13, name
        # All keys equal to k: same means, L_i = c<Q_i,k> + ln|A_i|.
        k = rng.normal(size=d)
        Ke = np.tile(k, (n, 1))
        c = 0.9
        Y, _, _, L = dense.forward(Q, Ke, V, c, A)
        assert rel(Y, mean) < 1e-13, name
        assert np.abs(L - (c * Q @ k + np.log(cnt))).max() < 1e-12, name
    # Causal with c = 0: prefix means.
    Y, _, _, _ = dense.forward(Q, K, V, 0.0, workloads.causal_allowed(n))
    pref = np.cumsum(V, 0) / np.arange(1, n + 1)[:, None]
    assert rel(Y, pref) < 1e-13
    # One allowed key per row, A_i = {pi(i)}: Y_i = V_pi(i), L_i = s_i,pi(i).
    pi = rng.permutation(n)
    A = np.zeros((n, n), bool)
    A[np.arange(n), pi] = True
    c = 1.3
    Y, _, _, L = dense.forward(Q, K, V, c, A)
    assert rel(Y, V[pi]) < 1e-15
    assert np.abs(L - c * (Q * K[pi]).sum(1)).max() < 1e-13
    # n = 1: Y = V, L = c<Q,K>.
    Y, _, _, L = dense.forward(Q[:1], K[:1], V[:1], c, None)
    assert rel(Y, V[:1]) < 1e-15 and abs(L[0] - c * Q[0] @ K[0]) < 1e-13
    # Two keys: Y_i = sigma(s1 - s2) V1 + sigma(s2 - s1) V2.
    Q2, K2, V2 = Q[:4], K[:2], V[:2]
    Y, _, _, L = dense.forward(Q2, K2, V2, c, np.ones((4, 2), bool))
    s = c * Q2 @ K2.T
    w1 = 1.0 / (1.0 + np.exp(s[:, 1] - s[:, 0]))
    assert rel(Y, w1[:, None] * V2[0] + (1 - w1)[:, None] * V2[1]) < 1e-13
    assert np.abs(L - np.logaddexp(s[:, 0], s[:, 1])).max() < 1e-13


def check_golden(dense, tiled):
    with open(os.path.join(GOLDEN, "closed_forms.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        Q, K, V = (np.array(case[k], float) for k in ("Q", "K", "V"))
        c = float(case["c"])
        A = None if case["mask"] == "none" else np.array(case["allowed"], bool)
        Y, _, _, L = dense.forward(Q, K, V, c, A)
        assert np.abs(Y - np.array(case["Y"])).max() < 1e-12, case["name"]
        assert np.abs(L - np.array([_num(x) for x in case["L"]])).max() < 1e-12, case["name"]
        for b in (1, 2, Q.shape[0]):
            Yt, _, _, Lt = tiled.forward(Q, K, V, c, A, b)
            assert np.abs(Yt - np.array(case["Y"])).max() < 1e-12, case["name"]
        if "G" in case:
            G = np.array(case["G"], float)
            exp = [np.array([[_num(x) for x in row] for row in case[k]]) for k in ("dQ", "dK", "dV")]
            for got in (dense.vjp(Q, K, V, c, A, G),):
                for g, e, nm in zip(got, exp, ("dQ", "dK", "dV")):
                    assert np.abs(g - e).max() < 1e-12, (case["name"], nm)
            Yt, mt, lt, _ = tiled.forward(Q, K, V, c, A, 1)
            got = tiled.reverse(Q, K, V, c, A, 1, Yt, mt, lt, G)
            for g, e, nm in zip(got, exp, ("dQ", "dK", "dV")):
                assert np.abs(g - e).max() < 1e-12, (case["name"], nm, "tiled")


def _num(x):
    """Golden numbers are floats or strings like 'ln(4)' / '0.75*ln(3)'."""
    if isinstance(x, (int, float)):
        return float(x)
    return float(eval(x, {"__builtins__": {}}, {"ln": math.log}))


def check_library_softmax(dense):
    rng = np.random.default_rng(12)
    n, d, v = 40, 7, 6
    Q, K, V = rng.normal(size=(n, d)), rng.normal(size=(n, d)), rng.normal(size=(n, v))
    for name, A in masks_for(rng, n).items():
        for c in (0.37, -1.1, 2.5):
            Y, m, ell, L = dense.forward(Q, K, V, c, A)
            Af = full(A, n)
            for i in range(n):
                idx = np.nonzero(Af[i])[0]
                s = c * K[idx] @ Q[i]
                w = scipy.special.softmax(s)
                assert np.abs(Y[i] - w @ V[idx]).max() < 1e-13, (name, c, i)
                assert abs(L[i] - scipy.special.logsumexp(s)) < 1e-12, (name, c, i)
                assert abs(m[i] - s.max()) < 1e-13
                assert abs(ell[i] - np.exp(s - s.max()).sum()) < 1e-12


def check_invariants(dense):
    rng = np.random.default_rng(13)
    n, d, v = 24, 6, 5
    Q, K, V = rng.normal(size=(n, d)), rng.normal(size=(n, d)), rng.normal(size=(n, v))
    c = 0.8
    for name, A in masks_for(rng, n).items():
        Af = full(A, n)
        Y, _, _, L = dense.forward(Q, K, V, c, A)
        # Key shift: K_j += u leaves Y, adds c<Q_i,u> to L.
        u = rng.normal(size=d)
        Y2, _, _, L2 = dense.forward(Q, K + u, V, c, A)
        assert rel(Y2, Y) < 1e-12 and np.abs(L2 - L - c * Q @ u).max() < 1e-12, name
        # Key permutation with the mask permuted the same way.
        p = rng.permutation(n)
        Y3, _, _, L3 = dense.forward(Q, K[p], V[p], c, Af[:, p])
        assert rel(Y3, Y) < 1e-13 and np.abs(L3 - L).max() < 1e-13, name
        # Query permutation permutes outputs.
        Y4, _, _, L4 = dense.forward(Q[p], K, V, c, Af[p])
        assert rel(Y4, Y[p]) < 1e-13 and np.abs(L4 - L[p]).max() < 1e-13, name
        # Convex hull of the allowed V_j.
        lo = np.where(Af[:, :, None], V[None], np.inf).min(1)
        hi = np.where(Af[:, :, None], V[None], -np.inf).max(1)
        assert np.all(Y >= lo - 1e-13) and np.all(Y <= hi + 1e-13), name
        # Probabilities recovered from L sum to one.
        S = c * Q @ K.T
        tot = np.where(Af, np.exp(np.where(Af, S, 0) - L[:, None]), 0).sum(1)
        assert np.abs(tot - 1).max() < 1e-13, name
        # Scaling c by t equals scaling Q by t.
        Y5, _, _, L5 = dense.forward(3 * Q, K, V, c, A)
        Y6, _, _, L6 = dense.forward(Q, K, V, 3 * c, A)
        assert rel(Y5, Y6) < 1e-13 and np.abs(L5 - L6).max() < 1e-12, name


def check_block_independence(dense, tiled):
    """Key-block route equals the definition for every block size."""
    for wname in ("f32_n256_d64", "f32_causal_n1000_d80"):
        prob = workloads.generate(wname)
        w = prob.w
        Q, K, V = prob.Q[0, 0], prob.K[0, 0], prob.V[0, 0]
        A = None if w.mask == "none" else prob.allowed(0)
        Yd, md, ld, Ld = dense.forward(Q, K, V, w.scale, A)
        for b in w.oracle_blocks:
            Yt, mt, lt, Lt = tiled.forward(Q, K, V, w.scale, A, b)
            assert rel(Yt, Yd) < 1e-12, (wname, b)
            assert np.abs(Lt - Ld).max() < 1e-12, (wname, b)
            assert np.abs(mt - md).max() < 1e-12, (wname, b)
    # Random mask with empty per-block intersections, odd sizes, many blocks.
    rng = np.random.default_rng(14)
    n, d, v = 77, 9, 4
    Q, K, V = rng.normal(size=(n, d)), rng.normal(size=(n, d)), rng.normal(size=(n, v))
    A = rand_mask(rng, n, p=0.05)
    Yd, _, _, Ld = dense.forward(Q, K, V, 0.6, A)
    for b in (1, 3, 16, 76, 77, 100):
        Yt, _, _, Lt = tiled.forward(Q, K, V, 0.6, A, b)
        assert rel(Yt, Yd) < 1e-12 and np.abs(Lt - Ld).max() < 1e-12, b


def check_wide_scores(dense, tiled):
    """Score ranges beyond exp's float64 range: the merge must use the true max."""
    rng = np.random.default_rng(15)
    n, d, v = 30, 4, 3
    Q, K, V = rng.normal(size=(n, d)), rng.normal(size=(n, d)), rng.normal(size=(n, v))
    K[::3] *= 40.0  # some keys give scores far above the others
    c = 60.0
    for name, A in masks_for(rng, n).items():
        S = c * Q @ K.T
        Af = full(A, n)
        spread = (np.where(Af, S, -np.inf).max(1) - np.where(Af, S, np.inf).min(1)).max()
        assert spread > 1500.0  # exp of the spread overflows float64
        Yd, _, _, Ld = dense.forward(Q, K, V, c, A)
        assert np.all(np.isfinite(Yd)) and np.all(np.isfinite(Ld))
        Af = full(A, n)
        # The winner per row dominates: Y_i is V at the row's argmax.
        arg = np.where(Af, S, -np.inf).argmax(1)
        srt = np.sort(np.where(Af, S, -np.inf), 1)
        gap = srt[:, -1] - srt[:, -2]
        clear = gap > 60.0
        assert clear.any() and np.abs(Yd[clear] - V[arg[clear]]).max(initial=0.0) < 1e-12
        for b in (1, 4, 7, n):
            Yt, _, _, Lt = tiled.forward(Q, K, V, c, A, b)
            assert np.all(np.isfinite(Yt)), (name, b)
            assert rel(Yt, Yd) < 1e-12 and np.abs(Lt - Ld).max() < 1e-9 * np.abs(Ld).max(), (name, b)


# ---------------------------------------------------------------------------
# Gradient pins
# ---------------------------------------------------------------------------

def fd_grads(forward_fn, Q, K, V, G, h=1e-6):
    """Central differences of <G, Y(Q, K, V)>."""
    out = []
    args = [Q, K, V]
    for which in range(3):
        X = args[which]
        g = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            vals = []
            for sgn in (1.0, -1.0):
                a = [x.copy() for x in args]
                a[which][idx] += sgn * h
                vals.append(float((G * forward_fn(*a)).sum()))
            g[idx] = (vals[0] - vals[1]) / (2 * h)
        out.append(g)
    return out


def check_dense_vjp_fd(dense):
    rng = np.random.default_rng(16)
    for n, d, v in ((1, 1, 1), (2, 3, 1), (5, 4, 3), (8, 3, 3)):
        Q, K, V = rng.normal(size=(n, d)), rng.normal(size=(n, d)), rng.normal(size=(n, v))
        G = rng.normal(size=(n, v))
        for name, A in masks_for(rng, n).items():
            for c in (0.7, -1.3):
                fwd = lambda q, k, vv: dense.forward(q, k, vv, c, A)[0]  # noqa: E731
                ref = fd_grads(fwd, Q, K, V, G)
                got = dense.vjp(Q, K, V, c, A, G)
                for g, r, nm in zip(got, ref, "QKV"):
                    assert np.abs(g - r).max() <= 1e-6 * max(1.0, np.abs(r).max()), (n, name, c, nm)


def check_tiled_reverse_fd(tiled):
    rng = np.random.default_rng(17)
    for n, d, v in ((2, 1, 1), (5, 3, 3), (8, 4, 3)):
        Q, K, V = rng.normal(size=(n, d)), rng.normal(size=(n, d)), rng.normal(size=(n, v))
        G = rng.normal(size=(n, v))
        for name, A in masks_for(rng, n).items():
            c = 0.9
            for b in (1, 3, n):
                fwd = lambda q, k, vv: tiled.forward(q, k, vv, c, A, b)[0]  # noqa: E731
                ref = fd_grads(fwd, Q, K, V, G)
                Y, m, ell, _ = tiled.forward(Q, K, V, c, A, b)
                got = tiled.reverse(Q, K, V, c, A, b, Y, m, ell, G)
                for g, r, nm in zip(got, ref, "QKV"):
                    assert np.abs(g - r).max() <= 1e-6 * max(1.0, np.abs(r).max()), (n, name, b, nm)


def check_reverse_routes_agree(dense, tiled):
    """delta-form block reverse vs rowsum(P o dP) dense VJP on the f32 workloads."""
    for wname in ("f32_n256_d64", "f32_causal_n1000_d80"):
        prob = workloads.generate(wname)
        w = prob.w
        Q, K, V, G = prob.Q[0, 0], prob.K[0, 0], prob.V[0, 0], prob.G[0, 0]
        A = None if w.mask == "none" else prob.allowed(0)
        ref = dense.vjp(Q, K, V, w.scale, A, G)
        for b in w.oracle_blocks:
            Y, m, ell, _ = tiled.forward(Q, K, V, w.scale, A, b)
            got = tiled.reverse(Q, K, V, w.scale, A, b, Y, m, ell, G)
            for g, r, nm in zip(got, ref, "QKV"):
                assert rel(g, r) < 1e-10, (wname, b, nm)


def check_grad_identities(dense, tiled):
    rng = np.random.default_rng(18)
    n, d, v = 19, 5, 4
    Q, K, V = rng.normal(size=(n, d)), rng.normal(size=(n, d)), rng.normal(size=(n, v))
    G = rng.normal(size=(n, v))
    for name, A in masks_for(rng, n).items():
        c = 0.75
        Y = dense.forward(Q, K, V, c, A)[0]
        Yt, mt, lt, _ = tiled.forward(Q, K, V, c, A, 4)
        for route, (dQ, dK, dV) in (("dense", dense.vjp(Q, K, V, c, A, G)),
                                    ("tiled", tiled.reverse(Q, K, V, c, A, 4, Yt, mt, lt, G))):
            tag = (name, route)
            assert np.abs(dK.sum(0)).max() < 1e-12, tag
            assert np.abs(dV.sum(0) - G.sum(0)).max() < 1e-12, tag
            assert abs((dQ * Q).sum() - (dK * K).sum()) < 1e-11, tag
            assert abs((dV * V).sum() - (G * Y).sum()) < 1e-11, tag
        # Zero cases.
        for route, grads in (("dense", dense.vjp(Q, K, V, 0.0, A, G)),
                             ("tiled", tiled.reverse(Q, K, V, 0.0, A, 4,
                                                     *tiled.forward(Q, K, V, 0.0, A, 4)[:3], G))):
            assert np.abs(grads[0]).max() < 1e-15 and np.abs(grads[1]).max() < 1e-15, (name, route)
        Z = np.zeros_like(Q)
        for route, grads in (("dense", dense.vjp(Z, K, V, c, A, G)),
                             ("tiled", tiled.reverse(Z, K, V, c, A, 4,
                                                     *tiled.forward(Z, K, V, c, A, 4)[:3], G))):
            assert np.abs(grads[1]).max() < 1e-15, (name, route)
        Ke = np.tile(rng.normal(size=d), (n, 1))
        for route, grads in (("dense", dense.vjp(Q, Ke, V, c, A, G)),
                             ("tiled", tiled.reverse(Q, Ke, V, c, A, 4,
                                                     *tiled.forward(Q, Ke, V, c, A, 4)[:3], G))):
            assert np.abs(grads[0]).max() < 1e-13, (name, route)
    # One key per row: no gradient reaches Q or K; dV_pi(i) = G_i.
    pi = rng.permutation(n)
    A = np.zeros((n, n), bool)
    A[np.arange(n), pi] = True
    dQ, dK, dV = dense.vjp(Q, K, V, 1.1, A, G)
    assert np.abs(dQ).max() < 1e-15 and np.abs(dK).max() < 1e-15
    assert np.abs(dV[pi] - G).max() < 1e-15
    Yt, mt, lt, _ = tiled.forward(Q, K, V, 1.1, A, 3)
    dQ, dK, dV = tiled.reverse(Q, K, V, 1.1, A, 3, Yt, mt, lt, G)
    # <G_i, V_j> and delta_i = <G_i, Y_i> are summed in different orders here.
    assert np.abs(dQ).max() < 1e-13 and np.abs(dK).max() < 1e-13
    assert np.abs(dV[pi] - G).max() < 1e-15


def check_self_attention_fd(dense):
    """Q = K = V = X, c = 1 (HarshvardhanJ README): dX = dQ + dK + dV."""
    rng = np.random.default_rng(19)
    n, d = 6, 3
    X = rng.normal(size=(n, d))
    G = rng.normal(size=(n, d))
    for name, A in masks_for(rng, n).items():
        f = lambda x: float((G * dense.forward(x, x, x, 1.0, A)[0]).sum())  # noqa: E731
        h = 1e-6
        ref = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            ref[idx] = (f(Xp) - f(Xm)) / (2 * h)
        dQ, dK, dV = dense.vjp(X, X, X, 1.0, A, G)
        assert np.abs(dQ + dK + dV - ref).max() <= 1e-6 * max(1, np.abs(ref).max()), name


def check_sampled_grads(dense):
    """Row/column-sampled reverse formulas equal the full dense VJP."""
    rng = np.random.default_rng(20)
    n, d, v = 50, 6, 7
    Q, K, V = rng.normal(size=(n, d)), rng.normal(size=(n, d)), rng.normal(size=(n, v))
    G = rng.normal(size=(n, v))
    for name, A in masks_for(rng, n).items():
        Af = full(A, n)
        c = 0.6
        Y, _, _, L = dense.forward(Q, K, V, c, A)
        rows = np.array([0, 7, 49])
        cols = np.array([1, 25, 48])
        dQs, dKs, dVs = dense.grads_sampled(Q, K, V, c, lambda r: Af[r], G, L, Y, rows, cols)
        dQ, dK, dV = dense.vjp(Q, K, V, c, A, G)
        assert rel(dQs, dQ[rows]) < 1e-12, name
        assert rel(dKs, dK[cols]) < 1e-12, name
        assert rel(dVs, dV[cols]) < 1e-12, name
        Yr, Lr = dense.forward_rows(Q, K, V, c, Af[rows], rows)
        assert rel(Yr, Y[rows]) < 1e-15 and np.abs(Lr - L[rows]).max() < 1e-15, name


# ---------------------------------------------------------------------------
# Tile map pins
# ---------------------------------------------------------------------------

def check_tilemap(tilemap):
    for n in (1, 5, 64, 100, 257):
        A = workloads.causal_allowed(n)
        for Bq, Bk in ((1, 1), (16, 16), (32, 64), (64, 32), (128, 128), (128, 64)):
            tm = tilemap.tile_map(A, Bq, Bk)
            assert np.array_equal(tm, tilemap.causal_tile_map(n, Bq, Bk)), (n, Bq, Bk)
            # Brute-force classification of each tile.
            for a in range(tm.shape[0]):
                for t in range(tm.shape[1]):
                    rows = range(a * Bq, min(n, (a + 1) * Bq))
                    cols = range(t * Bk, t * Bk + Bk)
                    vals = [j < n and j <= i for i in rows for j in cols]
                    want = 2 if all(vals) else (1 if any(vals) else 0)
                    assert tm[a, t] == want, (n, Bq, Bk, a, t)
    # Square aligned causal tiles: T(T+1)/2 nonempty, T of them partial.
    T = 8
    tm = tilemap.causal_tile_map(T * 32, 32, 32)
    assert tilemap.nonempty_tiles(tm) == T * (T + 1) // 2
    assert int((tm == 1).sum()) == T
    # No mask: all full except key-tail tiles.
    tm = tilemap.tile_map(np.ones((100, 100), bool), 32, 32)
    assert np.all(tm[:, :3] == 2) and np.all(tm[:, 3] == 1)
    # One allowed key per row at a known place.
    A = np.zeros((64, 64), bool)
    A[np.arange(64), (np.arange(64) * 7) % 64] = True
    tm = tilemap.tile_map(A, 16, 16)
    for a in range(4):
        hit = {((i * 7) % 64) // 16 for i in range(a * 16, a * 16 + 16)}
        for t in range(4):
            assert tm[a, t] == (1 if t in hit else 0)
