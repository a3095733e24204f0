"""Pins of the dropout oracle (oracle/dropout.py).

* The generator against the published known-answer vectors of
  Philox4x32-10 (the Random123 distribution's test vectors for the SC 2011
  generator family).
* Keep frequencies and byte uniformity of the 8-bit draws.
* The 4 x 4 block layout: a pair's decision does not depend on the problem
  shape (a smaller mask is the corner of a larger one) and differs across
  units and seeds.
* p8 = 0 reduces to attention without dropout (dense oracle).
* Central finite differences of the dropout forward (mask held fixed) for
  the VJP, under each mask mode.
* Unbiasedness: the mean over seeds of the dropout output tends to the
  undropped output.
"""

from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from oracle import dense, dropout

KAT = [  # (counter words, key words) -> output words
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,want", KAT)
def test_philox_known_answers(ctr, key, want):
    got = dropout.philox4x32_10(*[np.array([c]) for c in ctr], *key)
    assert tuple(int(x[0]) for x in got) == want


def test_draw_statistics():
    n = 512
    for p8 in (26, 128, 255):
        Z = dropout.keep_mask(seed=12345, unit=3, n=n, nk=n, p8=p8)
        keep = 1 - p8 / 256
        sd = np.sqrt(keep * (1 - keep) / Z.size)
        assert abs(Z.mean() - keep) < 6 * sd, (p8, Z.mean())
    # The 8-bit draws themselves: chi-square over 256 bins.
    i, j = np.arange(256)[:, None], np.arange(256)[None, :]
    words = dropout.philox4x32_10(j // 4, i // 4, np.full((256, 256), 7), 0, 99, 0)
    w = np.select([i % 4 == 0, i % 4 == 1, i % 4 == 2], words[:3], words[3])
    b = ((w >> (8 * (j % 4)).astype(np.uint32)) & 0xFF).ravel()
    counts = np.bincount(b, minlength=256)
    chi2 = ((counts - b.size / 256) ** 2 / (b.size / 256)).sum()
    assert chi2 < 255 + 6 * np.sqrt(2 * 255), chi2


def test_block_layout_is_shape_independent_and_keyed():
    big = dropout.keep_mask(seed=5, unit=1, n=70, nk=90, p8=100)
    small = dropout.keep_mask(seed=5, unit=1, n=33, nk=17, p8=100)
    assert np.array_equal(small, big[:33, :17])
    other_unit = dropout.keep_mask(seed=5, unit=2, n=70, nk=90, p8=100)
    other_seed = dropout.keep_mask(seed=6, unit=1, n=70, nk=90, p8=100)
    high_seed = dropout.keep_mask(seed=5 + (1 << 32), unit=1, n=70, nk=90, p8=100)
    for m in (other_unit, other_seed, high_seed):
        agree = (m == big).mean()
        assert 0.5 < agree < 0.75, agree  # independent masks agree with prob k^2 + (1-k)^2 ~ 0.6


def test_p8_rounding():
    assert dropout.p8_of(0.0) == 0 and dropout.p8_of(0.1) == 26 and dropout.p8_of(0.5) == 128
    assert dropout.p8_of(1 / 512) == 1 and dropout.p8_of(0.999) == 255
    with pytest.raises(ValueError):
        dropout.p8_of(1.0)


def _masks(n, nk, rng):
    return {"none": None, "causal": W.causal_allowed(n, nk=nk, offset=nk - n),
            "bitmask": (rng.random((n, nk)) < 0.5) | W.causal_allowed(n, nk=nk, offset=nk - n)}


def test_no_dropout_is_attention():
    rng = np.random.default_rng(1)
    n, nk, d, v = 9, 13, 4, 3
    Q, K, V, G = rng.normal(size=(n, d)), rng.normal(size=(nk, d)), rng.normal(size=(nk, v)), rng.normal(size=(n, v))
    Z = dropout.keep_mask(1, 0, n, nk, 0)
    assert Z.all()
    for name, A in _masks(n, nk, rng).items():
        Y, L = dropout.forward(Q, K, V, 0.6, A, Z, 0)
        Yr, _, _, Lr = dense.forward(Q, K, V, 0.6, A)
        assert np.abs(Y - Yr).max() < 1e-13 and np.abs(L - Lr).max() < 1e-13, name
        for x, r in zip(dropout.vjp(Q, K, V, 0.6, A, Z, 0, G), dense.vjp(Q, K, V, 0.6, A, G)):
            assert np.abs(x - r).max() < 1e-13, name


@pytest.mark.parametrize("mask", ["none", "causal", "bitmask"])
def test_dropout_vjp_finite_differences(mask):
    rng = np.random.default_rng(2)
    n, nk, d, v, c, p8 = 5, 7, 3, 2, 0.8, 77
    Q, K, V, G = rng.normal(size=(n, d)), rng.normal(size=(nk, d)), rng.normal(size=(nk, v)), rng.normal(size=(n, v))
    A = _masks(n, nk, rng)[mask]
    Z = dropout.keep_mask(31, 4, n, nk, p8)
    assert 0 < Z.mean() < 1
    grads = dropout.vjp(Q, K, V, c, A, Z, p8, G)
    h = 1e-6
    for which, dX in enumerate(grads):
        X = (Q, K, V)[which]
        ref = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            args_p, args_m = [Q.copy(), K.copy(), V.copy()], [Q.copy(), K.copy(), V.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            fp = (G * dropout.forward(*args_p, c, A, Z, p8)[0]).sum()
            fm = (G * dropout.forward(*args_m, c, A, Z, p8)[0]).sum()
            ref[idx] = (fp - fm) / (2 * h)
        assert np.abs(dX - ref).max() <= 1e-7 * max(1.0, np.abs(ref).max()), (mask, which)


def test_dropout_is_unbiased():
    rng = np.random.default_rng(3)
    n, nk, d, v, p8 = 4, 6, 3, 2, 64
    Q, K, V = rng.normal(size=(n, d)), rng.normal(size=(nk, d)), rng.normal(size=(nk, v))
    Y0, _, _, _ = dense.forward(Q, K, V, 1.0, None)
    ys = np.stack([dropout.forward(Q, K, V, 1.0, None, dropout.keep_mask(s, 0, n, nk, p8), p8)[0]
                   for s in range(3000)])
    se = ys.std(axis=0) / np.sqrt(len(ys))
    assert np.all(np.abs(ys.mean(axis=0) - Y0) < 6 * se + 1e-12)


@pytest.mark.parametrize("mask", ["none", "causal", "bitmask"])
def test_dropout_vjp_row_term_from_a_forward_output(mask):
    """D_i = sum_j P_ij dPd_ij = <G_i, Y_i>: given the forward's own output,
    the Y form equals the default; given a perturbed output (as a bf16 run
    stores it), it equals the reverse procedure of oracle/tiled.py fed the
    same output (p = 0, where both apply)."""
    from oracle import tiled

    rng = np.random.default_rng(5)
    n, nk, d, v, c = 6, 9, 4, 3, 0.7
    Q, K, V, G = rng.normal(size=(n, d)), rng.normal(size=(nk, d)), rng.normal(size=(nk, v)), rng.normal(size=(n, v))
    A = _masks(n, nk, rng)[mask]
    Z = dropout.keep_mask(8, 2, n, nk, 51)
    Y, _ = dropout.forward(Q, K, V, c, A, Z, 51)
    for x, r in zip(dropout.vjp(Q, K, V, c, A, Z, 51, G, Y), dropout.vjp(Q, K, V, c, A, Z, 51, G)):
        assert np.abs(x - r).max() <= 1e-12 * max(1.0, np.abs(r).max()), mask
    ones = dropout.keep_mask(8, 2, n, nk, 0)
    Y0, m, ell, _ = dense.forward(Q, K, V, c, A)
    Yp = Y0 * (1 + 1e-3 * rng.normal(size=Y0.shape))  # an output off by rounding-sized amounts
    for x, r in zip(dropout.vjp(Q, K, V, c, A, ones, 0, G, Yp), tiled.reverse(Q, K, V, c, A, nk, Yp, m, ell, G)):
        assert np.abs(x - r).max() <= 1e-12 * max(1.0, np.abs(r).max()), mask


@pytest.mark.parametrize("n,nk", [(37, 53), (64, 96), (130, 70)])
def test_keep_mask_at_index_sets(n, nk):
    """The block-wise draw at arbitrary row and column sets (unsorted,
    repeated blocks) gives keep_mask's decisions."""
    rng = np.random.default_rng(n + nk)
    for p8 in (1, 26, 128, 255):
        Z = dropout.keep_mask(987654321987, 5, n, nk, p8)
        r = rng.choice(n, 11, replace=False)
        c = rng.choice(nk, 13, replace=False)
        assert np.array_equal(dropout.keep_mask_at(987654321987, 5, r, c, p8), Z[r][:, c])
    assert np.array_equal(dropout.keep_mask_at(3, 1, np.arange(n), np.arange(nk), 77),
                          dropout.keep_mask(3, 1, n, nk, 77))


@pytest.mark.parametrize("mask", ["none", "causal", "random"])
def test_sampled_dropout_outputs_and_gradients(mask):
    """output_rows and grads_sampled, one row or column at a time, equal the
    whole-matrix forward and VJP (both taking D from the same Y)."""
    rng = np.random.default_rng(11)
    n, nk, d, v, p8, c = 41, 57, 8, 6, 40, 0.3
    Q, K, V, G = (rng.standard_normal(s) for s in ((n, d), (nk, d), (nk, v), (n, v)))
    A = None
    if mask == "causal":
        A = W.causal_allowed(n, nk=nk, offset=nk - n)
    elif mask == "random":
        A = rng.random((n, nk)) < 0.4
        A[np.arange(n), rng.integers(0, nk, n)] = True
    Z = dropout.keep_mask(42, 2, n, nk, p8)
    Y, L = dropout.forward(Q, K, V, c, A, Z, p8)
    Ah = np.ones((n, nk), bool) if A is None else A
    rows, cols = np.array([0, 5, 17, 40]), np.array([1, 2, 30, 56])
    Yr = dropout.output_rows(Q, K, V, c, lambda r: Ah[r], L, lambda r: Z[r], p8, rows)
    assert np.allclose(Yr, Y[rows], rtol=1e-12, atol=1e-14)
    Yd = Y + 1e-3 * rng.standard_normal(Y.shape)  # any output the reverse pass is handed
    dQ, dK, dV = dropout.vjp(Q, K, V, c, A, Z, p8, G, Yd)
    sQ, sK, sV = dropout.grads_sampled(Q, K, V, c, lambda r: Ah[r], G, L, Yd, rows, cols, Z[rows], Z[:, cols], p8)
    assert np.allclose(sQ, dQ[rows], rtol=1e-10, atol=1e-13)
    assert np.allclose(sK, dK[cols], rtol=1e-10, atol=1e-13)
    assert np.allclose(sV, dV[cols], rtol=1e-10, atol=1e-13)
