"""Seeded sweeps over combinations of the options, against the float64 oracle.

Each case draws (dtype and dims, n, nk, mask, causal offset, dropout,
scale) from a fixed seed, so the list is the same on every run.  The case
runs attn_fwd and both attn_bwd paths and compares O, L, dQ, dK and dV with
the oracle: the definition (oracle/dense.py), or with dropout the dropout
oracle (oracle/dropout.py) under its own mask.  Rows that allow no key must
give O = 0, L = -inf and dQ = 0.  The point is the interplay of options that
the focused tests cover one at a time.

``test_sweep`` holds every output to the stated tolerances relative to its
largest magnitude.  ``test_sweep_wide`` draws from wider distributions (n
off the tile grid, offsets near +-n, a handful of rows against thousands of
keys, dropout up to 0.9), where many gradients are small differences of
large terms: a row dominated by one key has dP_ij close to D_i, and a
single row's dQ is a sum of such differences.  No fp32 evaluation reaches
1e-5 of such a result (a plain fp32 evaluation of the same formulas misses
it too), so the wide sweep measures each output's error against the size
of the terms it sums: T(dV_j) = sum_i P~_ij |dO_i|, T(dQ_i) = |c| sum_j
P_ij (|Z_ij dP_ij / (1-p)| + sum_v |dO_iv O_iv|) |K_j| (dK alike with
|Q_i|), T(O_i) = sum_j P~_ij |V_j|, P~ the dropped and rescaled weights.
D_i = <dO_i, O_i> enters with the size of its own terms: the device forms
it from O as stored, which may differ from the reference's rounding of the
exact output by one bf16 ulp per element.  Wrong masking, a
missed or doubled tile, or a wrong row statistic moves an output by a
multiple of its terms and fails this bound as surely as the strict one.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import dense, dropout, tiled
from tests.gpu_common import (BF16_ABS, BF16_REL, DEV, F32_REL, allowance_full, compare, one_key_rows, stored,
                              zero_key_rows)

pytestmark = pytest.mark.gpu

DIMS = [("f32", 64, 64), ("f32", 80, 80), ("f32", 128, 128), ("f32", 64, 128),
        ("bf16", 64, 64), ("bf16", 80, 80), ("bf16", 128, 128), ("bf16", 64, 128)]


def _cases(count=40, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        dtype, d, v = DIMS[rng.integers(len(DIMS))]
        n = int(rng.choice([1, 3, 31, 64, 65, 127, 200, 333, 513, 700]))
        nk = n if rng.random() < 0.4 else int(rng.choice([1, 5, 64, 129, 300, 640, 1500]))
        mask = ["none", "causal", "bitmask"][rng.integers(3)]
        off = int(rng.integers(-n, nk + 1)) if mask == "causal" else 0
        p = float(rng.choice([0.0, 0.0, 0.15, 0.5]))
        scale = float(rng.choice([1 / np.sqrt(d), 0.3, -0.2, 0.0]))
        out.append(pytest.param(i, dtype, d, v, n, nk, mask, off, p, scale,
                                id=f"{i}-{dtype}-{d}x{v}-n{n}-nk{nk}-{mask}{off}-p{p}-c{scale:.3g}"))
    return out


def _wide_cases(count=160, seed=777):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(count):
        i = 5000 + k
        dtype, d, v = DIMS[rng.integers(len(DIMS))]
        n = int(rng.choice([1, 2, 7, 32, 33, 63, 96, 128, 129, 191, 255, 256, 257, 400, 511, 777, 1024, 1100]))
        nk = n if rng.random() < 0.4 else int(rng.choice([1, 2, 31, 32, 63, 127, 128, 255, 256, 257, 1023, 1024, 2049]))
        mask = ["none", "causal", "bitmask"][rng.integers(3)]
        off = int(rng.integers(-n - 2, nk + 3)) if mask == "causal" else 0
        p = float(rng.choice([0.0, 0.0, 0.1, 0.5, 0.9]))
        scale = float(rng.choice([1 / np.sqrt(d), 0.3, -0.2, 0.0, -0.5]))
        out.append(pytest.param(i, dtype, d, v, n, nk, mask, off, p, scale,
                                id=f"{i}-{dtype}-{d}x{v}-n{n}-nk{nk}-{mask}{off}-p{p}-c{scale:.3g}"))
    return out


def _dev(x, dtype):
    if dtype == "bf16":
        return torch.from_numpy(W.bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV)


def _run(i, dtype, d, v, n, nk, mask, off, p, scale, wide):
    import exact_tiled_attention_attn_amd as E

    H, seed = 2, 1000 + i
    rng = np.random.default_rng(i)
    Q = rng.standard_normal((1, H, n, d), dtype=np.float32)
    K = rng.standard_normal((1, H, nk, d), dtype=np.float32)
    V = rng.standard_normal((1, H, nk, v), dtype=np.float32)
    G = rng.standard_normal((1, H, n, v), dtype=np.float32)
    if dtype == "bf16":
        Q, K, V, G = (W.round_bf16(x) for x in (Q, K, V, G))
    if mask == "none":
        As, mdev = [None] * H, None
    elif mask == "causal":
        As, mdev = [W.causal_allowed(n, nk=nk, offset=off)] * H, None
    else:
        A = rng.random((H, n, nk)) < 0.35
        As, mdev = list(A), torch.from_numpy(W.pack_bits(A).view(np.int32)).to(DEV)
    q, k, val, g = (_dev(x, dtype) for x in (Q, K, V, G))
    kw = dict(causal_offset=off, dropout_p=p, dropout_seed=seed)
    o, L = E.fwd(q, k, val, scale, mask, mdev, **kw)
    res = {"atomic": E.bwd(q, k, val, o, g, L, scale, mask, mdev, deterministic=False, **kw),
           "det": E.bwd(q, k, val, o, g, L, scale, mask, mdev, deterministic=True, **kw)}
    torch.cuda.synchronize()
    got = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    p8 = dropout.p8_of(p)
    for h in range(H):
        Qh, Kh, Vh, Gh = (x[0, h].astype(np.float64) for x in (Q, K, V, G))
        A = np.ones((n, nk), bool) if As[h] is None else As[h]
        rows = np.nonzero(A.any(axis=1))[0]
        empty = np.setdiff1d(np.arange(n), rows)
        tag = (i, dtype, d, v, n, nk, mask, off, p, scale, h)
        Oh, Lh = got(o[0, h]), got(L[0, h])
        assert np.all(Oh[empty] == 0) and np.all(Lh[empty] == -np.inf), tag
        for _, (dq, _, _) in res.items():
            assert np.all(got(dq[0, h])[empty] == 0), tag
        if rows.size == 0:
            for _, (_, dk, dv) in res.items():
                assert np.all(got(dk[0, h]) == 0) and np.all(got(dv[0, h]) == 0), tag
            continue
        Qr, Gr, Ar = Qh[rows], Gh[rows], A[rows]
        if p8:
            Z = dropout.keep_mask(seed, h, n, nk, p8)[rows]
            Y, Lr = dropout.forward(Qr, Kh, Vh, scale, Ar, Z, p8)
            rdQ, rdK, rdV = dropout.vjp(Qr, Kh, Vh, scale, Ar, Z, p8, Gr, stored(Y, dtype))
        else:
            Y, m, ell, Lr = dense.forward(Qr, Kh, Vh, scale, Ar)
            rdQ, rdK, rdV = tiled.reverse(Qr, Kh, Vh, scale, Ar, nk, stored(Y, dtype), m, ell, Gr)
        if wide:
            _check_terms(Oh[rows], Lh[rows], res, h, rows, (Qr, Kh, Vh, Gr, Ar), Y, Lr, (rdQ, rdK, rdV),
                         Z if p8 else None, p8, scale, dtype, tag, got)
            continue
        # Magnitude bounds for outputs whose exact value is zero (keys no row allows).
        mq, mk, mv, mg = (float(np.abs(x).max(initial=0.0)) for x in (Qr, Kh, Vh, Gr))
        kinv = 256 / (256 - p8)
        bd = {"dQ": 2 * abs(scale) * mk * mg * mv * v * kinv + 1e-30,
              "dK": 2 * abs(scale) * mq * mg * mv * v * rows.size * kinv + 1e-30,
              "dV": mg * rows.size * kinv + 1e-30}
        few = int(Ar.sum(axis=1).max()) <= 2
        if few:
            # Every row has one or two keys: dQ and dK are differences of two
            # terms p_ij (dP_ij - D_i), so they are held to the size of those
            # terms (the wide sweep's bound) rather than to their own maximum.
            _check_terms(Oh[rows], Lh[rows], res, h, rows, (Qr, Kh, Vh, Gr, Ar), Y, Lr, (rdQ, rdK, rdV),
                         Z if p8 else None, p8, scale, dtype, tag, got)
            continue
        al = allowance_full(Qr, Kh, Vh, Gr, scale, Ar, stored(Y, dtype), Lr, dtype, Z if p8 else None, p8)
        compare("O", Oh[rows], Y, dtype, tag, extra=al.get("O"))
        compare("L", Lh[rows], Lr, dtype, tag)
        for path, (dq, dk, dv) in res.items():
            for name, x, r in (("dQ", got(dq[0, h])[rows], rdQ), ("dK", got(dk[0, h]), rdK), ("dV", got(dv[0, h]), rdV)):
                compare(name, x, r, dtype, (tag, path), bound=bd[name], extra=al.get(name),
                        zero_rows=one_key_rows(Ar) if name == "dQ" else zero_key_rows(Ar) if name == "dK" else None)


def _check_terms(Oh, Lh, res, h, rows, ins, Y, Lr, grads, Z, p8, scale, dtype, tag, got):
    """Errors against the size of the summed terms (see the module docstring)."""
    Qr, Kh, Vh, Gr, Ar = ins
    P = np.where(Ar, np.exp(scale * (Qr @ Kh.T) - Lr[:, None]), 0.0)
    Zs = np.ones_like(P) if Z is None else Z * (256 / (256 - p8))  # dropped and rescaled: Z / (1 - p)
    Pt = P * Zs
    Dt = np.sum(np.abs(Gr) * np.abs(Y), axis=1)  # size of the terms of D_i = <dO_i, O_i>
    Wm = P * (np.abs(Zs * (Gr @ Vh.T)) + Dt[:, None])
    T = {"O": Pt @ np.abs(Vh), "dQ": abs(scale) * Wm @ np.abs(Kh), "dK": abs(scale) * Wm.T @ np.abs(Qr),
         "dV": Pt.T @ np.abs(Gr)}
    compare("L", Lh, Lr, dtype, tag)
    tol = F32_REL if dtype == "f32" else BF16_REL
    outs = [("O", "", Oh, Y)]
    for path, (dq, dk, dv) in res.items():
        outs += [("dQ", path, got(dq[0, h])[rows], grads[0]), ("dK", path, got(dk[0, h]), grads[1]),
                 ("dV", path, got(dv[0, h]), grads[2])]
    for name, path, x, r in outs:
        t = T[name]
        scale_t = max(float(t.max(initial=0.0)), 1e-30)
        err = np.abs(x - r)
        assert np.all(np.isfinite(x)), (tag, path, name, "non-finite output")
        e = float(err.max(initial=0.0)) / scale_t
        assert e <= tol, (tag, path, name, e)
        if dtype == "bf16":
            bad = err > BF16_ABS * scale_t + BF16_REL * t
            assert not bad.any(), (tag, path, name, int(bad.sum()))


@pytest.mark.parametrize("i,dtype,d,v,n,nk,mask,off,p,scale", _cases())
def test_sweep(i, dtype, d, v, n, nk, mask, off, p, scale):
    _run(i, dtype, d, v, n, nk, mask, off, p, scale, wide=False)


@pytest.mark.parametrize("i,dtype,d,v,n,nk,mask,off,p,scale", _wide_cases())
def test_sweep_wide(i, dtype, d, v, n, nk, mask, off, p, scale):
    _run(i, dtype, d, v, n, nk, mask, off, p, scale, wide=True)
