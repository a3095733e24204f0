"""Rectangular problems on the device: n query rows against nk key rows.

The maitreyasuin page's tiled forward takes Tq query rows against Tk key
rows; a causal offset (key j allowed for query i iff j <= i + offset) gives
the bottom-right-aligned mask of queries appended after a cache of keys
(offset nk - n) and the mask of one key shard of a sequence (offset = query
start - key start).  Checked against the float64 oracle:

* O, L, dQ, dK, dV for none / causal-with-offset / bitmask masks, both dQ
  paths, with rows that allow no key giving O = 0, L = -inf and dQ = 0;
* the kernels' tile classification, bit for bit;
* short query blocks against long key ranges, where the forward splits the
  key range over several workgroups and merges their partial results;
* the one-GPU share of sequence sharding: results over disjoint key ranges
  merge exactly into the full result (L = ln sum_s e^{L_s},
  O = sum_s e^{L_s - L} O_s), and per-range gradients taken with the full
  O and L add up (dQ) or concatenate (dK, dV) to the full gradients.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import dense, tiled, tilemap
from tests.gpu_common import (DEV, allowance_full, compare, one_key_rows, output_rounding_bound, stored,
                              zero_key_rows)

pytestmark = pytest.mark.gpu

DIMS = [("f32", 64, 64), ("f32", 80, 80), ("bf16", 128, 128), ("bf16", 64, 128), ("bf16", 64, 64)]
# (n, nk, mask, offset)
SHAPES = [(300, 777, "causal", 477), (300, 777, "causal", 0), (300, 777, "none", 0),
          (777, 300, "causal", -477), (777, 300, "causal", 50), (777, 300, "bitmask", 0),
          (1, 513, "causal", 512), (129, 1, "none", 0), (200, 333, "causal", -150),
          # Key tiles whose first allowing row k0 - offset lies past the last row
          # but inside the last query tile: no row reaches them (dK = dV = 0).
          (400, 400, "causal", -144), (1, 255, "causal", 111), (777, 777, "causal", -190)]


def _dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(W.bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV)


def _inputs(H, n, nk, d, v, dtype, seed):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((1, H, n, d), dtype=np.float32)
    K = rng.standard_normal((1, H, nk, d), dtype=np.float32)
    V = rng.standard_normal((1, H, nk, v), dtype=np.float32)
    G = rng.standard_normal((1, H, n, v), dtype=np.float32)
    if dtype == "bf16":
        Q, K, V, G = (W.round_bf16(x) for x in (Q, K, V, G))
    return Q, K, V, G, rng


def _allowed(mask, n, nk, off, H, rng):
    if mask == "none":
        return [np.ones((n, nk), bool)] * H, None
    if mask == "causal":
        return [W.causal_allowed(n, nk=nk, offset=off)] * H, None
    A = (rng.random((H, n, nk)) < 0.3) | W.causal_allowed(n, nk=nk, offset=nk - n)[None]
    A[:, 5] = False  # a row with no allowed key
    return list(A), torch.from_numpy(W.pack_bits(A).view(np.int32)).to(DEV)


def _oracle(Q, K, V, G, c, A, dtype):
    """O, L, dQ over every row (zero / -inf where a row allows no key), dK, dV,
    the rows with an allowed key, and the bf16 operand rounding allowances
    (O, dQ of those rows; dK, dV of every key)."""
    n, v = Q.shape[0], V.shape[1]
    rows = np.nonzero(A.any(axis=1))[0]
    O, L, dQ = np.zeros((n, v)), np.full(n, -np.inf), np.zeros_like(Q, dtype=np.float64)
    dK, dV = np.zeros_like(K, dtype=np.float64), np.zeros_like(V, dtype=np.float64)
    al = {}
    if rows.size:
        Y, m, ell, Lr = dense.forward(Q[rows], K, V, c, A[rows])
        O[rows], L[rows] = Y, Lr
        dq, dK, dV = tiled.reverse(Q[rows], K, V, c, A[rows], K.shape[0], stored(Y, dtype), m, ell, G[rows])
        dQ[rows] = dq
        al = allowance_full(Q[rows], K, V, G[rows], c, A[rows], stored(Y, dtype), Lr, dtype)
    return O, L, dQ, dK, dV, rows, al


def _bounds(Q, K, V, G, c, nq, nk):
    mq, mk, mv, mg = (float(np.abs(x).max(initial=0.0)) for x in (Q, K, V, G))
    v = V.shape[1]
    return {"O": mv, "dV": mg * nq, "dQ": 2 * abs(c) * mk * mg * mv * v, "dK": 2 * abs(c) * mq * mg * mv * v * nq}


@pytest.mark.parametrize("n,nk,mask,off", SHAPES)
@pytest.mark.parametrize("dtype,d,v", DIMS)
def test_rectangular_parity(dtype, d, v, n, nk, mask, off):
    import exact_tiled_attention_attn_amd as E

    H, c = 2, 1.0 / np.sqrt(d)
    Q, K, V, G, rng = _inputs(H, n, nk, d, v, dtype, seed=n * 7 + nk + d)
    As, mdev = _allowed(mask, n, nk, off, H, rng)
    q, k, val, g = (_dev(x, dtype) for x in (Q, K, V, G))
    o, L = E.fwd(q, k, val, c, mask, mdev, causal_offset=off)
    res = {"": E.bwd(q, k, val, o, g, L, c, mask, mdev, deterministic=False, causal_offset=off),
           "det": E.bwd(q, k, val, o, g, L, c, mask, mdev, deterministic=True, causal_offset=off)}
    torch.cuda.synchronize()
    got = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    for h in range(H):
        Qh, Kh, Vh, Gh = (x[0, h].astype(np.float64) for x in (Q, K, V, G))
        rO, rL, rdQ, rdK, rdV, rows, al = _oracle(Qh, Kh, Vh, Gh, c, As[h], dtype)
        tag = (dtype, d, v, n, nk, mask, off, h)
        empty = np.setdiff1d(np.arange(n), rows)
        Oh, Lh = got(o[0, h]), got(L[0, h])
        assert np.all(Oh[empty] == 0) and np.all(Lh[empty] == -np.inf), tag
        if rows.size == 0:
            continue
        bd = _bounds(Qh, Kh, Vh, Gh, c, rows.size, nk)
        compare("O", Oh[rows], rO[rows], dtype, tag, bound=bd["O"], extra=al.get("O"))
        compare("L", Lh, rL, dtype, tag)
        for path, (dq, dk, dv) in res.items():
            dqh = got(dq[0, h])
            assert np.all(dqh[empty] == 0), (tag, path)
            compare("dQ", dqh[rows], rdQ[rows], dtype, (tag, path), bound=bd["dQ"], extra=al.get("dQ"),
                    zero_rows=one_key_rows(As[h][rows]))
            compare("dK", got(dk[0, h]), rdK, dtype, (tag, path), bound=bd["dK"], extra=al.get("dK"),
                    zero_rows=zero_key_rows(As[h][rows]))
            compare("dV", got(dv[0, h]), rdV, dtype, (tag, path), bound=bd["dV"], extra=al.get("dV"))


@pytest.mark.parametrize("is_bwd", [0, 1, 2])
@pytest.mark.parametrize("n,nk,off", [(300, 777, 477), (777, 300, -477), (777, 300, 50), (200, 333, -150)])
def test_rectangular_tile_map(n, nk, off, is_bwd):
    import exact_tiled_attention_attn_amd as E

    q = torch.empty((1, 1, n, 128), dtype=torch.bfloat16, device=DEV)
    k = torch.empty((1, 1, nk, 128), dtype=torch.bfloat16, device=DEV)
    got, bq, bk = E.debug_tile_map(q, k, k, 0.1, "causal", None, is_bwd, causal_offset=off)
    torch.cuda.synchronize()
    want = tilemap.tile_map(W.causal_allowed(n, nk=nk, offset=off), bq, bk)
    assert np.array_equal(got[0].cpu().numpy(), want), (n, nk, off, is_bwd, bq, bk)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
@pytest.mark.parametrize("splits", [[0, 384, 1000], [0, 1, 700, 999, 1000]])
def test_key_ranges_merge_into_the_full_result(dtype, d, splits):
    import exact_tiled_attention_attn_amd as E

    H, n, c = 2, 1000, 1.0 / np.sqrt(d)
    Q, K, V, G, _ = _inputs(H, n, n, d, d, dtype, seed=len(splits))
    q, k, val, g = (_dev(x, dtype) for x in (Q, K, V, G))
    o, L = E.fwd(q, k, val, c, "causal")
    dQf, dKf, dVf = E.bwd(q, k, val, o, g, L, c, "causal", deterministic=True)
    parts, dQ, dKs, dVs = [], torch.zeros_like(q, dtype=torch.float32), [], []
    for k0, k1 in zip(splits, splits[1:]):
        ks, vs = k[:, :, k0:k1].contiguous(), val[:, :, k0:k1].contiguous()
        parts.append(E.fwd(q, ks, vs, c, "causal", causal_offset=-k0))
        # Gradients of this key range with the full O and L.
        dq, dk, dv = E.bwd(q, ks, vs, o, g, L, c, "causal", deterministic=True, causal_offset=-k0)
        dQ += dq.float()
        dKs.append(dk)
        dVs.append(dv)
    Ls = torch.stack([p[1] for p in parts])
    Lm = torch.logsumexp(Ls, dim=0)
    Om = sum(torch.exp(Ls[s] - Lm)[..., None] * parts[s][0].float() for s in range(len(parts)))
    dK, dV = torch.cat(dKs, dim=2), torch.cat(dVs, dim=2)
    torch.cuda.synchronize()
    A = W.causal_allowed(n)
    got = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    for h in range(H):
        Qh, Kh, Vh, Gh = (x[0, h].astype(np.float64) for x in (Q, K, V, G))
        rO, rL, rdQ, rdK, rdV, _, al = _oracle(Qh, Kh, Vh, Gh, c, A, dtype)
        tag = (dtype, splits, h)
        # The merged output carries the rounding of each range's output too.
        compare("O", got(Om[0, h]), rO, dtype, tag, extra=None if "O" not in al else 2 * al["O"])
        compare("L", got(Lm[0, h]), rL, dtype, tag)
        compare("dQ", got(dQ[0, h]), rdQ, dtype, tag, extra=al.get("dQ"))
        compare("dK", got(dK[0, h]), rdK, dtype, tag, extra=al.get("dK"))
        compare("dV", got(dV[0, h]), rdV, dtype, tag, extra=al.get("dV"))
        # The same rows from the single square call: agreement at rounding level.
        assert np.abs(got(Om[0, h]) - got(o[0, h])).max() <= (1e-5 if dtype == "f32" else 1e-2) * np.abs(rO).max()
        assert np.abs(got(Lm[0, h]) - got(L[0, h])).max() <= 1e-4
        for x, y in ((dQ, dQf), (dK, dKf), (dV, dVf)):
            ref = np.abs(got(y[0, h])).max()
            assert np.abs(got(x[0, h]) - got(y[0, h])).max() <= (1e-5 if dtype == "f32" else 2e-2) * ref


SPLIT_SHAPES = [(100, 8192, "causal", 8092), (1, 4096, "causal", 4095), (128, 16384, "none", 0),
                (64, 5000, "bitmask", 0), (200, 3000, "causal", -100), (129, 2048, "causal", 1919)]


@pytest.mark.parametrize("n,nk,mask,off", SPLIT_SHAPES)
@pytest.mark.parametrize("d,v", [(128, 128), (64, 128), (64, 64)])
def test_split_key_forward(d, v, n, nk, mask, off):
    """Few query tiles against many key tiles: the forward runs key-range splits
    (visible as split workspace) and merges them; O and L against the oracle."""
    import exact_tiled_attention_attn_amd as E

    H, c, dtype = 2, 1.0 / np.sqrt(d), "bf16"
    Q, K, V, G, rng = _inputs(H, n, nk, d, v, dtype, seed=n + nk + d + v)
    As, mdev = _allowed(mask, n, nk, off, H, rng)
    q, k, val = (_dev(x, dtype) for x in (Q, K, V))
    o_like = torch.empty((1, H, n, v), dtype=torch.bfloat16, device=DEV)
    prob = E.make_problem(q, k, val, o_like, c, mask, mdev, causal_offset=off)
    map_bytes = 0 if mask != "bitmask" else -(-H * -(-n // 128) * -(-nk // 64) // 256) * 256
    assert E.workspace_size(prob, False) > map_bytes, "key-range splits expected"
    o, L = E.fwd(q, k, val, c, mask, mdev, causal_offset=off)
    torch.cuda.synchronize()
    got = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    for h in range(H):
        Qh, Kh, Vh, Gh = (x[0, h].astype(np.float64) for x in (Q, K, V, G))
        rO, rL, _, _, _, rows = _oracle_fwd_only(Qh, Kh, Vh, c, As[h])
        tag = (d, v, n, nk, mask, off, h)
        empty = np.setdiff1d(np.arange(n), rows)
        Oh, Lh = got(o[0, h]), got(L[0, h])
        assert np.all(Oh[empty] == 0) and np.all(Lh[empty] == -np.inf), tag
        Arows = As[h][rows]
        orb = output_rounding_bound(Qh[rows], Kh, Vh, rL[rows], c, lambda r: Arows[r], dtype)
        compare("O", Oh[rows], rO[rows], dtype, tag, extra=orb)
        compare("L", Lh, rL, dtype, tag)


@pytest.mark.parametrize("d,v", [(128, 128), (64, 128)])
def test_split_key_forward_growing_scores(d, v):
    """Key-range splits whose scores grow from one 64-key tile to the next by
    far more than the rescale slack: every split raises its reference max
    mid-range (the forward's exact path) before the splits are merged."""
    import exact_tiled_attention_attn_amd as E

    H, n, nk, c, dtype = 2, 100, 4096, 1.0 / np.sqrt(d), "bf16"
    Q, K, V, G, rng = _inputs(H, n, nk, d, v, "f32", seed=d + v + 7)
    K = K * ((1.0 + 4.0 * (np.arange(nk) % 512 // 64)) * (1.0 + np.arange(nk) / nk))[None, None, :, None]
    Q, K, V = (W.round_bf16(x.astype(np.float32)) for x in (Q, K, V))
    q, k, val = (_dev(x, dtype) for x in (Q, K, V))
    o_like = torch.empty((1, H, n, v), dtype=torch.bfloat16, device=DEV)
    assert E.workspace_size(E.make_problem(q, k, val, o_like, c, "none"), False) > 0, "key-range splits expected"
    o, L = E.fwd(q, k, val, c, "none")
    torch.cuda.synchronize()
    got = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    A = np.ones((n, nk), bool)
    for h in range(H):
        Qh, Kh, Vh = (x[0, h].astype(np.float64) for x in (Q, K, V))
        rO, rL, _, _, _, rows = _oracle_fwd_only(Qh, Kh, Vh, c, A)
        orb = output_rounding_bound(Qh, Kh, Vh, rL, c, lambda r: A[r], dtype)
        compare("O", got(o[0, h]), rO, dtype, (d, v, h), extra=orb)
        compare("L", got(L[0, h]), rL, dtype, (d, v, h))


@pytest.mark.parametrize("n,nk,mask,off", SPLIT_SHAPES)
@pytest.mark.parametrize("d,v", [(128, 128), (64, 128), (64, 64)])
def test_split_key_backward(d, v, n, nk, mask, off):
    """The same shapes through the backward: the deterministic dQ kernel
    splits the key range (visible as partial-dQ workspace), the splits are
    added in order (bitwise reproducible); dQ, dK, dV against the oracle on
    both dQ paths."""
    import exact_tiled_attention_attn_amd as E

    H, c, dtype = 2, 1.0 / np.sqrt(d), "bf16"
    Q, K, V, G, rng = _inputs(H, n, nk, d, v, dtype, seed=n + nk + d + v + 1)
    As, mdev = _allowed(mask, n, nk, off, H, rng)
    q, k, val, g = (_dev(x, dtype) for x in (Q, K, V, G))
    o, L = E.fwd(q, k, val, c, mask, mdev, causal_offset=off)
    pb = E.make_problem(q, k, val, o, c, mask, mdev, True, off)
    npad = -(-n // 128) * 128
    assert E.workspace_size(pb, True) >= 2 * 4 * H * npad + 2 * 4 * H * n * d, "dQ key-range splits expected"
    det = E.bwd(q, k, val, o, g, L, c, mask, mdev, deterministic=True, causal_offset=off)
    det2 = E.bwd(q, k, val, o, g, L, c, mask, mdev, deterministic=True, causal_offset=off)
    atom = E.bwd(q, k, val, o, g, L, c, mask, mdev, deterministic=False, causal_offset=off)
    torch.cuda.synchronize()
    for x, y in zip(det, det2):
        assert torch.equal(x, y)
    got = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    for h in range(H):
        Qh, Kh, Vh, Gh = (x[0, h].astype(np.float64) for x in (Q, K, V, G))
        rO, rL, rdQ, rdK, rdV, rows, al = _oracle(Qh, Kh, Vh, Gh, c, As[h], dtype)
        if rows.size == 0:
            continue
        bd = _bounds(Qh, Kh, Vh, Gh, c, rows.size, nk)
        empty = np.setdiff1d(np.arange(n), rows)
        for path, (dq, dk, dv) in (("det", det), ("atomic", atom)):
            tag = (d, v, n, nk, mask, off, h, path)
            dqh = got(dq[0, h])
            assert np.all(dqh[empty] == 0), tag
            compare("dQ", dqh[rows], rdQ[rows], dtype, tag, bound=bd["dQ"], extra=al.get("dQ"),
                    zero_rows=one_key_rows(As[h][rows]))
            compare("dK", got(dk[0, h]), rdK, dtype, tag, bound=bd["dK"], extra=al.get("dK"),
                    zero_rows=zero_key_rows(As[h][rows]))
            compare("dV", got(dv[0, h]), rdV, dtype, tag, bound=bd["dV"], extra=al.get("dV"))


def _oracle_fwd_only(Q, K, V, c, A):
    n, v = Q.shape[0], V.shape[1]
    rows = np.nonzero(A.any(axis=1))[0]
    O, L = np.zeros((n, v)), np.full(n, -np.inf)
    if rows.size:
        Y, _, _, Lr = dense.forward(Q[rows], K, V, c, A[rows])
        O[rows], L[rows] = Y, Lr
    return O, L, None, None, None, rows
