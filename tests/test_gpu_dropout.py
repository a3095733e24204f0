"""Dropout on the device against the float64 oracle (oracle/dropout.py).

The reverse pass must replay the forward's realised mask (alphabetamath
page, reverse procedure): the kernels regenerate each keep decision from
(seed, unit, i, j) with Philox4x32-10, so the checks are

* the kernels' keep decisions equal the oracle's, bit for bit;
* O, L and dQ, dK, dV (both dQ paths) equal the oracle's dropout forward
  and VJP taken with the oracle's own mask, within the dtype tolerance;
* the same seed gives bitwise the same results, another seed other ones;
* with few query rows against many keys the forward's and the dQ
  kernel's key-range splits carry the mask too;
* the autograd wrapper passes the dropout through to the backward.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import dropout
from tests.gpu_common import DEV, allowance_full, compare, stored

pytestmark = pytest.mark.gpu


def _dev(x, dtype):
    if dtype == "bf16":
        return torch.from_numpy(W.bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV)


@pytest.mark.parametrize("seed,p,unit_bh,i0,j0,rows,cols", [
    (0, 0.1, (0, 0), 0, 0, 64, 96), (12345678901234, 0.5, (1, 2), 120, 44, 37, 53),
    ((1 << 64) - 1, 0.9, (0, 1), 4, 1000, 8, 5)])
def test_keep_decisions_match_the_oracle(seed, p, unit_bh, i0, j0, rows, cols):
    import exact_tiled_attention_attn_amd as E

    B, H = 2, 3
    q = torch.empty((B, H, 2048, 64), dtype=torch.bfloat16, device=DEV)
    got = E.dropout_mask(q, q, q, p, seed, unit_bh[0], unit_bh[1], i0, j0, rows, cols)
    torch.cuda.synchronize()
    p8 = dropout.p8_of(p)
    full = dropout.keep_mask(seed, unit_bh[0] * H + unit_bh[1], i0 + rows, j0 + cols, p8)
    assert np.array_equal(got.cpu().numpy().astype(bool), full[i0:, j0:])


DIMS = [("f32", 64, 64), ("f32", 80, 80), ("bf16", 128, 128), ("bf16", 64, 128), ("bf16", 64, 64)]


@pytest.mark.parametrize("mask", ["none", "causal", "bitmask"])
@pytest.mark.parametrize("dtype,d,v", DIMS)
def test_dropout_parity(dtype, d, v, mask):
    import exact_tiled_attention_attn_amd as E

    B, H, n, nk, p, seed = 1, 2, 333, 333, 0.2, 2024
    rng = np.random.default_rng(d + v + len(mask))
    Q = rng.standard_normal((B, H, n, d), dtype=np.float32)
    K = rng.standard_normal((B, H, nk, d), dtype=np.float32)
    V = rng.standard_normal((B, H, nk, v), dtype=np.float32)
    G = rng.standard_normal((B, H, n, v), dtype=np.float32)
    if dtype == "bf16":
        Q, K, V, G = (W.round_bf16(x) for x in (Q, K, V, G))
    A, mdev = None, None
    if mask == "causal":
        A = W.causal_allowed(n)
    elif mask == "bitmask":
        A = (rng.random((n, nk)) < 0.3) | W.causal_allowed(n)
        mdev = torch.from_numpy(W.pack_bits(np.stack([A] * H)).view(np.int32)).to(DEV)  # [H, n, words]
    q, k, val, g = (_dev(x, dtype) for x in (Q, K, V, G))
    c = 1 / np.sqrt(d)
    kw = dict(dropout_p=p, dropout_seed=seed)
    o, L = E.fwd(q, k, val, c, mask, mdev, **kw)
    grads = {"atomic": E.bwd(q, k, val, o, g, L, c, mask, mdev, deterministic=False, **kw),
             "det": E.bwd(q, k, val, o, g, L, c, mask, mdev, deterministic=True, **kw)}
    o2, L2 = E.fwd(q, k, val, c, mask, mdev, **kw)
    o3, _ = E.fwd(q, k, val, c, mask, mdev, dropout_p=p, dropout_seed=seed + 1)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(L, L2)  # the same seed replays the same mask
    assert not torch.equal(o, o3)
    p8 = dropout.p8_of(p)
    got = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    for h in range(H):
        Z = dropout.keep_mask(seed, h, n, nk, p8)
        Qh, Kh, Vh, Gh = (x[0, h].astype(np.float64) for x in (Q, K, V, G))
        Y, Lr = dropout.forward(Qh, Kh, Vh, c, A, Z, p8)
        rdQ, rdK, rdV = dropout.vjp(Qh, Kh, Vh, c, A, Z, p8, Gh, stored(Y, dtype))
        tag = (dtype, d, v, mask, h)
        al = allowance_full(Qh, Kh, Vh, Gh, c, A, stored(Y, dtype), Lr, dtype, Z, p8)
        compare("O", got(o[0, h]), Y, dtype, tag, extra=al.get("O"))
        compare("L", got(L[0, h]), Lr, dtype, tag)
        for path, (dq, dk, dv) in grads.items():
            compare("dQ", got(dq[0, h]), rdQ, dtype, (tag, path), extra=al.get("dQ"))
            compare("dK", got(dk[0, h]), rdK, dtype, (tag, path), extra=al.get("dK"))
            compare("dV", got(dv[0, h]), rdV, dtype, (tag, path), extra=al.get("dV"))


@pytest.mark.parametrize("d,v", [(128, 128), (64, 128)])
@pytest.mark.parametrize("mask", ["none", "causal", "bitmask"])
def test_dropout_with_key_range_splits(d, v, mask):
    """Few query rows against many keys (the forward and the dQ kernel split
    their key range): the mask through the split O and dQ partials and their
    merges, bitwise reproducible, against the oracle."""
    import exact_tiled_attention_attn_amd as E

    H, n, nk, p, seed = 2, 70, 3000, 0.25, 99
    off = nk - n if mask == "causal" else 0
    rng = np.random.default_rng(d + v + nk)
    Q, K, V, G = (W.round_bf16(rng.standard_normal((1, H, r, x), dtype=np.float32))
                  for r, x in ((n, d), (nk, d), (nk, v), (n, v)))
    A, mdev = None, None
    if mask == "causal":
        A = W.causal_allowed(n, nk=nk, offset=off)
    elif mask == "bitmask":  # a quarter of the pairs
        A = rng.random((n, nk)) < 0.25
        mdev = torch.from_numpy(W.pack_bits(np.stack([A] * H)).view(np.int32)).to(DEV)
    q, k, val, g = (_dev(x, "bf16") for x in (Q, K, V, G))
    c = 1 / np.sqrt(d)
    kw = dict(dropout_p=p, dropout_seed=seed, causal_offset=off)
    o, L = E.fwd(q, k, val, c, mask, mdev, **kw)
    pb = E.make_problem(q, k, val, o, c, mask, mdev, True, off, p, seed)
    assert E.workspace_size(pb, True) >= 2 * 4 * H * 128 + 2 * 4 * H * n * d, "dQ key-range splits expected"
    assert E.workspace_size(pb, False) >= 2 * 4 * H * n * (v + 1), "forward key-range splits expected"
    det = E.bwd(q, k, val, o, g, L, c, mask, mdev, deterministic=True, **kw)
    det2 = E.bwd(q, k, val, o, g, L, c, mask, mdev, deterministic=True, **kw)
    torch.cuda.synchronize()
    for x, y in zip(det, det2):
        assert torch.equal(x, y)
    p8 = dropout.p8_of(p)
    got = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    for h in range(H):
        Z = dropout.keep_mask(seed, h, n, nk, p8)
        Qh, Kh, Vh, Gh = (x[0, h].astype(np.float64) for x in (Q, K, V, G))
        Y, Lr = dropout.forward(Qh, Kh, Vh, c, A, Z, p8)
        rdQ, rdK, rdV = dropout.vjp(Qh, Kh, Vh, c, A, Z, p8, Gh, stored(Y, "bf16"))
        al = allowance_full(Qh, Kh, Vh, Gh, c, A, stored(Y, "bf16"), Lr, "bf16", Z, p8)
        tag = (d, v, mask, h)
        compare("O", got(o[0, h]), Y, "bf16", tag, extra=al.get("O"))
        compare("dQ", got(det[0][0, h]), rdQ, "bf16", tag, extra=al.get("dQ"))
        compare("dK", got(det[1][0, h]), rdK, "bf16", tag, extra=al.get("dK"))
        compare("dV", got(det[2][0, h]), rdV, "bf16", tag, extra=al.get("dV"))


def test_autograd_passes_dropout_through():
    import exact_tiled_attention_attn_amd as E

    g0 = torch.Generator().manual_seed(0)
    q, k, val, G = (torch.randn((1, 2, 200, 64), generator=g0).to(torch.bfloat16).to(DEV) for _ in range(4))
    for t in (q, k, val):
        t.requires_grad_(True)
    o = E.attention(q, k, val, 0.125, "causal", dropout_p=0.3, dropout_seed=77)
    o.backward(G)
    ro, rl = E.fwd(q.detach(), k.detach(), val.detach(), 0.125, "causal", dropout_p=0.3, dropout_seed=77)
    dq, dk, dv = E.bwd(q.detach(), k.detach(), val.detach(), ro, G, rl, 0.125, "causal", deterministic=True,
                       dropout_p=0.3, dropout_seed=77)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), ro)
    assert torch.equal(q.grad, dq) and torch.equal(k.grad, dk) and torch.equal(val.grad, dv)


@pytest.mark.parametrize("p", [1 / 256, 0.1, 0.5, 255 / 256])
@pytest.mark.parametrize("d", [128, 64])
def test_pipelined_kernels_keep_decisions_bit_exact(p, d):
    """The pipelined kernels' own keep decisions, read off outputs built to
    expose them, equal the oracle's bit for bit: all scores 0 (Q = 0) and a
    bitmask that allows only a 128-key window KW (keys 1990..2117, across
    three 64-key tiles) to every row, so P = 1/128 on the window, then
      forward: V_j = e_(j - kw)    -> O_i[c] = Z_i,kw+c / (128 keep)
      dK/dV:   dO_i = e_(i - rw) on a 128-row window RW (rows 1003..1130)
                                   -> dV_j[c] = Z_rw+c,j / (128 keep)
      dQ:      K_j = e_(j - kw), V_j = dO_i = e_0, so dP = 1
                                   -> dQ_i[c] = (Z_i,kw+c / keep - D_i) / 128.
    Both units, with the forward's and the dQ kernel's key-range splits."""
    import exact_tiled_attention_attn_amd as E

    H, n, nk, v, seed = 2, 1200, 2200, 128, 0xC0FFEE123456789
    kw, rw = 1990, 1003
    p8 = dropout.p8_of(p)
    keep = (256 - p8) / 256.0
    A = np.zeros((n, nk), bool)
    A[:, kw:kw + 128] = True
    mdev = torch.from_numpy(W.pack_bits(np.stack([A] * H)).view(np.int32)).to(DEV)
    kw_ = dict(dropout_p=p, dropout_seed=seed)
    zeros = lambda *s: np.zeros((1, H) + s, np.float32)  # noqa: E731
    Z = [dropout.keep_mask(seed, h, n, nk, p8) for h in range(H)]

    # Forward: one-hot V rows on the window.
    Q, K, V = zeros(n, d), zeros(nk, d), zeros(nk, v)
    V[0, :, kw + np.arange(128), np.arange(128)] = 1.0
    q, k, val = (_dev(x, "bf16") for x in (Q, K, V))
    o, L = E.fwd(q, k, val, 1.0, "bitmask", mdev, **kw_)
    torch.cuda.synchronize()
    ofl = o.float().cpu().numpy()
    for h in range(H):
        assert np.array_equal(ofl[0, h] != 0, Z[h][:, kw:kw + 128]), ("forward", h)
        assert np.allclose(ofl[0, h][ofl[0, h] != 0], 1 / (128 * keep), rtol=2 ** -8)

    # dK/dV kernel: one-hot dO rows on the row window.
    G = zeros(n, v)
    G[0, :, rw + np.arange(128), np.arange(128)] = 1.0
    g = _dev(G, "bf16")
    _, _, dv = E.bwd(q, k, val, o, g, L, 1.0, "bitmask", mdev, deterministic=True, **kw_)
    torch.cuda.synchronize()
    dvf = dv.float().cpu().numpy()
    for h in range(H):
        assert np.array_equal(dvf[0, h, kw:kw + 128].T != 0, Z[h][rw:rw + 128, kw:kw + 128]), ("dV", h)

    # dQ kernel: one-hot K rows on the window, dP = 1.
    K = zeros(nk, d)
    cols = min(d, 128)
    K[0, :, kw + np.arange(cols), np.arange(cols)] = 1.0
    V, G = zeros(nk, v), zeros(n, v)
    V[..., 0] = 1.0
    G[..., 0] = 1.0
    k, val, g = (_dev(x, "bf16") for x in (K, V, G))
    o, L = E.fwd(q, k, val, 1.0, "bitmask", mdev, **kw_)
    dq, _, _ = E.bwd(q, k, val, o, g, L, 1.0, "bitmask", mdev, deterministic=True, **kw_)
    torch.cuda.synchronize()
    dqf = dq.float().cpu().numpy()
    D = o.float().cpu().numpy()[0, :, :, 0].astype(np.float64)  # D_i = <dO_i, O_i> from O as stored
    for h in range(H):
        mid = (0.5 / keep - D[h])[:, None] / 128  # halfway between the kept and the dropped value
        assert np.array_equal(dqf[0, h][:, :cols] > mid, Z[h][:, kw:kw + cols]), ("dQ", h)


def test_dropout_full_size_headline():
    """The headline workload (1 x 32 heads, n = 16384, d = v = 128, bf16,
    causal) with dropout as `bench.py --dropout 0.1` runs it (seed 1234), in
    that launch configuration: O and L on every row of three heads, dQ on
    sampled rows and dK, dV on sampled key columns of those heads, against
    the oracle's dropout forward and VJP with its own keep mask (drawn
    block-wise: oracle/dropout.py keep_mask_at), D taken on the oracle's
    output both as stored and exact."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    import threadpoolctl

    import exact_tiled_attention_attn_amd as E
    from oracle import dense
    from tests.gpu_common import margins_report, margins_scope, operand_rounding_bound, output_rounding_bound, to_dev

    prob = W.generate("bf16_causal_h32_n16384_d128")
    w = prob.w
    n, p, seed = w.n, 0.1, 1234
    p8 = dropout.p8_of(p)
    heads = (0, 13, 31)
    print("[dropout full size] device run", flush=True)
    q, k, val, g = (to_dev(prob, x) for x in "QKVG")
    kw = dict(dropout_p=p, dropout_seed=seed)
    o, L = E.fwd(q, k, val, w.scale, "causal", None, **kw)
    dq, dk, dv = E.bwd(q, k, val, o, g, L, w.scale, "causal", None, deterministic=True, **kw)
    torch.cuda.synchronize()
    got = {name: {h: t[0, h].float().cpu().numpy() for h in heads}
           for name, t in (("O", o), ("L", L), ("dQ", dq), ("dK", dk), ("dV", dv))}
    del q, k, val, g, o, L, dq, dk, dv
    causal = prob.allowed(0)

    def A_rows(r):
        return causal[r]

    def unit(h):
        errs = {}

        def check(name, gv, rv, extra=None):
            errs[name] = max(errs.get(name, 0.0), compare(name[:2] if name != "L" else "L", gv, rv, "bf16",
                                                          ("dropout full size", h, name), extra=extra))

        Q, K, V, G = (getattr(prob, x)[0, h] for x in "QKVG")
        L = dense.forward(Q, K, V, w.scale, causal)[3]  # the undropped softmax's logsumexp
        Z = dropout.keep_mask_at(seed, h, np.arange(n), np.arange(n), p8)

        def Z_rows(r):
            return Z[r]

        Y = np.concatenate([dropout.output_rows(Q, K, V, w.scale, A_rows, L, Z_rows, p8, np.arange(r0, min(n, r0 + 2048)))
                            for r0 in range(0, n, 2048)])
        E_O = output_rounding_bound(Q, K, V, L, w.scale, A_rows, "bf16", Z_rows=Z_rows, p8=p8)
        check("O", got["O"][h], Y, E_O)
        check("L", got["L"][h], L)
        rng = np.random.default_rng(h)
        rows = np.unique(np.concatenate([np.arange(128), np.arange(n - 128, n), rng.choice(n, 32, replace=False)]))
        cols = np.unique(np.concatenate([np.arange(128), np.arange(n - 128, n), rng.choice(n, 32, replace=False)]))
        Zr, Zc = Z[rows], Z[:, cols]
        Ys = stored(Y, "bf16")
        allow = operand_rounding_bound(Q, K, V, G, Ys, L, E_O, w.scale, A_rows, rows, cols, "bf16", Zr, Zc, p8)
        for ref, Yd in (("stored", Ys), ("exact", Y)):
            rq, rk, rv = dropout.grads_sampled(Q, K, V, w.scale, A_rows, G, L, Yd, rows, cols, Zr, Zc, p8)
            check("dQ/" + ref, got["dQ"][h][rows], rq, allow.get("dQ"))
            check("dK/" + ref, got["dK"][h][cols], rk, allow.get("dK"))
            check("dV/" + ref, got["dV"][h][cols], rv, allow.get("dV"))
        return errs

    workers = max(1, min(len(heads), len(os.sched_getaffinity(0))))
    threads = max(1, min(16, len(os.sched_getaffinity(0))) // workers)
    print(f"[dropout full size] oracle on heads {heads}", flush=True)
    total = {}
    with margins_scope(), threadpoolctl.threadpool_limits(threads, user_api="blas"), ThreadPoolExecutor(workers) as ex:
        for errs in ex.map(unit, heads):
            for k_, v_ in errs.items():
                total[k_] = max(total.get(k_, 0.0), v_)
        print("dropout full size", {k_: f"{v_:.2e}" for k_, v_ in total.items()}, flush=True)
        print(margins_report("dropout full size"), flush=True)
