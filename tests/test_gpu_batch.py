"""Several batches and heads at once, against the float64 oracle per unit.

Every (batch, head) unit u = b H + h is an independent problem.  Checked
here with B = 3, H = 2 and every unit compared:

* per-batch bitmasks ([B, H, n, words], batch stride nonzero), where the
  tile maps and the kernels must pick the mask of (b, h), not of h alone;
* dropout, whose draws are keyed by the unit index b H + h;
* a causal offset with nk != n;
* tensors given as [B, n, H, d] memory viewed as [B, H, n, d] (row stride
  H d), and the contiguous layout.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import dense, dropout, tiled
from tests.gpu_common import DEV, allowance_full, compare, one_key_rows, zero_key_rows, stored

pytestmark = pytest.mark.gpu

DIMS = [("f32", 64, 64), ("bf16", 128, 128), ("bf16", 64, 128), ("bf16", 80, 80)]


def _dev(x: np.ndarray, dtype: str, layout: str) -> torch.Tensor:
    """[B, H, rows, w] values on the device, in the requested memory layout."""
    if layout == "bnhd":
        x = np.ascontiguousarray(x.transpose(0, 2, 1, 3))  # memory [B, rows, H, w]
    if dtype == "bf16":
        t = torch.from_numpy(W.bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(DEV)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV)
    return t.permute(0, 2, 1, 3) if layout == "bnhd" else t


@pytest.mark.parametrize("p", [0.0, 0.25])
@pytest.mark.parametrize("mask", ["bitmask", "causal"])
@pytest.mark.parametrize("layout", ["bhnd", "bnhd"])
@pytest.mark.parametrize("dtype,d,v", DIMS)
def test_every_unit(dtype, d, v, layout, mask, p):
    import exact_tiled_attention_attn_amd as E

    B, H, n, nk, seed = 3, 2, 200, 333, 99
    off = nk - n if mask == "causal" else 0
    rng = np.random.default_rng(d + v + 7 * len(layout) + len(mask))
    Q = rng.standard_normal((B, H, n, d), dtype=np.float32)
    K = rng.standard_normal((B, H, nk, d), dtype=np.float32)
    V = rng.standard_normal((B, H, nk, v), dtype=np.float32)
    G = rng.standard_normal((B, H, n, v), dtype=np.float32)
    if dtype == "bf16":
        Q, K, V, G = (W.round_bf16(x) for x in (Q, K, V, G))
    if mask == "bitmask":
        # Different per unit: density 0.3 plus a unit-dependent band, one empty row per unit.
        A = rng.random((B, H, n, nk)) < 0.3
        for b in range(B):
            for h in range(H):
                A[b, h] |= W.causal_allowed(n, nk=nk, offset=off + 40 * (b * H + h) - 100)
                A[b, h, 3 + b * H + h] = False
        mdev = torch.from_numpy(W.pack_bits(A).view(np.int32)).to(DEV)  # [B, H, n, words]
        assert mdev.dim() == 4 and mdev.stride(0) != 0
    else:
        A = np.broadcast_to(W.causal_allowed(n, nk=nk, offset=off), (B, H, n, nk))
        mdev = None
    q, k, val, g = (_dev(x, dtype, layout) for x in (Q, K, V, G))
    c = 1 / np.sqrt(d)
    kw = dict(causal_offset=off, dropout_p=p, dropout_seed=seed)
    o = torch.empty_like(g)  # the layout of dO
    o, L = E.fwd(q, k, val, c, mask, mdev, out=o, **kw)
    res = {"atomic": E.bwd(q, k, val, o, g, L, c, mask, mdev, deterministic=False, **kw),
           "det": E.bwd(q, k, val, o, g, L, c, mask, mdev, deterministic=True, **kw)}
    torch.cuda.synchronize()
    got = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    p8 = dropout.p8_of(p)
    for b in range(B):
        for h in range(H):
            u = b * H + h
            Qh, Kh, Vh, Gh = (x[b, h].astype(np.float64) for x in (Q, K, V, G))
            Au = np.array(A[b, h])
            rows = np.nonzero(Au.any(axis=1))[0]
            empty = np.setdiff1d(np.arange(n), rows)
            tag = (dtype, d, v, layout, mask, p, b, h)
            Oh, Lh = got(o[b, h]), got(L[b, h])
            assert np.all(Oh[empty] == 0) and np.all(Lh[empty] == -np.inf), tag
            Qr, Gr, Ar = Qh[rows], Gh[rows], Au[rows]
            if p8:
                Z = dropout.keep_mask(seed, u, n, nk, p8)[rows]
                Y, Lr = dropout.forward(Qr, Kh, Vh, c, Ar, Z, p8)
                rdQ, rdK, rdV = dropout.vjp(Qr, Kh, Vh, c, Ar, Z, p8, Gr, stored(Y, dtype))
            else:
                Y, m, ell, Lr = dense.forward(Qr, Kh, Vh, c, Ar)
                rdQ, rdK, rdV = tiled.reverse(Qr, Kh, Vh, c, Ar, nk, stored(Y, dtype), m, ell, Gr)
            al = allowance_full(Qr, Kh, Vh, Gr, c, Ar, stored(Y, dtype), Lr, dtype, Z if p8 else None, p8)
            compare("O", Oh[rows], Y, dtype, tag, extra=al.get("O"))
            compare("L", Lh[rows], Lr, dtype, tag)
            mq, mk, mv, mg = (float(np.abs(x).max()) for x in (Qr, Kh, Vh, Gr))
            kinv = 256 / (256 - p8)
            bd = {"dQ": 2 * c * mk * mg * mv * v * kinv, "dK": 2 * c * mq * mg * mv * v * rows.size * kinv,
                  "dV": mg * rows.size * kinv}
            for path, (dq, dk, dv) in res.items():
                dqh = got(dq[b, h])
                assert np.all(dqh[empty] == 0), (tag, path)
                compare("dQ", dqh[rows], rdQ, dtype, (tag, path), bound=bd["dQ"], extra=al.get("dQ"),
                        zero_rows=one_key_rows(Ar))
                compare("dK", got(dk[b, h]), rdK, dtype, (tag, path), bound=bd["dK"], extra=al.get("dK"),
                        zero_rows=zero_key_rows(Ar))
                compare("dV", got(dv[b, h]), rdV, dtype, (tag, path), bound=bd["dV"], extra=al.get("dV"))
