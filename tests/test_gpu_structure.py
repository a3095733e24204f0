"""Mask/skip structure and edge cases of the HIP path (needs an MI355X).

* the tile classification the kernels use equals the oracle's, bit for bit;
* a key outside A_i cannot leak into row i: perturbing it leaves O_i, L_i and
  the deterministic dQ_i bitwise unchanged;
* keys that no row allows get exactly zero dK, dV;
* causal row 0 reproduces V_0 bitwise; empty rows are defined;
* strided layouts give bitwise the same results as contiguous ones;
* negative and zero scale, and Q = K = V aliasing, against the oracle;
* score ranges that grow by far more than the rescale slack per key tile;
* bitmask pad bits past nk and padding words of padded mask rows are ignored.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import dense, tilemap
from tests.gpu_common import DEV, compare, mask_dev, oracle_unit, run_gpu, to_dev

pytestmark = pytest.mark.gpu


def _bitmask_problem(n=700, H=2, d=64, v=128, dtype="bf16", seed=5, p=0.2):
    rng = np.random.default_rng(seed)
    allowed = rng.random((H, n, n)) < p
    allowed |= W.window_allowed(n, 64)[None]
    Q, K, V, G = (rng.standard_normal((1, H, n, x), dtype=np.float32) for x in (d, d, v, v))
    return W.custom(Q, K, V, G, scale=1 / np.sqrt(d), mask="bitmask", allowed=allowed, dtype=dtype)


@pytest.mark.parametrize("mask", ["none", "causal", "bitmask"])
@pytest.mark.parametrize("is_bwd", [0, 1, 2])
def test_tile_map_matches_oracle(mask, is_bwd):
    import exact_tiled_attention_attn_amd as E

    if mask == "bitmask":
        prob = _bitmask_problem(n=1000)
        # make some tiles fully empty and some fully allowed
        prob.mask_bool[0, :, 300:500] = False
        prob.mask_bool[0, np.arange(1000), np.arange(1000)] = True
        prob.mask_bool[1, 0:256, 0:512] = True
        prob.mask_words = W.pack_bits(prob.mask_bool)
    else:
        rng = np.random.default_rng(6)
        n = 1000
        Q, K, V, G = (rng.standard_normal((1, 2, n, 64), dtype=np.float32) for _ in range(4))
        prob = W.custom(Q, K, V, G, scale=0.125, mask=mask, dtype="bf16")
    w = prob.w
    q, k, v = (to_dev(prob, x) for x in "QKV")
    tmap, bq, bk = E.debug_tile_map(q, k, v, w.scale, w.mask, mask_dev(prob), is_bwd=is_bwd)
    got = tmap.cpu().numpy()
    units = got.shape[0]
    for u in range(units):
        want = tilemap.tile_map(prob.allowed(u), bq, bk)
        assert np.array_equal(got[u], want), (mask, is_bwd, u)
    if mask == "causal":
        assert np.array_equal(got[0], tilemap.causal_tile_map(w.n, bq, bk))
    print(mask, is_bwd, "tiles", bq, bk, "nonempty", tilemap.nonempty_tiles(got), flush=True)


def _run(prob, deterministic=True):
    import exact_tiled_attention_attn_amd as E

    w = prob.w
    q, k, v, g = (to_dev(prob, x) for x in "QKVG")
    m = mask_dev(prob)
    o, L = E.fwd(q, k, v, w.scale, w.mask, m)
    dq, dk, dv = E.bwd(q, k, v, o, g, L, w.scale, w.mask, m, deterministic=deterministic)
    torch.cuda.synchronize()
    return [t.cpu() for t in (o, L, dq, dk, dv)]


@pytest.mark.parametrize("mask", ["causal", "bitmask"])
def test_masked_key_perturbation_does_not_leak(mask):
    if mask == "bitmask":
        prob = _bitmask_problem(n=700)
    else:
        rng = np.random.default_rng(7)
        n = 700
        Q, K, V, G = (rng.standard_normal((1, 2, n, 128), dtype=np.float32) for _ in range(4))
        prob = W.custom(Q, K, V, G, scale=1 / np.sqrt(128), mask="causal", dtype="bf16")
    base = _run(prob)
    j = 333
    K2, V2 = prob.K.copy(), prob.V.copy()
    rng = np.random.default_rng(8)
    K2[:, :, j] = 50.0 * rng.standard_normal(K2.shape[-1])
    V2[:, :, j] = 100.0 * rng.standard_normal(V2.shape[-1])
    allowed = prob.mask_bool if mask == "bitmask" else None
    pert = W.custom(prob.Q, K2, V2, prob.G, scale=prob.w.scale, mask=mask, allowed=allowed, dtype="bf16")
    new = _run(pert)
    for h in range(prob.w.H):
        A = prob.allowed(h)
        out_rows = ~A[:, j]
        in_rows = A[:, j]
        assert out_rows.any() and in_rows.any()
        for idx, name in ((0, "O"), (1, "L"), (2, "dQ")):
            a, b = base[idx][0, h], new[idx][0, h]
            assert torch.equal(a[out_rows], b[out_rows]), (mask, h, name)
        assert not torch.equal(base[0][0, h][in_rows], new[0][0, h][in_rows])


def test_unreferenced_keys_get_zero_gradients():
    prob = _bitmask_problem(n=600)
    dead = [5, 100, 599]
    prob.mask_bool[:, :, dead] = False
    prob.mask_bool[:, np.arange(600), (np.arange(600) + 1) % 600] = True  # keep rows nonempty
    prob.mask_bool[:, :, dead] = False
    assert prob.mask_bool.any(axis=2).all()
    prob.mask_words = W.pack_bits(prob.mask_bool)
    for det in (True, False):
        o, L, dq, dk, dv = _run(prob, det)
        for j in dead:
            assert torch.all(dk[0, :, j] == 0) and torch.all(dv[0, :, j] == 0), (det, j)


def test_causal_row0_is_v0_bitwise():
    prob = W.generate("bf16_causal_h32_n16384_d128", heads=2, n=300)
    o, L, *_ = _run(prob)
    v = to_dev(prob, "V").cpu()
    assert torch.equal(o[0, :, 0], v[0, :, 0])
    # L_0 = c <Q_0, K_0>
    s = prob.w.scale * (prob.Q[0, :, 0].astype(np.float64) * prob.K[0, :, 0]).sum(-1)
    assert np.abs(L[0, :, 0].numpy() - s).max() < 1e-4 * max(1, np.abs(s).max())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_empty_rows_are_defined(dtype):
    prob = _bitmask_problem(n=500, dtype=dtype, d=64, v=64)
    empty = [0, 77, 499]
    prob.mask_bool[:, empty, :] = False
    prob.mask_words = W.pack_bits(prob.mask_bool)
    for det in (True, False):
        o, L, dq, dk, dv = _run(prob, det)
        assert torch.all(o[0, :, empty] == 0)
        assert torch.all(torch.isneginf(L[0, :, empty]))
        assert torch.all(dq[0, :, empty] == 0)
        keep = np.setdiff1d(np.arange(500), empty)
        for h in range(prob.w.H):
            # Reference: the same problem without the empty rows (they contribute nothing).
            Q, K, V, G = (getattr(prob, x)[0, h].astype(np.float64) for x in "QKVG")
            A = prob.mask_bool[h][keep]
            Y, m, ell, Lr = dense.forward(Q[keep], K, V, prob.w.scale, A)
            from tests.gpu_common import allowance_full, stored
            from oracle import tiled
            rdq, rdk, rdv = tiled.reverse(Q[keep], K, V, prob.w.scale, A, 500, stored(Y, dtype), m, ell, G[keep])
            al = allowance_full(Q[keep], K, V, G[keep], prob.w.scale, A, stored(Y, dtype), Lr, dtype)
            compare("O", o[0, h][keep].double().numpy(), Y, dtype, ("empty", h), extra=al.get("O"))
            compare("dQ", dq[0, h][keep].double().numpy(), rdq, dtype, ("empty", h, det), extra=al.get("dQ"))
            compare("dK", dk[0, h].double().numpy(), rdk, dtype, ("empty", h, det), extra=al.get("dK"))
            compare("dV", dv[0, h].double().numpy(), rdv, dtype, ("empty", h, det), extra=al.get("dV"))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_strided_layout_matches_contiguous_bitwise(dtype):
    import exact_tiled_attention_attn_amd as E

    rng = np.random.default_rng(9)
    B, H, n, d = 2, 3, 333, 128
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    base = [torch.from_numpy(rng.standard_normal((B, n, H, d), dtype=np.float32)).to(DEV).to(tdt)
            for _ in range(4)]
    strided = [t.permute(0, 2, 1, 3) for t in base]  # [B, H, n, d] view, row stride H*d
    contig = [t.contiguous() for t in strided]
    outs = []
    for q, k, v, g in (strided, contig):
        o = torch.empty_like(q)  # preserves the strided layout
        o, L = E.fwd(q, k, v, 0.1, "causal", out=o)
        dq, dk, dv = E.bwd(q, k, v, o, g, L, 0.1, "causal", deterministic=True)
        torch.cuda.synchronize()
        outs.append([x.contiguous().cpu() for x in (o, L, dq, dk, dv)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    assert not strided[0].is_contiguous()


@pytest.mark.parametrize("scale", [-0.3, 0.0])
@pytest.mark.parametrize("mask", ["none", "causal", "bitmask"])
def test_negative_and_zero_scale(scale, mask):
    rng = np.random.default_rng(10)
    n, d = 300, 64
    Q, K, V, G = (rng.standard_normal((1, 2, n, d), dtype=np.float32) for _ in range(4))
    allowed = None
    if mask == "bitmask":
        allowed = rng.random((2, n, n)) < 0.3
        allowed[:, np.arange(n), np.arange(n)] = True
    for dtype in ("f32", "bf16"):
        prob = W.custom(Q, K, V, G, scale=scale, mask=mask, allowed=allowed, dtype=dtype)
        got = run_gpu(prob)
        for h in range(2):
            ref = oracle_unit(prob, 0, h)
            for name in ("O", "L", "dQ", "dK", "dV"):
                if scale == 0.0 and name in ("dQ", "dK"):
                    assert np.all(got[name][0, h] == 0) and np.all(got[name + "_det"][0, h] == 0)
                    continue
                ex = ref["allow"].get(name)
                compare(name, got[name][0, h], ref[name], dtype, (scale, mask, dtype, name), extra=ex)
                if name in ("dQ", "dK", "dV"):
                    compare(name, got[name + "_det"][0, h], ref[name], dtype, (scale, mask, dtype, name, "det"),
                            extra=ex)


@pytest.mark.parametrize("mask", ["none", "causal", "bitmask"])
@pytest.mark.parametrize("d", [64, 128])
def test_reference_max_raised_between_tiles(mask, d):
    """Scores whose range grows from one 64-key tile to the next by far more
    than the lazy-rescale slack, so that the running reference max is raised
    in the middle of the key sequence (the pipelined forward's exact path);
    with the bitmask, even rows have no allowed key before key 300 (their
    reference is still -inf when their first weights arrive)."""
    rng = np.random.default_rng(21 + d)
    n = nk = 640
    Q = rng.standard_normal((1, 2, n, d), dtype=np.float32)
    K = rng.standard_normal((1, 2, nk, d), dtype=np.float32)
    K *= (1.0 + 4.0 * (np.arange(nk) // 64))[None, None, :, None].astype(np.float32)
    V = rng.standard_normal((1, 2, nk, 128), dtype=np.float32)
    G = rng.standard_normal((1, 2, n, 128), dtype=np.float32)
    allowed = None
    if mask == "bitmask":
        allowed = np.ones((2, n, nk), bool)
        allowed[:, 0::2, :300] = False
    prob = W.custom(Q, K, V, G, scale=1 / np.sqrt(d), mask=mask, allowed=allowed, dtype="bf16")
    got = run_gpu(prob)
    for h in range(2):
        ref = oracle_unit(prob, 0, h)
        for name in ("O", "L", "dQ", "dK", "dV"):
            ex = ref["allow"].get(name)
            compare(name, got[name][0, h], ref[name], "bf16", (mask, d, name), extra=ex)
            if name in ("dQ", "dK", "dV"):
                compare(name, got[name + "_det"][0, h], ref[name], "bf16", (mask, d, name, "det"), extra=ex)


def test_self_attention_aliased_inputs():
    import exact_tiled_attention_attn_amd as E

    rng = np.random.default_rng(11)
    n, d = 257, 64
    X = rng.standard_normal((1, 1, n, d), dtype=np.float32)
    G = rng.standard_normal((1, 1, n, d), dtype=np.float32)
    x = torch.from_numpy(X).to(DEV)
    g = torch.from_numpy(G).to(DEV)
    o, L = E.fwd(x, x, x, 1.0 / 8, "causal")
    dq, dk, dv = E.bwd(x, x, x, o, g, L, 1.0 / 8, "causal", deterministic=True)
    torch.cuda.synchronize()
    A = W.causal_allowed(n)
    Y, _, _, Lr = dense.forward(X[0, 0], X[0, 0], X[0, 0], 1 / 8, A)
    rdq, rdk, rdv = dense.vjp(X[0, 0], X[0, 0], X[0, 0], 1 / 8, A, G[0, 0])
    compare("O", o[0, 0].cpu().double().numpy(), Y, "f32")
    compare("L", L[0, 0].cpu().double().numpy(), Lr, "f32")
    dx = (dq + dk + dv)[0, 0].cpu().double().numpy()
    compare("dQ", dx, rdq + rdk + rdv, "f32")


@pytest.mark.parametrize("dtype,d,v", [(torch.bfloat16, 128, 128), (torch.bfloat16, 64, 128), (torch.float32, 80, 80)])
def test_mask_pad_bits_and_padded_rows_are_ignored(dtype, d, v):
    """Bits past nk in a row's last word, and words past ceil(nk / 32) in a
    padded row (mask row stride above the word count), are never read as
    allowed keys: set to ones, they leave every output bitwise unchanged."""
    import exact_tiled_attention_attn_amd as E

    H, n, nk = 2, 300, 333  # 11 words per row, the last one with 13 key bits and 19 pad bits
    rng = np.random.default_rng(d + v)
    A = rng.random((H, n, nk)) < 0.3
    A[:, np.arange(n), rng.integers(0, nk, n)] = True
    words = W.pack_bits(A)  # [H, n, 11] uint32, pad bits 0
    assert words.shape[-1] == 11
    padded = np.full((H, n, 16), 0xFFFFFFFF, np.uint32)  # row stride 16 words, padding all ones
    padded[..., :11] = words
    padded[..., 10] |= np.uint32(~((1 << (nk % 32)) - 1) & 0xFFFFFFFF)  # pad bits past nk set
    clean = torch.from_numpy(words.view(np.int32)).to(DEV)
    dirty = torch.from_numpy(padded.view(np.int32)).to(DEV)
    g0 = torch.Generator().manual_seed(d)
    q = torch.randn((1, H, n, d), generator=g0).to(dtype).to(DEV)
    k = torch.randn((1, H, nk, d), generator=g0).to(dtype).to(DEV)
    val = torch.randn((1, H, nk, v), generator=g0).to(dtype).to(DEV)
    g = torch.randn((1, H, n, v), generator=g0).to(dtype).to(DEV)
    c = d ** -0.5
    res = []
    for m in (clean, dirty):
        o, L = E.fwd(q, k, val, c, "bitmask", m)
        det = E.bwd(q, k, val, o, g, L, c, "bitmask", m, deterministic=True)
        maps = [E.debug_tile_map(q, k, val, c, "bitmask", m, is_bwd=i)[0] for i in range(3)]
        res.append([o, L, *det, *maps])
    torch.cuda.synchronize()
    names = ["O", "L", "dQ", "dK", "dV", "map_fwd", "map_bwd", "map_dq"]
    for name, a, b in zip(names, *res):
        assert torch.equal(a, b), name


def _count_case(dtype, d, v, n, nk, mask, off, seed):
    rng = np.random.default_rng(seed)
    H = 2
    Q, K, V, G = (rng.standard_normal((1, H, r, c), dtype=np.float32) for r, c in ((n, d), (nk, d), (nk, v), (n, v)))
    if mask == "bitmask":
        A = rng.random((H, n, nk)) < 0.02
        A[:, :, : nk // 3] = False  # whole empty key tiles
        A[:, : n // 4] = False      # whole empty query tiles
        A[0, : n // 4, -40:] = True  # and a few nonempty among them
        allowed = [A[h] for h in range(H)]
    elif mask == "causal":
        allowed = [W.causal_allowed(n, nk=nk, offset=off)] * H
    else:
        allowed = [np.ones((n, nk), bool)] * H
    return (Q, K, V, G), allowed, H


@pytest.mark.parametrize("dtype,d,v", [("bf16", 128, 128), ("bf16", 64, 128), ("bf16", 80, 80), ("f32", 64, 64)])
@pytest.mark.parametrize("mask,n,nk,off", [("none", 700, 700, 0), ("causal", 1000, 1000, 0),
                                          ("causal", 300, 1500, 1200), ("causal", 900, 600, -250),
                                          ("causal", 128, 4096, 3968), ("bitmask", 800, 900, 0),
                                          ("bitmask", 128, 4096, 0)])
def test_executed_tiles_equal_nonempty_tiles(dtype, d, v, mask, n, nk, off):
    """Every kernel computes exactly the tiles the oracle's classification
    calls nonempty, at its own tiling (key-range splits included), and skips
    the rest: the debug counters against oracle/tilemap.py."""
    import exact_tiled_attention_attn_amd as E

    (Q, K, V, G), allowed, H = _count_case(dtype, d, v, n, nk, mask, off, seed=n + nk + d)

    def dev(x):
        if dtype == "bf16":
            return torch.from_numpy(W.bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(DEV)
        return torch.from_numpy(x).to(DEV)

    q, k, val, g = (dev(x) for x in (Q, K, V, G))
    mdev = None
    if mask == "bitmask":
        mdev = torch.from_numpy(W.pack_bits(np.stack(allowed)).view(np.int32)).to(DEV)
    def nonempty(is_bwd, det=True):
        _, bq, bk = E.debug_tile_map(q, k, val, 0.125, mask, mdev, is_bwd=is_bwd, causal_offset=off,
                                     deterministic=det)
        return sum(tilemap.nonempty_tiles(tilemap.tile_map(allowed[h], bq, bk)) for h in range(H))

    want = [nonempty(is_bwd) for is_bwd in (0, 1, 2)]
    want_atomic_kv = nonempty(1, det=False)  # the fused kernel's key-tile-outer tiling
    counters = torch.zeros(3, dtype=torch.int64, device=DEV)
    E.count_tiles(counters)
    try:
        o, L = E.fwd(q, k, val, 0.125, mask, mdev, causal_offset=off)
        E.bwd(q, k, val, o, g, L, 0.125, mask, mdev, deterministic=True, causal_offset=off)
        torch.cuda.synchronize()
        got_det = counters.cpu().tolist()
        counters.zero_()
        E.bwd(q, k, val, o, g, L, 0.125, mask, mdev, deterministic=False, causal_offset=off)
        torch.cuda.synchronize()
        got_atomic = counters.cpu().tolist()
    finally:
        E.count_tiles(None)
    print(dtype, d, v, mask, n, nk, off, "nonempty", want, "executed", got_det, got_atomic, flush=True)
    assert got_det == want, (got_det, want)
    assert got_atomic == [0, want_atomic_kv, 0], (got_atomic, want_atomic_kv)
