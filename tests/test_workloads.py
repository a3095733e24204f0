"""The seeded input generator: bf16 rounding, mask packing and recipes (CPU)."""

import numpy as np
import torch

import workloads as W


def test_bf16_rne_matches_torch_bitwise():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000, dtype=np.float32) * np.float32(3.0),
        np.float32([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, -3.4e38, 1e-40, -1e-40]),
        # exact ties: mantissa low half 0x8000, odd and even kept bits
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x40490FDB], dtype=np.uint32).view(np.float32),
    ])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(W.bf16_bits(x), want)
    assert np.array_equal(W.round_bf16(x), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_pack_bits_layout():
    rng = np.random.default_rng(1)
    for n in (1, 31, 32, 33, 100, 257):
        A = rng.random((3, n, n)) < 0.3
        words = W.pack_bits(A)
        assert words.dtype == np.uint32 and words.shape == (3, n, (n + 31) // 32)
        assert np.array_equal(W.unpack_bits(words, n), A)
        for _ in range(50):
            h, i, j = rng.integers(0, 3), rng.integers(0, n), rng.integers(0, n)
            assert bool((int(words[h, i, j >> 5]) >> (j & 31)) & 1) == bool(A[h, i, j])
        # pad bits are zero
        if n % 32:
            assert np.all(words[..., -1] >> np.uint32(n % 32) == 0)


def test_recipes_are_deterministic_and_shaped():
    for name in W.ORDER:
        w = W.WORKLOADS[name]
        p1 = W.generate(name, heads=1, n=min(w.n, 300))
        p2 = W.generate(name, heads=1, n=min(w.n, 300))
        for a in ("Q", "K", "V", "G"):
            x = getattr(p1, a)
            assert np.array_equal(x, getattr(p2, a))
            assert x.shape[:3] == (w.B, 1, min(w.n, 300))
            if w.dtype == "bf16":
                assert np.array_equal(W.round_bf16(x), x)
        assert p1.Q.shape[-1] == w.d and p1.V.shape[-1] == w.v


def test_qk_scale_recipe():
    p = W.generate("bf16_b4h16_n4096_d128", heads=1, n=512)
    assert 0.45 < p.Q.std() < 0.55 and 0.9 < p.V.std() < 1.1
    p = W.generate("bf16_bitmask_b2h8_n8192_d64v128", heads=1, n=1024)
    assert 1.8 < p.K.std() < 2.2


def test_bitmask_recipe_rows():
    p = W.generate("bf16_bitmask_b2h8_n8192_d64v128", heads=2, n=2048)
    w = p.w
    M = p.mask_bool
    assert M.shape == (2, 2048, 2048)
    assert M.any(axis=2).all()  # every row nonempty (the window holds j = i)
    assert M[:, np.arange(2048), np.arange(2048)].all()
    win = W.window_allowed(2048, w.window)
    assert np.all(M[:, win])  # the window is always allowed
    assert win[1000].sum() == 1024  # interior rows have exactly `window` keys
    extra = (M & ~win).sum(axis=2).mean()
    exp = w.n_global / 2048 * (2048 - win.sum(1).mean())
    assert abs(extra - exp) < 0.1 * exp
    assert np.array_equal(W.unpack_bits(p.mask_words, 2048), M)


def test_pair_and_flop_counts():
    w = W.WORKLOADS["bf16_causal_h32_n16384_d128"]
    pairs = W.allowed_pairs(w)
    assert pairs == 32 * 16384 * 16385 // 2
    f, b = W.flops(w, pairs)
    assert abs(f - 2.1992e12) / 2.1992e12 < 1e-4 and abs(b - 5.4979e12) / 5.4979e12 < 1e-4
