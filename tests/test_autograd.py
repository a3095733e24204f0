"""Host logic of the autograd wrapper and the saved-state measurement (CPU).

The library's fwd / bwd are replaced here by float64-oracle functions on CPU
tensors, so that what the wrapper saves, which gradient goes to which input
and the shared-input sum can be checked without a GPU.  The GPU versions of
these checks (tests/test_gpu_autograd.py) run the real kernels.

The saved-state figures re-run the measurement of the "What Ordinary
Autograd Saves" page: a tiled forward traced by ordinary autograd retains
quadratic state, the wrapper exactly Q, K, V, O and L.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from exact_tiled_attention_attn_amd import _binding
from exact_tiled_attention_attn_amd import autograd as AG
from oracle import dense
from tests.payload import retained_by, traced_tiled_forward


def _allowed(mask_mode, mask, n, nk, offset=0):
    if mask_mode == "none":
        return lambda b, h: None
    if mask_mode == "causal":
        A = W.causal_allowed(n, nk=nk, offset=offset)
        return lambda b, h: A
    words = mask.numpy().view(np.uint32)
    return lambda b, h: W.unpack_bits(words[h] if words.ndim == 3 else words[b, h], nk)


def _oracle_fwd(q, k, v, scale, mask_mode="none", mask=None, causal_offset=0, dropout_p=0.0, dropout_seed=0):
    assert dropout_p == 0.0
    B, H, n, _ = q.shape
    A = _allowed(mask_mode, mask, n, k.shape[2], causal_offset)
    o = torch.empty((B, H, n, v.shape[-1]), dtype=q.dtype)
    L = torch.empty((B, H, n), dtype=torch.float32)
    for b in range(B):
        for h in range(H):
            Y, _, _, Lr = dense.forward(q[b, h].double().numpy(), k[b, h].double().numpy(),
                                        v[b, h].double().numpy(), scale, A(b, h))
            o[b, h] = torch.from_numpy(Y).to(q.dtype)
            L[b, h] = torch.from_numpy(Lr).float()
    return o, L


def _oracle_bwd(q, k, v, o, do, lse, scale, mask_mode="none", mask=None, *, deterministic=False,
                causal_offset=0, dropout_p=0.0, **_):
    assert dropout_p == 0.0
    B, H, n, _ = q.shape
    A = _allowed(mask_mode, mask, n, k.shape[2], causal_offset)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    for b in range(B):
        for h in range(H):
            r = dense.vjp(q[b, h].double().numpy(), k[b, h].double().numpy(), v[b, h].double().numpy(),
                          scale, A(b, h), do[b, h].double().numpy())
            for t, x in zip((dq, dk, dv), r):
                t[b, h] = torch.from_numpy(x).to(t.dtype)
    return dq, dk, dv


@pytest.fixture
def cpu_kernels(monkeypatch):
    calls = []

    def fwd(*a, **kw):
        calls.append("fwd")
        return _oracle_fwd(*a, **kw)

    def bwd(*a, **kw):
        calls.append(("bwd", kw.get("deterministic")))
        return _oracle_bwd(*a, **kw)

    monkeypatch.setattr(_binding, "fwd", fwd)
    monkeypatch.setattr(_binding, "bwd", bwd)
    return calls


def _inputs(B, H, n, d, v, seed=0, dtype=torch.float64):
    g = torch.Generator().manual_seed(seed)
    q, k = (torch.randn((B, H, n, d), generator=g, dtype=dtype) for _ in range(2))
    val = torch.randn((B, H, n, v), generator=g, dtype=dtype)
    G = torch.randn((B, H, n, v), generator=g, dtype=dtype)
    return q, k, val, G


def test_saved_state_is_q_k_v_o_l(cpu_kernels):
    B, H, n, d, v = 2, 3, 40, 5, 7
    q, k, val, G = _inputs(B, H, n, d, v)
    for t in (q, k, val):
        t.requires_grad_(True)
    c = retained_by(lambda: AG.attention(q, k, val, 0.3, "causal").backward(G))
    es = q.element_size()
    assert c.events == 5
    assert c.bytes == es * B * H * n * (2 * d + 2 * v) + 4 * B * H * n
    assert cpu_kernels == ["fwd", ("bwd", True)]


@pytest.mark.parametrize("mask_mode", ["none", "causal", "bitmask"])
def test_gradients_route_to_their_inputs(cpu_kernels, mask_mode):
    B, H, n, d, v = 1, 2, 33, 3, 6  # d != v, so a swapped dK / dV cannot pass
    q, k, val, G = _inputs(B, H, n, d, v, seed=1)
    mask = None
    if mask_mode == "bitmask":
        rng = np.random.default_rng(2)
        A = (rng.random((H, n, n)) < 0.4) | np.eye(n, dtype=bool)[None]
        mask = torch.from_numpy(W.pack_bits(A).view(np.int32))
    for t in (q, k, val):
        t.requires_grad_(True)
    o, lse = AG.attention(q, k, val, 0.7, mask_mode, mask, return_lse=True)
    assert not lse.requires_grad
    o.backward(G)
    ref = _oracle_bwd(q.detach(), k.detach(), val.detach(), None, G, None, 0.7, mask_mode, mask)
    for got, want in zip((q.grad, k.grad, val.grad), ref):
        assert torch.equal(got, want)
    ro, rl = _oracle_fwd(q.detach(), k.detach(), val.detach(), 0.7, mask_mode, mask)
    assert torch.equal(o.detach(), ro) and torch.equal(lse, rl)


def test_only_requested_gradients(cpu_kernels):
    q, k, val, G = _inputs(1, 1, 9, 4, 4, seed=3)
    k.requires_grad_(True)
    AG.attention(q, k, val, 0.5).backward(G)
    assert q.grad is None and val.grad is None and k.grad is not None


def test_default_scale_and_flags(cpu_kernels, monkeypatch):
    seen = {}

    def fwd(q, k, v, scale, mask_mode="none", mask=None, causal_offset=0, **kw):
        seen["scale"], seen["mask"] = scale, mask_mode
        return _oracle_fwd(q, k, v, scale, mask_mode, mask, causal_offset, **kw)

    def bwd(*a, deterministic=False, **kw):
        seen["det"] = deterministic
        return _oracle_bwd(*a, **kw)

    monkeypatch.setattr(_binding, "fwd", fwd)
    monkeypatch.setattr(_binding, "bwd", bwd)
    q, k, val, G = _inputs(1, 1, 5, 16, 4, seed=4)
    q.requires_grad_(True)
    AG.attention(q, k, val, deterministic=False).backward(G)
    assert seen == {"scale": 0.25, "mask": "none", "det": False}


def test_self_attention_sums_the_three_gradients(cpu_kernels):
    """Q = K = V = X, c = 1 (HarshvardhanJ README, self-attention): dX = dQ + dK + dV."""
    x, _, _, G = _inputs(1, 2, 17, 6, 6, seed=5)
    x.requires_grad_(True)
    AG.self_attention(x, 1.0, "causal").backward(G)
    dq, dk, dv = _oracle_bwd(x.detach(), x.detach(), x.detach(), None, G, None, 1.0, "causal")
    assert torch.allclose(x.grad, dq + dk + dv, rtol=0, atol=1e-14)


def test_traced_tiled_forward_retains_quadratic_state():
    """The page's experiment at d = 32, block 32: traced tiled state grows ~4x per
    doubling of T (quadratic), the wrapper's 2x (linear, exactly Q, K, V, O, L)."""
    d, block = 32, 32
    traced, ours = [], []
    for T in (128, 256, 512):
        g = torch.Generator().manual_seed(T)
        q, k, v = (torch.randn((T, d), generator=g, requires_grad=True) for _ in range(3))
        c = retained_by(lambda: traced_tiled_forward(q, k, v, d ** -0.5, block).sum().backward())
        traced.append(c.bytes)
        ours.append(3 * T * d * 4 + T * d * 4 + 4 * T)  # fp32 Q, K, V, O and L
        # The traced forward computes the same function as the definition.
        Y, _, _, _ = dense.forward(q.detach().double().numpy(), k.detach().double().numpy(),
                                   v.detach().double().numpy(), d ** -0.5, None)
        out = traced_tiled_forward(q.detach(), k.detach(), v.detach(), d ** -0.5, block)
        assert np.abs(out.double().numpy() - Y).max() < 1e-5
    for a, b_ in zip(traced, traced[1:]):
        assert 3.2 < b_ / a < 4.0, traced
    for a, b_ in zip(ours, ours[1:]):
        assert b_ == 2 * a
    assert traced[-1] > 10 * ours[-1]
