"""The autograd wrapper on the device: saved state, gradients, shared input.

* What autograd retains (saved-tensor hooks, the measurement of the "What
  Ordinary Autograd Saves" page): exactly Q, K, V, O and L, i.e.
  es (2d + 2v) n + 4 n bytes per head, linear in n.
* The gradients are the library's backward, bit for bit (deterministic dQ).
* Shared input Q = K = V = X with c = 1 (HarshvardhanJ README,
  self-attention): X's gradient is dQ + dK + dV, against the oracle.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import dense
from tests.gpu_common import DEV, allowance_full, compare, stored
from tests.payload import retained_by

pytestmark = pytest.mark.gpu


def _tensors(B, H, n, d, v, dtype, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    q, k = (torch.randn((B, H, n, d), generator=g) for _ in range(2))
    val = torch.randn((B, H, n, v), generator=g)
    G = torch.randn((B, H, n, v), generator=g)
    return [t.to(dtype).to(DEV) for t in (q, k, val, G)]


@pytest.mark.parametrize("dtype,d,v,mask", [(torch.bfloat16, 128, 128, "causal"),
                                             (torch.bfloat16, 64, 128, "none"),
                                             (torch.float32, 64, 64, "causal")])
def test_saved_state_is_linear(dtype, d, v, mask):
    import exact_tiled_attention_attn_amd as E

    B, H = 1, 2
    sizes = []
    for n in (128, 256, 512, 1024):
        q, k, val, G = _tensors(B, H, n, d, v, dtype, n)
        for t in (q, k, val):
            t.requires_grad_(True)
        c = retained_by(lambda: E.attention(q, k, val, None, mask).backward(G))
        torch.cuda.synchronize()
        es = q.element_size()
        assert c.events == 5
        assert c.bytes == es * B * H * n * (2 * d + 2 * v) + 4 * B * H * n
        sizes.append(c.bytes)
    assert all(b_ == 2 * a for a, b_ in zip(sizes, sizes[1:]))


@pytest.mark.parametrize("dtype,mask", [(torch.bfloat16, "causal"), (torch.float32, "none")])
def test_gradients_are_the_library_backward(dtype, mask):
    import exact_tiled_attention_attn_amd as E

    d = 128 if dtype == torch.bfloat16 else 64
    q, k, val, G = _tensors(2, 3, 777, d, d, dtype, 7)
    for t in (q, k, val):
        t.requires_grad_(True)
    o, lse = E.attention(q, k, val, 0.1, mask, return_lse=True)
    o.backward(G)
    ro, rl = E.fwd(q.detach(), k.detach(), val.detach(), 0.1, mask)
    dq, dk, dv = E.bwd(q.detach(), k.detach(), val.detach(), ro, G, rl, 0.1, mask, deterministic=True)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), ro) and torch.equal(lse, rl)
    assert torch.equal(q.grad, dq) and torch.equal(k.grad, dk) and torch.equal(val.grad, dv)


@pytest.mark.parametrize("dtype,mask", [(torch.float32, "causal"), (torch.float32, "none"),
                                        (torch.bfloat16, "causal")])
def test_self_attention_gradient(dtype, mask):
    import exact_tiled_attention_attn_amd as E

    n, d = 300, 64
    rng = np.random.default_rng(23)
    X = rng.standard_normal((1, 1, n, d), dtype=np.float32) * 0.25
    G = rng.standard_normal((1, 1, n, d), dtype=np.float32)
    tag = "f32" if dtype == torch.float32 else "bf16"
    if tag == "bf16":
        X, G = W.round_bf16(X), W.round_bf16(G)
    x = torch.from_numpy(X).to(dtype).to(DEV).requires_grad_(True)
    y = E.self_attention(x, 1.0, mask)
    y.backward(torch.from_numpy(G).to(dtype).to(DEV))
    torch.cuda.synchronize()
    A = W.causal_allowed(n) if mask == "causal" else None
    X64, G64 = X[0, 0].astype(np.float64), G[0, 0].astype(np.float64)
    Y, _, _, L = dense.forward(X64, X64, X64, 1.0, A)
    rdq, rdk, rdv = dense.vjp(X64, X64, X64, 1.0, A, G64)
    compare("O", y[0, 0].detach().float().cpu().double().numpy(), Y, tag, (dtype, mask),
            extra=allowance_full(X64, X64, X64, G64, 1.0, A, stored(Y, tag), L, tag).get("O"))
    # The reference is the exact VJP; dX = dQ + dK + dV carries the
    # allowances of all three (gpu_common.allowance_full).
    al = allowance_full(X64, X64, X64, G64, 1.0, A, stored(Y, tag), L, tag)
    extra = al.get("dQ", 0.0) + al.get("dK", 0.0) + al.get("dV", 0.0)
    compare("dQ", x.grad[0, 0].float().cpu().double().numpy(), rdq + rdk + rdv, tag, (dtype, mask), extra=extra)


def test_any_gradient_layout_and_input_views():
    """o.sum() hands the backward an expanded (all-zero-stride) gradient;
    inputs may be views with gaps between rows, or rows with a non-unit
    element stride (copied by attention()).  Each gives the library's
    backward of the same values, bit for bit."""
    import exact_tiled_attention_attn_amd as E

    B, H, n, d, c = 1, 2, 300, 64, 0.125
    g = torch.Generator().manual_seed(11)
    base = [torch.randn((B, H, n, d), generator=g).to(torch.bfloat16).to(DEV) for _ in range(3)]
    ro, rl = E.fwd(*base, c, "causal")
    ones = torch.ones_like(ro)
    ref = E.bwd(*base, ro, ones, rl, c, "causal", deterministic=True)

    # Expanded upstream gradient.
    q, k, v = (t.clone().requires_grad_(True) for t in base)
    E.attention(q, k, v, c, "causal").sum().backward()
    for x, r in zip((q.grad, k.grad, v.grad), ref):
        assert torch.equal(x, r)

    # Views with gaps: every other row of a twice-as-tall leaf.
    tall = [torch.zeros((B, H, 2 * n, d), dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    for t, b in zip(tall, base):
        t[:, :, ::2] = b
        t.requires_grad_(True)
    E.attention(*(t[:, :, ::2] for t in tall), c, "causal").sum().backward()
    for t, r in zip(tall, ref):
        assert torch.equal(t.grad[:, :, ::2], r) and not t.grad[:, :, 1::2].any()

    # Rows with a non-unit element stride: [B, H, d, n] memory seen as [B, H, n, d].
    wide = [b.transpose(-1, -2).contiguous().requires_grad_(True) for b in base]
    E.attention(*(w.transpose(-1, -2) for w in wide), c, "causal").sum().backward()
    for w, r in zip(wide, ref):
        assert torch.equal(w.grad.transpose(-1, -2), r)


def test_double_backward_is_refused():
    import exact_tiled_attention_attn_amd as E

    g = torch.Generator().manual_seed(3)
    q, k, v = (torch.randn((1, 1, 64, 64), generator=g).to(DEV).requires_grad_(True) for _ in range(3))
    with pytest.raises(RuntimeError, match="double backward"):
        torch.autograd.grad(E.attention(q, k, v).sum(), q, create_graph=True)
    o = E.attention(q, k, v)  # a plain backward still works
    o.backward(torch.ones_like(o))
    assert q.grad is not None and torch.isfinite(q.grad).all()


def test_binding_checks_tensor_arguments():
    """The library sees only pointers: the binding refuses host tensors,
    mixed dtypes or devices, and outputs of the wrong shape or dtype before
    any address reaches it."""
    import exact_tiled_attention_attn_amd as E

    q, k, v, G = _tensors(1, 2, 100, 64, 64, torch.bfloat16, 5)
    o, L = E.fwd(q, k, v, 0.125)
    with pytest.raises(ValueError, match="GPU memory"):
        E.fwd(q.cpu(), k, v, 0.125)
    with pytest.raises(TypeError, match="dtype"):
        E.fwd(q, k.float(), v, 0.125)
    with pytest.raises(ValueError, match="shape"):
        E.fwd(q, k, v, 0.125, out=torch.empty((1, 2, 99, 64), dtype=q.dtype, device=DEV))
    with pytest.raises(TypeError, match="dtype"):
        E.fwd(q, k, v, 0.125, lse=torch.empty((1, 2, 100), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(TypeError, match="dtype"):
        E.bwd(q, k, v, o, G.float(), L, 0.125)
    with pytest.raises(ValueError, match="shape"):
        E.bwd(q, k, v, o, G, L[:, :, :50], 0.125)
    with pytest.raises(TypeError, match="dtype"):
        E.bwd(q, k, v, o, G, L, 0.125, dq=torch.empty(q.shape, device=DEV))
    with pytest.raises(ValueError, match="GPU memory"):
        E.fwd(q, k, v, 0.125, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    torch.cuda.synchronize()
