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
from tests.gpu_common import DEV, compare
from tests.payload import payload

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
        c = payload(lambda a, b_, c_: E.attention(a, b_, c_, None, mask), q, k, val, grad=G)
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
    Y, _, _, _ = dense.forward(X64, X64, X64, 1.0, A)
    rdq, rdk, rdv = dense.vjp(X64, X64, X64, 1.0, A, G64)
    compare("O", y[0, 0].detach().float().cpu().double().numpy(), Y, tag, (dtype, mask))
    compare("dQ", x.grad[0, 0].float().cpu().double().numpy(), rdq + rdk + rdv, tag, (dtype, mask))
