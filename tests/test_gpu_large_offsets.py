"""Large offsets: 64-bit slice bases, 32-bit offsets up to the 2 GiB limit.

The kernels form each (batch, head) slice's base address in 64 bits and
address inside a slice with 32-bit offsets.  Two layouts must give, bit for
bit, the results of the same data in contiguous tensors (deterministic dQ
path):

* every tensor with a batch stride of 2^31 + 1024 elements, so that batch 1
  starts past 4 GiB of its allocation;
* one head of 1024 rows whose padded row stride puts the end of the last
  row just below 2^31 bytes, so that 1024 times the stride is past 2^31:
  buffer sizes taken as whole rows times the stride must not wrap.
"""

from __future__ import annotations

import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,d,mask", [(torch.bfloat16, 128, "causal"), (torch.bfloat16, 64, "none"),
                                          (torch.float32, 80, "causal")])
def test_batch_slices_beyond_4gib(dtype, d, mask):
    import exact_tiled_attention_attn_amd as E

    dev = "cuda:0"
    B, H, n = 2, 1, 300
    stride_b = (1 << 31) + 1024  # elements: batch 1 begins beyond 4 GiB (bf16) / 8 GiB (fp32)
    gen = torch.Generator(device="cpu").manual_seed(d)
    dense = [torch.randn((B, H, n, d), generator=gen).to(dtype).to(dev) for _ in range(4)]  # q, k, v, do

    def far(t=None):
        store = torch.empty(stride_b + H * n * d, dtype=dtype, device=dev)
        view = store.as_strided((B, H, n, d), (stride_b, n * d, d, 1))
        if t is not None:
            view.copy_(t)
        return view

    q, k, v, g = (far(t) for t in dense)
    o, dq, dk, dv = far(), far(), far(), far()
    L = torch.empty((B, H, n), dtype=torch.float32, device=dev)
    E.fwd(q, k, v, 0.125, mask, out=o, lse=L)
    E.bwd(q, k, v, o, g, L, 0.125, mask, dq=dq, dk=dk, dv=dv, deterministic=True)
    ro, rL = E.fwd(*dense[:3], 0.125, mask)
    rdq, rdk, rdv = E.bwd(*dense[:3], ro, dense[3], rL, 0.125, mask, deterministic=True)
    torch.cuda.synchronize()
    for name, x, r in (("O", o, ro), ("L", L, rL), ("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        assert torch.equal(x, r), name
    del q, k, v, g, o, dq, dk, dv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,d,v,mask", [(torch.bfloat16, 128, 128, "causal"), (torch.bfloat16, 64, 128, "none"),
                                            (torch.bfloat16, 80, 80, "causal"), (torch.float32, 64, 64, "none")])
def test_rows_up_to_the_2gib_limit(dtype, d, v, mask):
    import exact_tiled_attention_attn_amd as E

    dev = "cuda:0"
    n, es = 1024, torch.tensor([], dtype=dtype).element_size()
    stride = (1 << 31) // (n * es) + 16 // es  # elements per row, a 16-byte multiple
    assert n * stride * es > (1 << 31) and (n - 1) * stride * es + max(d, v) * es < (1 << 31)
    gen = torch.Generator(device="cpu").manual_seed(d + v)
    dense = [torch.randn((1, 1, n, w), generator=gen).to(dtype).to(dev) for w in (d, d, v, v)]  # q, k, v, do

    def far(w, t=None):
        store = torch.empty((n - 1) * stride + w, dtype=dtype, device=dev)
        view = store.as_strided((1, 1, n, w), (n * stride, n * stride, stride, 1))
        if t is not None:
            view.copy_(t)
        return view

    q, k, val, g = far(d, dense[0]), far(d, dense[1]), far(v, dense[2]), far(v, dense[3])
    o, dq, dk, dv = far(v), far(d), far(d), far(v)
    L = torch.empty((1, 1, n), dtype=torch.float32, device=dev)
    c = d ** -0.5
    E.fwd(q, k, val, c, mask, out=o, lse=L)
    E.bwd(q, k, val, o, g, L, c, mask, dq=dq, dk=dk, dv=dv, deterministic=True)
    adq, adk, adv = far(d), far(d), far(v)  # atomic path, outputs in the same layout
    E.bwd(q, k, val, o, g, L, c, mask, dq=adq, dk=adk, dv=adv, deterministic=False)
    ro, rL = E.fwd(*dense[:3], c, mask)
    rdq, rdk, rdv = E.bwd(*dense[:3], ro, dense[3], rL, c, mask, deterministic=True)
    torch.cuda.synchronize()
    for name, x, r in (("O", o, ro), ("L", L, rL), ("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        assert torch.equal(x, r), name
    tol = 1e-5 if dtype == torch.float32 else 2e-2
    for name, x, r in (("dQ", adq, rdq), ("dK", adk, rdk), ("dV", adv, rdv)):
        err = float((x.float() - r.float()).abs().max() / r.float().abs().max())
        assert err <= tol, (name, err)
    del q, k, val, g, o, dq, dk, dv, adq, adk, adv
    torch.cuda.empty_cache()
