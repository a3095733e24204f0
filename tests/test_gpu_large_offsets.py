"""Batch slices more than 4 GiB apart: 64-bit base addresses in every kernel.

The kernels form each (batch, head) slice's base address in 64 bits and
address inside a slice with 32-bit offsets.  Here every tensor has a batch
stride of 2^31 + 1024 elements, so batch 1 starts past 4 GiB of its
allocation; its results must equal, bit for bit, those of the same data in
contiguous tensors (deterministic dQ path).
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
