"""attn_bwd_noalloc on the device: the backward with the library's static
scratch as its workspace gives the workspace backward's results, on two
calls in a row (the second smaller), and allocates no device memory."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_common import DEV, compare

pytestmark = pytest.mark.gpu


def _case(H, n, d, v, mask, seed, dtype=torch.bfloat16):
    g = torch.Generator(device="cpu").manual_seed(seed)
    q, k = (torch.randn((1, H, n, d), generator=g).to(dtype).to(DEV) for _ in range(2))
    val, do = (torch.randn((1, H, n, v), generator=g).to(dtype).to(DEV) for _ in range(2))
    mdev = None
    if mask == "bitmask":
        rng = np.random.default_rng(seed)
        A = (rng.random((H, n, n)) < 0.2) | W.causal_allowed(n)[None]
        mdev = torch.from_numpy(W.pack_bits(A).view(np.int32)).to(DEV)
    return q, k, val, do, mdev


@pytest.mark.parametrize("deterministic", [True, False])
def test_noalloc_backward_equals_workspace_backward(deterministic):
    import exact_tiled_attention_attn_amd as E

    # The second call is smaller; it also runs the dQ kernel's key-range splits.
    cases = [(16, 4096, 128, 128, "causal", 1), (2, 1000, 64, 128, "bitmask", 2)]
    for H, n, d, v, mask, seed in cases:
        q, k, val, do, mdev = _case(H, n, d, v, mask, seed)
        c = d ** -0.5
        o, L = E.fwd(q, k, val, c, mask, mdev)
        ref = E.bwd(q, k, val, o, do, L, c, mask, mdev, deterministic=deterministic)
        outs = [torch.empty_like(t) for t in ref]
        torch.cuda.synchronize()
        # Resolve the scratch address once (the first call on this GPU loads
        # the array), then check that a call allocates nothing.
        E.bwd_noalloc(q, k, val, o, do, L, c, mask, mdev, dq=outs[0], dk=outs[1], dv=outs[2],
                      deterministic=deterministic)
        torch.cuda.synchronize()
        for t in outs:
            t.fill_(float("nan"))
        free0, alloc0 = torch.cuda.mem_get_info()[0], torch.cuda.memory_allocated()
        E.bwd_noalloc(q, k, val, o, do, L, c, mask, mdev, dq=outs[0], dk=outs[1], dv=outs[2],
                      deterministic=deterministic)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free0 and torch.cuda.memory_allocated() == alloc0
        for name, a, b in zip(("dQ", "dK", "dV"), outs, ref):
            if deterministic:
                assert torch.equal(a, b), (H, n, mask, name)  # same kernels, same arithmetic
            else:
                # dQ by fp32 atomics: run-to-run rounding order; dK, dV equal.
                x, r = a.float().cpu().numpy().astype(np.float64), b.float().cpu().numpy().astype(np.float64)
                compare(name, x.reshape(-1, x.shape[-1]), r.reshape(-1, r.shape[-1]), "bf16", (H, n, mask, name))


def test_noalloc_backward_with_dropout():
    """The same with dropout (the pipelined backward kernels replay the mask;
    both calls, the second smaller, also run the dQ key-range splits)."""
    import exact_tiled_attention_attn_amd as E

    for H, n, d, v, mask, seed in [(4, 2048, 128, 128, "causal", 4), (2, 512, 64, 128, "none", 5)]:
        q, k, val, do, mdev = _case(H, n, d, v, mask, seed)
        c, kw = d ** -0.5, dict(dropout_p=0.15, dropout_seed=seed)
        o, L = E.fwd(q, k, val, c, mask, mdev, **kw)
        ref = E.bwd(q, k, val, o, do, L, c, mask, mdev, deterministic=True, **kw)
        outs = [torch.full_like(t, float("nan")) for t in ref]
        E.bwd_noalloc(q, k, val, o, do, L, c, mask, mdev, dq=outs[0], dk=outs[1], dv=outs[2], deterministic=True,
                      **kw)
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), outs, ref):
            assert torch.equal(a, b), (H, n, mask, name)


def test_noalloc_refuses_problems_beyond_the_scratch():
    import exact_tiled_attention_attn_amd as E

    q, k, val, do, _ = _case(32, 4096, 128, 128, "causal", 3)  # atomic path: 4 B H n d = 64 MiB + D, L rows
    o, L = E.fwd(q, k, val, 0.1, "causal")
    with pytest.raises(E.AttnError, match="static"):
        E.bwd_noalloc(q, k, val, o, do, L, 0.1, "causal", deterministic=False)
