"""Forward + backward captured in a HIP graph and replayed.

Launch-bound loops (small problems, decode steps) are replayed from a
captured graph instead of being launched call by call.  The library issues
kernels only (no memsets, no allocation, no host synchronisation) on the
caller's stream, so a capture of attn_fwd + attn_bwd with caller-owned
outputs and workspaces replays correctly.  Checked here: several replays,
with eager work and new input values in between, each equal bit for bit
to the eager calls on the same inputs (deterministic dQ path).  Also: calls
on two streams at once give the results of the same calls made in sequence.
"""

from __future__ import annotations

import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,d,mask,nq,nk", [(torch.bfloat16, 128, "causal", 1000, 1000),
                                                (torch.bfloat16, 64, "none", 64, 4096),
                                                (torch.float32, 80, "causal", 333, 333)])
def test_graph_replays_match_eager(dtype, d, mask, nq, nk):
    import exact_tiled_attention_attn_amd as E

    dev = "cuda:0"
    B, H, c = 1, 4, d ** -0.5
    off = nk - nq if mask == "causal" else 0
    gen = torch.Generator(device="cpu").manual_seed(d + nq)
    mk = lambda rows, w: torch.randn((B, H, rows, w), generator=gen).to(dtype).to(dev)  # noqa: E731
    q, k, v, g = mk(nq, d), mk(nk, d), mk(nk, d), mk(nq, d)
    o = torch.empty((B, H, nq, d), dtype=dtype, device=dev)
    L = torch.empty((B, H, nq), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    pf = E.make_problem(q, k, v, o, c, mask, causal_offset=off)
    pb = E.make_problem(q, k, v, o, c, mask, None, True, off)
    ws_f = torch.empty(max(E.workspace_size(pf, False), 256), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(max(E.workspace_size(pb, True), 256), dtype=torch.uint8, device=dev)

    def step():
        E.fwd(q, k, v, c, mask, out=o, lse=L, workspace=ws_f, causal_offset=off)
        E.bwd(q, k, v, o, g, L, c, mask, dq=dq, dk=dk, dv=dv, workspace=ws_b, deterministic=True,
              causal_offset=off)

    def eager_ref():
        step()
        torch.cuda.synchronize()
        return [t.clone() for t in (o, L, dq, dk, dv)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream, as capture requires
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for it in range(3):
        if it == 2:  # new input values in the captured buffers
            for t in (q, k, v, g):
                t.copy_(torch.randn(t.shape, generator=gen).to(dtype).to(dev))
        torch.cuda.synchronize()
        ref = eager_ref()
        for t in (o, L, dq, dk, dv):
            t.fill_(float("nan"))  # eager work between replays; a stale output would show
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("O", "L", "dQ", "dK", "dV"), (o, L, dq, dk, dv), ref):
            assert torch.equal(got, want), (it, name)


def test_concurrent_streams_match_sequential_calls():
    """The library keeps no device state between calls: two problems issued
    on two streams at once, each with its own outputs and workspaces, give
    bit for bit the results of the same calls one after the other."""
    import exact_tiled_attention_attn_amd as E

    dev = "cuda:0"
    gen = torch.Generator(device="cpu").manual_seed(42)
    probs = []
    for (n, d, mask) in ((2048, 128, "causal"), (1500, 64, "none")):
        t = [torch.randn((2, 4, n, d), generator=gen).to(torch.bfloat16).to(dev) for _ in range(4)]
        probs.append((t, d ** -0.5, mask))

    def run(tensors, c, mask):
        q, k, v, g = tensors
        o, L = E.fwd(q, k, v, c, mask)
        return [o, L, *E.bwd(q, k, v, o, g, L, c, mask, deterministic=True)]

    ref = [run(*pr) for pr in probs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    got = []
    for _ in range(3):
        outs = []
        for s, pr in zip(streams, probs):
            with torch.cuda.stream(s):
                outs.append(run(*pr))
        torch.cuda.synchronize()
        got.append(outs)
    for outs in got:
        for r_list, g_list in zip(ref, outs):
            for name, r, x in zip(("O", "L", "dQ", "dK", "dV"), r_list, g_list):
                assert torch.equal(r, x), name
