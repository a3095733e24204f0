"""HIP path vs the float64 oracle, element by element (needs an MI355X).

Small and ragged problems are compared in full; the large workloads run at
full size in the benchmark's launch configuration and are compared on
sampled query rows (O, L, dQ) and key columns (dK, dV) that the oracle
evaluates one by one.
"""

from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from oracle import dense
from tests.gpu_common import compare, magnitude_bounds, oracle_unit, run_gpu, stored

pytestmark = pytest.mark.gpu


def _full_compare(prob, tag, exact_vjp=False):
    got = run_gpu(prob)
    w = prob.w
    errs = {}
    names = ["O", "L", "dQ", "dK", "dV"]
    for b in range(w.B):
        for h in range(w.H):
            ref = oracle_unit(prob, b, h, exact_vjp=exact_vjp)
            bounds = magnitude_bounds(prob, b, h)
            pairs = [(x, x) for x in names] + [(x + "_det", x) for x in ("dQ", "dK", "dV")]
            if exact_vjp:
                pairs += [(x, x + "_exact") for x in ("dQ", "dK", "dV")]
            for gname, rname in pairs:
                if w.dtype == "bf16" and w.n <= 2 and gname[:2] in ("dQ", "dK"):
                    # With at most two keys, dQ and dK are the difference of two
                    # terms p_ij (dP_ij - D_i); D_i = <dO_i, O_i> on the
                    # bf16-stored O carries O's +-1 ulp, which can exceed the
                    # difference.  Reported, not asserted (fp32 covers n <= 2).
                    e = np.abs(got[gname][b, h] - ref[rname]).max() / max(np.abs(ref[rname]).max(), 1e-30)
                    print(tag, gname, f"bf16 two-key relative error {e:.2e} (not asserted)")
                    assert np.all(np.isfinite(got[gname][b, h]))
                    continue
                errs[gname + "/" + rname] = max(
                    errs.get(gname + "/" + rname, 0.0),
                    compare(gname[:2], got[gname][b, h], ref[rname], w.dtype, (tag, b, h, gname),
                            bounds.get(gname[:2]), elementwise=w.n > 2, cond=1.0 if w.n > 2 else 4.0))
    print(tag, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    return errs


@pytest.mark.parametrize("name", ["f32_n256_d64", "f32_causal_n1000_d80"])
def test_fp32_workloads_full(name):
    _full_compare(W.generate(name), name, exact_vjp=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mask", ["none", "causal", "bitmask"])
@pytest.mark.parametrize("dims", [(64, 64), (80, 80), (128, 128), (64, 128)])
@pytest.mark.parametrize("n", [1, 2, 33, 127, 129, 200])
def test_ragged_small(dtype, mask, dims, n):
    d, v = dims
    rng = np.random.default_rng(1000 + n * 7 + d + v)
    B, H = 1, 2
    Q = rng.standard_normal((B, H, n, d), dtype=np.float32)
    K = rng.standard_normal((B, H, n, d), dtype=np.float32)
    V = rng.standard_normal((B, H, n, v), dtype=np.float32)
    G = rng.standard_normal((B, H, n, v), dtype=np.float32)
    allowed = None
    if mask == "bitmask":
        allowed = rng.random((H, n, n)) < 0.3
        allowed[:, np.arange(n), rng.integers(0, n, n)] = True
    prob = W.custom(Q, K, V, G, scale=1.0 / np.sqrt(d), mask=mask, allowed=allowed, dtype=dtype,
                    name=f"ragged_{dtype}_{mask}_{d}x{v}_n{n}")
    _full_compare(prob, prob.w.name)


def _sampled_compare(prob, units, n_rows=48, seed=0):
    """Full-size GPU run; oracle on sampled rows / columns of a few units."""
    w = prob.w
    got = run_gpu(prob)
    rng = np.random.default_rng(seed)
    n = w.n
    pick = lambda: np.unique(np.concatenate([np.arange(16), np.arange(n - 16, n),  # noqa: E731
                                             rng.choice(n, n_rows, replace=False)]))
    errs = {}
    for (b, h) in units:
        Q, K, V, G = (getattr(prob, x)[b, h] for x in ("Q", "K", "V", "G"))
        A_rows = (lambda r, h=h: np.ones((len(r), n), bool)) if w.mask == W.MASK_NONE \
            else (lambda r, h=h: prob.allowed(h, r))
        Y, _, _, L = dense.forward(Q, K, V, w.scale, None if w.mask == W.MASK_NONE else prob.allowed(h))
        rows, cols = pick(), pick()
        # delta from the forward output as stored (see oracle_unit).
        dQ, dK, dV = dense.grads_sampled(Q, K, V, w.scale, A_rows, G, L, stored(Y, w.dtype), rows, cols)
        tag = (w.name, b, h)
        checks = [("O", got["O"][b, h][rows], Y[rows]), ("L", got["L"][b, h][rows], L[rows])]
        for sfx in ("", "_det"):
            checks += [("dQ" + sfx, got["dQ" + sfx][b, h][rows], dQ),
                       ("dK" + sfx, got["dK" + sfx][b, h][cols], dK),
                       ("dV" + sfx, got["dV" + sfx][b, h][cols], dV)]
        for name, g, r in checks:
            errs[name] = max(errs.get(name, 0.0), compare(name[:2] if name != "L" else name, g, r, w.dtype, (tag, name)))
        # Whole-tensor invariants at any size: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i.
        sdk = got["dK"][b, h].sum(0)
        assert np.abs(sdk).max() <= 2e-2 * np.abs(got["dK"][b, h]).sum(0).max() + 1e-6, tag
        sdv, sg = got["dV"][b, h].sum(0), G.astype(np.float64).sum(0)
        assert np.abs(sdv - sg).max() <= 2e-2 * np.abs(G).sum(0).max(), tag
    print(w.name, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    return errs


def test_bf16_noncausal_b4h16_n4096_full_size():
    prob = W.generate("bf16_b4h16_n4096_d128")
    _sampled_compare(prob, [(0, 0), (1, 7), (3, 15)])


def test_bf16_causal_h32_n16384_full_size():
    prob = W.generate("bf16_causal_h32_n16384_d128")
    _sampled_compare(prob, [(0, 0), (0, 15), (0, 31)])


def test_bf16_bitmask_b2h8_n8192_full_size():
    prob = W.generate("bf16_bitmask_b2h8_n8192_d64v128")
    _sampled_compare(prob, [(0, 0), (1, 3), (1, 7)])


@pytest.mark.parametrize("name", ["bf16_b4h16_n4096_d128", "bf16_causal_h32_n16384_d128",
                                  "bf16_bitmask_b2h8_n8192_d64v128"])
def test_bf16_workloads_reduced_full_compare(name):
    """Same recipe with fewer heads and n = 1000 (ragged tail): compare everything."""
    prob = W.generate(name, heads=2, n=1000)
    _full_compare(prob, name + "_reduced", exact_vjp=True)


@pytest.mark.parametrize("name", ["bf16_causal_h32_n16384_d128", "bf16_bitmask_b2h8_n8192_d64v128",
                                  "f32_causal_n1000_d80"])
def test_deterministic_backward_is_bitwise_reproducible(name):
    import torch

    import exact_tiled_attention_attn_amd as E
    from tests.gpu_common import mask_dev, to_dev

    prob = W.generate(name, heads=2, n=1500)
    w = prob.w
    q, k, v, g = (to_dev(prob, x) for x in "QKVG")
    m = mask_dev(prob)
    o, L = E.fwd(q, k, v, w.scale, w.mask, m)
    first = E.bwd(q, k, v, o, g, L, w.scale, w.mask, m, deterministic=True)
    first = [t.clone() for t in first]
    for _ in range(3):
        again = E.bwd(q, k, v, o, g, L, w.scale, w.mask, m, deterministic=True)
        for a, b_ in zip(first, again):
            assert torch.equal(a, b_)
    # The forward is deterministic too.
    o2, L2 = E.fwd(q, k, v, w.scale, w.mask, m)
    assert torch.equal(o, o2) and torch.equal(L, L2)
