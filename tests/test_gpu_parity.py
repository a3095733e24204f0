"""HIP path vs the float64 oracle, element by element (needs an MI355X).

Small and ragged problems are compared in full.  The large workloads run at
full size in the benchmark's launch configuration: O and L are compared on
every row of every (batch, head) unit against the dense definition, and the
gradients on sampled query rows (dQ) and key columns (dK, dV) of every unit,
which the oracle evaluates one by one.

Gradients have two references: the reverse procedure with delta_i taken on
the forward output as stored (the procedure consumes a forward run's Y), and
the exact VJP (float64 Y, or the rowsum(P o dP) form of oracle/dense.py).
Every device result is held to the same bar against both: eps <= 2e-2 of
the largest magnitude, and elementwise 1e-2 rms(R) + 2e-2 |R| plus the
rounding allowance of the bf16 path (gpu_common.allowance_full).
"""

from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from oracle import dense
from tests.gpu_common import (allowance_full, compare, magnitude_bounds, margins_report, margins_scope,
                              one_key_rows,
                              operand_rounding_bound, oracle_unit, output_rounding_bound, run_gpu, stored,
                              term_bound, zero_key_rows)

pytestmark = pytest.mark.gpu


def _full_compare(prob, tag):
    """Every output of every unit against the forward definition, the
    stored-Y reverse procedure and the exact dense VJP."""
    got = run_gpu(prob)
    w = prob.w
    errs = {}
    for b in range(w.B):
        for h in range(w.H):
            ref = oracle_unit(prob, b, h, exact_vjp=True)
            bounds = magnitude_bounds(prob, b, h)
            A = None if w.mask == W.MASK_NONE else prob.allowed(h)
            Q, K, V, G = (getattr(prob, x)[b, h] for x in "QKVG")
            # Rounding allowances of the bf16 path (both references).
            allow = allowance_full(Q, K, V, G, w.scale, A, stored(ref["O"], w.dtype), ref["L"], w.dtype)
            zq, zk = one_key_rows(A), zero_key_rows(A)
            if w.n <= 2:
                # One or two keys per row: dQ and dK are differences of two
                # terms; their rounding allowance (gpu_common.term_bound)
                # applies to the eps check as well.
                eq, ek = term_bound(Q, K, V, G, w.scale, A, w.dtype)
                allow = dict(allow, dQ=eq + allow.get("dQ", 0.0), dK=ek + allow.get("dK", 0.0))
            pairs = [("O", "O"), ("L", "L")]
            for g in ("dQ", "dK", "dV"):
                pairs += [(g, g), (g + "_det", g), (g, g + "_exact"), (g + "_det", g + "_exact")]
            for gname, rname in pairs:
                key = gname + "/" + rname
                e = compare(gname[:2] if gname != "L" else "L", got[gname][b, h], ref[rname], w.dtype,
                            (tag, b, h, key), bounds.get(gname[:2]), extra=allow.get(gname[:2]),
                            extra_eps=w.n <= 2, zero_rows={"dQ": zq, "dK": zk}.get(gname[:2]))
                errs[key] = max(errs.get(key, 0.0), e)
    print(tag, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    return errs


@pytest.mark.parametrize("name", ["f32_n256_d64", "f32_causal_n1000_d80"])
def test_fp32_workloads_full(name):
    _full_compare(W.generate(name), name)


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


def _full_size_compare(prob, n_edge=256, n_rand=48, seed=0):
    """Full-size run in the benchmark's launch configuration.

    O and L: every row of every unit.  dQ: the first and last ``n_edge``
    rows plus ``n_rand`` random rows of every unit; dK, dV: the same choice
    of key columns.  Both gradient references, both dQ paths.  The oracle
    work of the units runs on a thread pool (one-thread BLAS each).
    """
    from concurrent.futures import ThreadPoolExecutor

    import threadpoolctl

    w = prob.w
    n = w.n
    print(f"[{w.name}] device run", flush=True)
    got = run_gpu(prob)
    print(f"[{w.name}] oracle on {w.B * w.H} units", flush=True)
    causal = prob.allowed(0) if w.mask == W.MASK_CAUSAL else None
    rng = np.random.default_rng(seed)
    picks = {}
    for b in range(w.B):
        for h in range(w.H):
            picks[(b, h)] = [np.unique(np.concatenate([np.arange(min(n_edge, n)), np.arange(max(0, n - n_edge), n),
                                                       rng.choice(n, n_rand, replace=False)])) for _ in range(2)]

    def unit(bh):
        b, h = bh
        errs = {}

        def check(name, g, r, tag, extra=None, zero_rows=None):
            errs[name] = max(errs.get(name, 0.0), compare(name[:2] if name != "L" else "L", g, r, w.dtype, tag,
                                                          extra=extra, zero_rows=zero_rows))

        Q, K, V, G = (getattr(prob, x)[b, h] for x in "QKVG")
        Ah = None if w.mask == W.MASK_NONE else (causal if causal is not None else prob.allowed(h))
        Y, _, _, L = dense.forward(Q, K, V, w.scale, Ah)
        tag = (w.name, b, h)
        if Ah is None:
            def A_rows(r):
                return np.ones((len(r), n), bool)
        else:
            def A_rows(r):
                return Ah if len(r) == n else Ah[r]
        E_O = output_rounding_bound(Q, K, V, L, w.scale, A_rows, w.dtype)
        check("O", got["O"][b, h], Y, tag, E_O)
        check("L", got["L"][b, h], L, tag)
        rows, cols = picks[bh]
        Ys = stored(Y, w.dtype)
        allow = operand_rounding_bound(Q, K, V, G, Ys, L, E_O, w.scale, A_rows, rows, cols, w.dtype)
        zq = None if Ah is None else one_key_rows(A_rows(rows))
        for ref_name, Yd in (("stored", Ys), ("exact", Y)):
            dQ, dK, dV = dense.grads_sampled(Q, K, V, w.scale, A_rows, G, L, Yd, rows, cols)
            for sfx in ("", "_det"):
                check("dQ" + sfx + "/" + ref_name, got["dQ" + sfx][b, h][rows], dQ, tag, allow.get("dQ"), zq)
                check("dK" + sfx + "/" + ref_name, got["dK" + sfx][b, h][cols], dK, tag, allow.get("dK"))
                check("dV" + sfx + "/" + ref_name, got["dV" + sfx][b, h][cols], dV, tag, allow.get("dV"))
        # Whole-tensor invariants at any size: sum_j dK_j = 0, sum_j dV_j = sum_i dO_i.
        for sfx in ("", "_det"):
            sdk = got["dK" + sfx][b, h].sum(0)
            assert np.abs(sdk).max() <= 2e-2 * np.abs(got["dK" + sfx][b, h]).sum(0).max() + 1e-6, tag
            sdv, sg = got["dV" + sfx][b, h].sum(0), G.astype(np.float64).sum(0)
            assert np.abs(sdv - sg).max() <= 2e-2 * np.abs(G).sum(0).max(), tag
        return errs

    import os

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    total = {}
    with margins_scope(), threadpoolctl.threadpool_limits(1, user_api="blas"), ThreadPoolExecutor(workers) as ex:
        for errs in ex.map(unit, list(picks)):
            for k_, v_ in errs.items():
                total[k_] = max(total.get(k_, 0.0), v_)
        print(w.name, {k: f"{v:.2e}" for k, v in total.items()}, flush=True)
        print(margins_report(w.name), flush=True)
    return total


def test_bf16_noncausal_b4h16_n4096_full_size():
    _full_size_compare(W.generate("bf16_b4h16_n4096_d128"))


def test_bf16_causal_h32_n16384_full_size():
    _full_size_compare(W.generate("bf16_causal_h32_n16384_d128"))


def test_bf16_bitmask_b2h8_n8192_full_size():
    _full_size_compare(W.generate("bf16_bitmask_b2h8_n8192_d64v128"))


@pytest.mark.parametrize("name", ["bf16_b4h16_n4096_d128", "bf16_causal_h32_n16384_d128",
                                  "bf16_bitmask_b2h8_n8192_d64v128"])
def test_bf16_workloads_reduced_full_compare(name):
    """Same recipe with fewer heads and n = 1000 (ragged tail): compare everything."""
    prob = W.generate(name, heads=2, n=1000)
    _full_compare(prob, name + "_reduced")


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
