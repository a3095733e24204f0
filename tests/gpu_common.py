"""Helpers shared by the GPU parity tests: upload a generated problem,
run the HIP path through the binding, evaluate the float64 oracle, compare."""

from __future__ import annotations

import numpy as np
import torch

import workloads as W
from oracle import dense, tiled

DEV = "cuda:0"

# Tolerances (max relative error eps(X) = max|X-R| / max|R|).
F32_REL = 1e-5
BF16_REL = 2e-2
BF16_ABS = 1e-2  # elementwise |X-R| <= 1e-2 max|R| + 2e-2 |R|
L_TOL = {"f32": 1e-5, "bf16": 1e-4}  # |L - L_ref| <= tol * max(1, |L_ref|)


def to_dev(prob: W.Problem, name: str) -> torch.Tensor:
    if prob.w.dtype == "bf16":
        bits = prob.bits[name]
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(getattr(prob, name)).to(DEV)


def mask_dev(prob: W.Problem):
    if prob.mask_words is None:
        return None
    return torch.from_numpy(prob.mask_words.view(np.int32)).to(DEV)


def run_gpu(prob: W.Problem, want_bwd: bool = True):
    """Forward and backward (both dQ paths) on the device; float64 numpy results.

    Keys dQ/dK/dV come from the atomic path, dQ_det/dK_det/dV_det from the
    deterministic (query-tile-outer dQ) path.
    """
    import exact_tiled_attention_attn_amd as E

    w = prob.w
    q, k, v, g = (to_dev(prob, n) for n in ("Q", "K", "V", "G"))
    m = mask_dev(prob)
    o, L = E.fwd(q, k, v, w.scale, w.mask, m)
    out = {"O": o, "L": L}
    if want_bwd:
        dq, dk, dv = E.bwd(q, k, v, o, g, L, w.scale, w.mask, m)
        out.update(dQ=dq, dK=dk, dV=dv)
        dq, dk, dv = E.bwd(q, k, v, o, g, L, w.scale, w.mask, m, deterministic=True)
        out.update(dQ_det=dq, dK_det=dk, dV_det=dv)
    torch.cuda.synchronize()
    return {k_: t.float().cpu().numpy().astype(np.float64) for k_, t in out.items()}


def stored(Y: np.ndarray, dtype: str) -> np.ndarray:
    """The forward output as the device stores it (RNE to the output dtype)."""
    if dtype == "bf16":
        return W.round_bf16(np.asarray(Y, np.float32)).astype(np.float64)
    return np.asarray(Y, np.float32).astype(np.float64)


def oracle_unit(prob: W.Problem, b: int, h: int, want_bwd: bool = True, exact_vjp: bool = False):
    """Float64 oracle for one (batch, head) unit.

    Forward: the dense definition.  Gradients: the reverse procedure with
    delta_i = <G_i, Y_i> taken on the forward output as stored in the output
    dtype (the procedure consumes the forward run's Y), one key block.  With
    ``exact_vjp`` also the exact dense VJP (rowsum form) as ``*_exact``.
    """
    w = prob.w
    Q, K, V, G = (getattr(prob, n)[b, h] for n in ("Q", "K", "V", "G"))
    A = None if w.mask == W.MASK_NONE else prob.allowed(h)
    Y, m, ell, L = dense.forward(Q, K, V, w.scale, A)
    out = {"O": Y, "L": L}
    if want_bwd:
        dQ, dK, dV = tiled.reverse(Q, K, V, w.scale, A, w.n, stored(Y, w.dtype), m, ell, G)
        out.update(dQ=dQ, dK=dK, dV=dV)
        if exact_vjp:
            dQ, dK, dV = dense.vjp(Q, K, V, w.scale, A, G)
            out.update(dQ_exact=dQ, dK_exact=dK, dV_exact=dV)
    return out


# When the exact result is zero (e.g. dQ = dK = 0 for a single allowed key)
# the relative error is undefined; the check then bounds |X| by a fraction of
# the largest magnitude the output can have for these inputs.
ZERO_REF_FRAC = {"f32": 1e-7, "bf16": 1e-4}


def magnitude_bounds(prob: W.Problem, b: int, h: int) -> dict:
    """Upper bounds of |output| from the inputs: |gamma_ij| <= 2 p_ij max|G| max|V| v."""
    w = prob.w
    mq, mk, mv, mg = (float(np.abs(getattr(prob, x)[b, h]).max(initial=0.0)) for x in "QKVG")
    return {"O": mv, "dV": mg * w.n, "dQ": 2 * abs(w.scale) * mk * mg * mv * w.v,
            "dK": 2 * abs(w.scale) * mq * mg * mv * w.v * w.n}


def compare(name: str, got: np.ndarray, ref: np.ndarray, dtype: str, tag="", bound=None,
            elementwise=True, cond=1.0):
    """Assert the tolerance of the dtype; returns the max relative error.

    bf16: eps <= 2e-2 and, when ``elementwise``, |X - R| <= 1e-2 max|R| +
    2e-2 |R| per element.  The elementwise part is skipped for problems with
    at most two keys: there dS_i1 = -dS_i0 up to the term D_i = <dO_i, O_i>,
    which inherits the +-1 ulp ambiguity of the bf16-stored O.  ``cond``
    multiplies the relative bound for such one- and two-key problems, whose
    gradients are small differences of the two terms p_ij (dP_ij - D_i):
    the rounding of the length-v dot products dP_ij and D_i is then large
    relative to the result.
    """
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if bound is not None and name != "L" and ref.ndim == 2:
        # Rows whose exact value is zero (a row with a single allowed key has
        # dQ_i = 0; a key no row allows has dK_j = dV_j = 0) carry only
        # rounding noise: bound it by the output's magnitude bound.
        zero = np.abs(ref).max(axis=1) <= 1e-9 * bound
        if zero.any():
            e0 = float(np.abs(got[zero]).max(initial=0.0) / bound)
            assert e0 <= ZERO_REF_FRAC[dtype], (tag, name, "zero reference", e0)
            got, ref = got[~zero], ref[~zero]
            if ref.size == 0:
                return 0.0
    if name == "L":
        fin = np.isfinite(ref)
        assert np.array_equal(fin, np.isfinite(got)), (tag, "L finiteness differs")
        err = np.abs(got[fin] - ref[fin]) / np.maximum(1.0, np.abs(ref[fin]))
        e = float(err.max(initial=0.0))
        assert e <= L_TOL[dtype], (tag, name, e)
        return e
    assert np.all(np.isfinite(got)), (tag, name, "non-finite output")
    den = max(float(np.abs(ref).max(initial=0.0)), 1e-30)
    e = float(np.abs(got - ref).max(initial=0.0) / den)
    if dtype == "f32":
        assert e <= F32_REL * cond, (tag, name, e)
    else:
        assert e <= BF16_REL * cond, (tag, name, e)
        if not elementwise:
            return e
        # "1e-2 absolute at unit-scale outputs": the absolute term is 1e-2
        # of the tensor's scale max|R|.
        bound = BF16_ABS * den + BF16_REL * np.abs(ref)
        bad = np.abs(got - ref) > bound
        assert not bad.any(), (tag, name, int(bad.sum()), float((np.abs(got - ref) - bound).max()))
    return e
