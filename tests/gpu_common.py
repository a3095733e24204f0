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
BF16_ABS = 1e-2  # elementwise |X-R| <= 1e-2 rms(R) + 2e-2 |R|
L_TOL = {"f32": 1e-5, "bf16": 1e-4}  # |L - L_ref| <= tol * max(1, |L_ref|)
# Term-size factor of the one- and two-key problems (see term_bound).
TERM_U = {"f32": 2.0 ** -20, "bf16": 2.0 ** -7}
# Relative rounding of O as stored, which D_i = <dO_i, O_i> inherits on the
# device (half an ulp, with room for the fp32 sum): see _d_terms.
STORE_U = {"f32": 2.0 ** -23, "bf16": 2.0 ** -8}
# Standard deviations allowed for sums of independent roundings (Hoeffding:
# exceeded with probability at most 2 exp(-32) = 2.5e-14 per element).
ROUND_LAMBDA = 8.0

# Worst margins seen by compare() in this process, per (tensor, dtype):
# eps / tol and, for bf16, the largest elementwise |X - R| / bound.
MARGINS: dict = {}


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
        dq, dk, dv = E.bwd(q, k, v, o, g, L, w.scale, w.mask, m, deterministic=False)
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
    ``allow``: the bf16 operand rounding allowances (allowance_full).
    """
    w = prob.w
    Q, K, V, G = (getattr(prob, n)[b, h] for n in ("Q", "K", "V", "G"))
    A = None if w.mask == W.MASK_NONE else prob.allowed(h)
    Y, m, ell, L = dense.forward(Q, K, V, w.scale, A)
    out = {"O": Y, "L": L}
    if want_bwd:
        out["allow"] = allowance_full(Q, K, V, G, w.scale, A, stored(Y, w.dtype), L, w.dtype)
        dQ, dK, dV = tiled.reverse(Q, K, V, w.scale, A, w.n, stored(Y, w.dtype), m, ell, G)
        out.update(dQ=dQ, dK=dK, dV=dV)
        if exact_vjp:
            dQ, dK, dV = dense.vjp(Q, K, V, w.scale, A, G)
            out.update(dQ_exact=dQ, dK_exact=dK, dV_exact=dV)
    return out


# When the whole exact tensor is zero (dQ and dK with one allowed key per
# row: p_ij = 1 and dP_ij - D_i = 0 exactly), the relative error is
# undefined; the check then bounds |X| by a fraction of the largest
# magnitude the output can have for these inputs.
ZERO_REF_FRAC = {"f32": 1e-7, "bf16": 1e-4}


def magnitude_bounds(prob: W.Problem, b: int, h: int) -> dict:
    """Upper bounds of |output| from the inputs: |gamma_ij| <= 2 p_ij max|G| max|V| v."""
    w = prob.w
    mq, mk, mv, mg = (float(np.abs(getattr(prob, x)[b, h]).max(initial=0.0)) for x in "QKVG")
    return {"O": mv, "dV": mg * w.n, "dQ": 2 * abs(w.scale) * mk * mg * mv * w.v,
            "dK": 2 * abs(w.scale) * mq * mg * mv * w.v * w.n}


def term_bound(Q, K, V, G, scale, A, dtype):
    """Rounding allowance of dQ and dK for problems whose rows hold one or two keys.

    There dQ_i and dK_j are differences of the two terms p_ij (dP_ij - D_i)
    (with two keys, dS_i0 = -dS_i1 up to D_i), so the rounding of those terms
    is large relative to the result.  The device forms D_i = <dO_i, O_i> from
    O as stored (bf16: each element within half an ulp, 2^-9 relative, of the
    exact output) and rounds P and dS to bf16 before the products with K and
    Q.  The allowance is TERM_U[dtype] times the size of the summed terms,
    T(dQ_i) = |c| sum_j P_ij (|dP_ij| + sum_a |dO_ia O_ia|) |K_j| and dK alike
    with |Q_i|: 2^-7 covers two bf16 roundings of each term, 2^-20 a few fp32
    roundings of the length-v dot products.  Returns (E_dQ, E_dK) elementwise.
    """
    Q, K, V, G = (np.asarray(x, np.float64) for x in (Q, K, V, G))
    A = np.ones((Q.shape[0], K.shape[0]), bool) if A is None else np.asarray(A, bool)
    S = np.where(A, scale * (Q @ K.T), -np.inf)
    m = S.max(axis=1, keepdims=True)
    P = np.where(A, np.exp(S - m), 0.0)
    P /= P.sum(axis=1, keepdims=True)
    Y = P @ V
    Dt = np.sum(np.abs(G) * np.abs(Y), axis=1)
    Wm = P * (np.abs(G @ V.T) + Dt[:, None])
    u = TERM_U[dtype]
    return u * abs(scale) * (Wm @ np.abs(K)), u * abs(scale) * (Wm.T @ np.abs(Q))


def _d_terms(G, Yd, E_O, dtype):
    """Bound of |D_dev,i - delta_i| per row.

    The device forms D_i = <dO_i, O_i> from its own O as stored.  That O
    differs from the reference's Y by the forward's rounding (at most E_O,
    allowance_full's O allowance) plus the output's own rounding (u
    |Y|, u = STORE_U[dtype]), so |D_dev,i - delta_i| <= sum_a |dO_ia| (E_O,ia
    + u |Y_ia|) whether delta_i is taken on the exact Y or on Y as stored.
    """
    u = STORE_U[dtype]
    E = u * np.abs(Yd) if E_O is None else E_O + u * np.abs(Yd)
    return np.sum(np.abs(G) * E, axis=1)


def _allow(P, Pw, dS, T, V, G, K, Q, scale, rows_only=False):
    lam, c = ROUND_LAMBDA * 2.0 ** -8, abs(scale)
    out = {"O": lam * np.sqrt(Pw ** 2 @ V ** 2),
           # D enters dQ_i as -c D_i sum_j P_ij K_j (one value per row).
           "dQ": lam * c * np.sqrt(dS ** 2 @ K ** 2) + c * T[:, None] * np.abs(P @ K)}
    if not rows_only:
        out["dV"] = lam * np.sqrt((Pw ** 2).T @ G ** 2)
        # ... and dK_j as -c sum_i P_ij D_i Q_i: independent rows, LAMBDA deviations.
        out["dK"] = lam * c * (np.sqrt((dS ** 2).T @ Q ** 2) + np.sqrt((P * T[:, None]).T ** 2 @ Q ** 2))
    return out


def allowance_full(Q, K, V, G, scale, A, Yd, L, dtype, Z=None, p8=0):
    """Elementwise allowances of the bf16 path for every row and column of a
    small unit (bf16 only; {} for fp32).

    Rounding of the MFMA operands: the bf16 path rounds P and dS to bf16
    (round to nearest even, relative error at most u = 2^-8) before the
    products P V, P^T dO, dS K and dS^T Q, and accumulates in fp32.  An
    output is then off by sum_t e_t x_t over its terms x_t (P_ij V_j,
    P_ij dO_i, c dS_ij K_j, c dS_ij Q_i) with |e_t| <= u; the rounding errors
    of different terms are independent and centred, so by Hoeffding's
    inequality the sum stays below ROUND_LAMBDA u sqrt(sum_t x_t^2) except
    with probability 2 exp(-LAMBDA^2 / 2) per element.  A cancellation-heavy
    element (terms much larger than their sum) needs this beyond 1e-2 rms(R)
    + 2e-2 |R|; a wrong or missing tile moves it by the terms themselves.

    D from the device's own O (_d_terms): dQ_i moves by -c (D_dev,i -
    delta_i) sum_j P_ij K_j, dK_j by -c sum_i P_ij (D_dev,i - delta_i) Q_i.

    With dropout's keep mask Z the weights that multiply V and dO are
    Pw = P Z 256 / (256 - p8), and dS_ij = P_ij (Z_ij dP_ij 256 / (256 - p8)
    - D_i).  Rows without an allowed key have P = 0.  Yd: the forward output
    as stored; L: the logsumexp of every row.
    """
    if dtype != "bf16":
        return {}
    Q, K, V, G, Yd, L = (np.asarray(x, np.float64) for x in (Q, K, V, G, Yd, L))
    A = np.ones((Q.shape[0], K.shape[0]), bool) if A is None else np.asarray(A, bool)
    fin = np.isfinite(L)
    Lf = np.where(fin, L, 0.0)
    P = np.where(A & fin[:, None], np.exp(np.where(A, scale * (Q @ K.T), 0.0) - Lf[:, None]), 0.0)
    kz = np.ones_like(P) if Z is None else np.asarray(Z, np.float64) * (256.0 / (256 - p8))
    Pw = P * kz
    dS = P * (kz * (G @ V.T) - np.sum(G * Yd, axis=1)[:, None])
    E_O = ROUND_LAMBDA * 2.0 ** -8 * np.sqrt(Pw ** 2 @ V ** 2)
    return _allow(P, Pw, dS, _d_terms(G, Yd, E_O, dtype), V, G, K, Q, scale)


def output_rounding_bound(Q, K, V, L, scale, A_rows, dtype, row_chunk=1024, Z_rows=None, p8=0):
    """allowance_full's O allowance for every row of a large unit, in row
    chunks (with dropout: the weights P Z / keep, Z_rows(r) the keep mask's
    rows)."""
    if dtype != "bf16":
        return None
    Q, K, V, L = (np.asarray(x, np.float64) for x in (Q, K, V, L))
    n = Q.shape[0]
    out = np.empty((n, V.shape[1]))
    V2 = V ** 2
    for r0 in range(0, n, row_chunk):
        r = np.arange(r0, min(n, r0 + row_chunk))
        A = A_rows(r)
        P = np.where(A, np.exp(np.where(A, scale * (Q[r] @ K.T), 0.0) - L[r, None]), 0.0)
        if Z_rows is not None:
            P = P * Z_rows(r) * (256.0 / (256 - p8))
        out[r] = ROUND_LAMBDA * 2.0 ** -8 * np.sqrt(P ** 2 @ V2)
    return out


def operand_rounding_bound(Q, K, V, G, Yd, L, E_O, scale, A_rows, rows, cols, dtype, Z_r=None, Z_c=None, p8=0):
    """allowance_full's dQ allowance for sampled rows and dK, dV allowances
    for sampled key columns of a large unit.  E_O: the O allowance of every
    row (output_rounding_bound).  With dropout Z_r = Z[rows], Z_c = Z[:, cols]
    (allowance_full's weights and dS).  Returns {dQ, dK, dV}."""
    if dtype != "bf16":
        return {}
    Q, K, V, G, Yd, L = (np.asarray(x, np.float64) for x in (Q, K, V, G, Yd, L))
    n = Q.shape[0]
    delta = np.sum(G * Yd, axis=1)
    T = _d_terms(G, Yd, E_O, dtype)
    rows, cols = np.asarray(rows), np.asarray(cols)
    kr = 1.0 if Z_r is None else Z_r * (256.0 / (256 - p8))
    kc = 1.0 if Z_c is None else Z_c * (256.0 / (256 - p8))
    Ar = A_rows(rows)
    Pr = np.where(Ar, np.exp(np.where(Ar, scale * (Q[rows] @ K.T), 0.0) - L[rows, None]), 0.0)
    dSr = Pr * (kr * (G[rows] @ V.T) - delta[rows, None])
    out = {"dQ": _allow(Pr, Pr * kr, dSr, T[rows], V, G, K, Q, scale, rows_only=True)["dQ"]}
    Ac = A_rows(np.arange(n))[:, cols]
    Pc = np.where(Ac, np.exp(np.where(Ac, scale * (Q @ K[cols].T), 0.0) - L[:, None]), 0.0)
    dSc = Pc * (kc * (G @ V[cols].T) - delta[:, None])
    lam, c = ROUND_LAMBDA * 2.0 ** -8, abs(scale)
    out["dV"] = lam * np.sqrt(((Pc * kc) ** 2).T @ G ** 2)
    out["dK"] = lam * c * (np.sqrt((dSc ** 2).T @ Q ** 2) + np.sqrt((Pc * T[:, None]).T ** 2 @ Q ** 2))
    return out


def one_key_rows(A):
    """Rows whose dQ is exactly zero by the mask: a single allowed key gives
    p_ij = 1 and dP_ij - D_i = 0 (None: every key allowed; the caller knows
    whether there is only one)."""
    if A is None:
        return None
    return np.asarray(A, bool).sum(axis=1) == 1


def zero_key_rows(A):
    """Keys whose dK is exactly zero by the mask: every row that allows the
    key allows no other, so every dS_ij of the key is zero (this includes
    keys no row allows)."""
    if A is None:
        return None
    A = np.asarray(A, bool)
    single = A.sum(axis=1) == 1
    return ~(A & ~single[:, None]).any(axis=0)


def _record(name, dtype, eps_ratio, el_ratio, pure_ratio=0.0, over=0, count=0):
    key = (name, dtype)
    e0, w0, p0, o0, c0 = MARGINS.get(key, (0.0, 0.0, 0.0, 0, 0))
    MARGINS[key] = (max(e0, eps_ratio), max(w0, el_ratio), max(p0, pure_ratio), o0 + over, c0 + count)


class margins_scope:
    """Collect the margins of one block of comparisons on their own (they
    are merged into the session's afterwards)."""

    def __enter__(self):
        self.saved = dict(MARGINS)
        MARGINS.clear()
        return self

    def __exit__(self, *exc):
        mine = dict(MARGINS)
        MARGINS.clear()
        MARGINS.update(self.saved)
        for (n, d), (e, w, p, o, c) in mine.items():
            _record(n, d, e, w, p, o, c)
        return False


def margins_report(tag="") -> str:
    """One line per (tensor, dtype): the worst eps / tol, the worst elementwise
    ratio to the asserted bound, and to 1e-2 rms(R) + 2e-2 |R| alone (with the
    number of elements above that bare bound, of all compared)."""
    return "\n".join(f"margin {tag} {n} {d}: eps/tol {e:.3f} elementwise {w:.3f} "
                      f"bare {p:.3f} ({o} of {c} elements above the bare bound)"
                      for (n, d), (e, w, p, o, c) in sorted(MARGINS.items()))


def compare(name: str, got: np.ndarray, ref: np.ndarray, dtype: str, tag="", bound=None,
            elementwise=True, extra=None, extra_eps=False, zero_rows=None):
    """Assert the tolerance of the dtype; returns the max relative error.

    fp32: eps = max|X - R| / max|R| <= 1e-5.  bf16: eps <= 2e-2 and, when
    ``elementwise``, |X - R| <= 1e-2 rms(R) + 2e-2 |R| per element, the
    absolute term taken at the scale of the tensor ("1e-2 absolute at
    unit-scale outputs").  Every row is held to these bars, including rows
    whose exact value is zero (a key no row allows, a row with one allowed
    key): their residuals must stay at the rounding scale of the tensor.  A
    tensor that is zero altogether is bounded by ZERO_REF_FRAC of ``bound``,
    the largest magnitude the output can have.  ``extra`` (elementwise,
    broadcastable) is an additional rounding allowance of the elementwise
    check (allowance_full), and of the eps check too with ``extra_eps``
    (term_bound, one- and two-key problems).  ``zero_rows`` marks rows whose
    exact value is zero by the mask (one_key_rows): they are compared with
    exact zeros, not with the float64 oracle's rounding residue of zero.  L: |L - L_ref| <= tol max(1,
    |L_ref|), with the same infinities.
    """
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if zero_rows is not None and np.any(zero_rows):
        ref = ref.copy()
        ref[np.asarray(zero_rows, bool)] = 0.0
    if name == "L":
        fin = np.isfinite(ref)
        assert np.array_equal(fin, np.isfinite(got)), (tag, "L finiteness differs")
        assert np.array_equal(got[~fin], ref[~fin]), (tag, "L infinities differ")
        err = np.abs(got[fin] - ref[fin]) / np.maximum(1.0, np.abs(ref[fin]))
        e = float(err.max(initial=0.0))
        _record(name, dtype, e / L_TOL[dtype], 0.0)
        assert e <= L_TOL[dtype], (tag, name, e)
        return e
    assert np.all(np.isfinite(got)), (tag, name, "non-finite output")
    den = float(np.abs(ref).max(initial=0.0))
    if den == 0.0:
        assert bound is not None, (tag, name, "zero reference needs a magnitude bound")
        e0 = float(np.abs(got).max(initial=0.0)) / max(bound, 1e-300)
        _record(name + "(zero)", dtype, e0 / ZERO_REF_FRAC[dtype], 0.0)
        assert e0 <= ZERO_REF_FRAC[dtype], (tag, name, "zero reference", e0)
        return 0.0
    err = np.abs(got - ref)
    ex = 0.0 if extra is None else np.broadcast_to(np.asarray(extra, np.float64), err.shape)
    e = float(np.maximum(err - (ex if extra_eps else 0.0), 0.0).max(initial=0.0) / den)
    tol = F32_REL if dtype == "f32" else BF16_REL
    el = pure = 0.0
    over = 0
    if dtype == "bf16" and elementwise:
        rms = float(np.sqrt(np.mean(ref * ref)))
        bare = BF16_ABS * rms + BF16_REL * np.abs(ref)
        ratio = err / np.maximum(bare + ex, 1e-300)
        el = float(ratio.max(initial=0.0))
        bare_ratio = err / np.maximum(bare, 1e-300)
        pure = float(bare_ratio.max(initial=0.0))
        over = int((bare_ratio > 1.0).sum())
    _record(name, dtype, e / tol, el, pure, over, err.size)
    assert e <= tol, (tag, name, e)
    assert el <= 1.0, (tag, name, "elementwise", int((ratio > 1.0).sum()), el)
    return e
