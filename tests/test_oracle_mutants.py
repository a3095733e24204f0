"""Plant one plausible mistake at a time in a copy of the oracle and check
that the pins catch it (CPU only).  The real oracle is never modified."""

import inspect
import types

import pytest

from oracle import dense, tiled, tilemap
from tests import oracle_pins as P

# (module, exact source fragment, replacement, what the mistake is)
MUTANTS = [
    (dense, "dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))", "dS = P * dP", "dropped -rowsum term"),
    (dense, "dQ = c * (dS @ K)", "dQ = c * (dS @ Q)", "wrong operand in dQ"),
    (dense, "dK = c * (dS.T @ Q)", "dK = (dS.T @ Q)", "dropped scale in dK"),
    (dense, "dV = P.T @ G", "dV = P @ G", "untransposed P in dV"),
    (dense, "dK = c * (dS.T @ Q)", "dK = -c * (dS.T @ Q)", "wrong sign in dK"),
    (dense, "S = c * (Q[r0:r1] @ K.T)", "S = (Q[r0:r1] @ K.T)", "dropped scale in scores"),
    (dense, "Y[r0:r1] = (E @ V) / li[:, None]", "Y[r0:r1] = (E @ V)", "missing normalisation"),
    (dense, "S = np.where(A, S, -np.inf)", "S = S", "mask ignored"),
    (dense, "return Y, m, ell, m + np.log(ell)", "return Y, m, ell, m + ell", "L without log"),
    (dense, "E = np.exp(S - mi[:, None])", "E = np.exp(S)", "no max subtraction"),
    (tiled, "return M, a * l + a2 * l2, a[:, None] * z + a2[:, None] * z2",
     "return M, l + l2, a[:, None] * z + a2[:, None] * z2", "denominator not rescaled"),
    (tiled, "return M, a * l + a2 * l2, a[:, None] * z + a2[:, None] * z2",
     "return M, a * l + a2 * l2, z + a2[:, None] * z2", "accumulator not rescaled"),
    (tiled, "M = np.maximum(m, m2)", "M = m2", "running max from the current block only"),
    (tiled, "state |= has", "state = has", "skipped block resets the summary"),
    (tiled, "gam = P * (G @ V[t0:t1].T - delta[:, None])", "gam = P * (G @ V[t0:t1].T)", "dropped delta"),
    (tiled, "dV[t0:t1] += P.T @ G", "dV[t0:t1] += gam.T @ G", "gamma instead of p in dV"),
    (tiled, "dQ += c * (gam @ K[t0:t1])", "dQ += c * (P @ K[t0:t1])", "p instead of gamma in dQ"),
    (tiled, "delta = (G * Y).sum(axis=1)", "delta = (G * G).sum(axis=1)", "delta from G only"),
    (tilemap, "elif k0 + Bk <= nk and blk.all():", "elif blk.all():", "key tail classified full"),
    (tilemap, "elif k_hi <= q_lo and k_hi < n:", "elif k_hi <= q_hi and k_hi < n:", "diagonal tile classified full"),
]

CHECKS = [
    lambda d, t, m: P.check_closed_forms(d),
    lambda d, t, m: P.check_golden(d, t),
    lambda d, t, m: P.check_library_softmax(d),
    lambda d, t, m: P.check_invariants(d),
    lambda d, t, m: P.check_block_independence(d, t),
    lambda d, t, m: P.check_wide_scores(d, t),
    lambda d, t, m: P.check_dense_vjp_fd(d),
    lambda d, t, m: P.check_tiled_reverse_fd(t),
    lambda d, t, m: P.check_reverse_routes_agree(d, t),
    lambda d, t, m: P.check_grad_identities(d, t),
    lambda d, t, m: P.check_tilemap(m),
]


def mutate(mod, old, new):
    src = inspect.getsource(mod)
    assert src.count(old) == 1, (mod.__name__, old)
    m = types.ModuleType(mod.__name__ + "_mutant")
    m.__dict__["__builtins__"] = __builtins__
    exec(compile(src.replace(old, new), mod.__file__ + "<mutant>", "exec"), m.__dict__)
    return m


@pytest.mark.parametrize("mod,old,new,what", MUTANTS, ids=[m[3] for m in MUTANTS])
def test_pins_catch_planted_mistake(mod, old, new, what):
    d = mutate(dense, old, new) if mod is dense else dense
    t = mutate(tiled, old, new) if mod is tiled else tiled
    tm = mutate(tilemap, old, new) if mod is tilemap else tilemap
    caught = []
    for chk in CHECKS:
        try:
            chk(d, t, tm)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(chk)
            break
    assert caught, f"no pin caught: {what}"
