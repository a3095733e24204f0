"""Dense float64 definition of masked scaled dot-product attention.

Test infrastructure only (see the package docstring).

Definition followed (alphabetamath page, "Inputs" and the reverse procedure;
the scale c multiplies <Q_i, K_j> as in the reverse procedure's dQ, dK
update; HarshvardhanJ/FlashAttention README, "Standard self-attention"):

    s_ij = c <Q_i, K_j>                  for j in A_i
    m_i  = max_{j in A_i} s_ij
    l_i  = sum_{j in A_i} exp(s_ij - m_i)
    Y_i  = sum_{j in A_i} exp(s_ij - m_i) V_j / l_i
    L_i  = m_i + ln l_i                  (logsumexp statistic; ob1 page, part 1)

Gradients with upstream G (= dY):

    P    = softmax over A_i of s_i.       (p_ij = 0 for j not in A_i)
    dV   = P^T G
    dP   = G V^T
    dS   = P o (dP - rowsum(P o dP))      (softmax Jacobian, written out)
    dQ   = c dS K,    dK = c dS^T Q

The rowsum(P o dP) form is used on purpose: it is the quantity the
D_i = dY_i . Y_i identity replaces (HarshvardhanJ/FlashAttention README,
backward section), so this route shares nothing with the tiled reverse.

Rows are independent in the definition; ``forward`` evaluates them in groups
of ``row_chunk`` rows only so that an n x n float64 array never has to exist
for large n.  No other blocking or reordering is done.
"""

from __future__ import annotations

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def _check_rows(allowed):
    if not np.all(allowed.any(axis=1)):
        raise ValueError("allowed-key sets must be nonempty (precondition)")


def forward(Q, K, V, c, allowed, row_chunk: int = 1024):
    """Y, m, l, L for one (batch, head) unit.

    Q [n,d], K [nk,d], V [nk,v]; ``allowed`` bool [n,nk] (None = all keys);
    nk = n for the square problems of the pages, any nk >= 1 otherwise.
    Returns float64 Y [n,v], m [n], l [n], L [n].
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    n = Q.shape[0]
    Y = np.empty((n, V.shape[1]))
    m = np.empty(n)
    ell = np.empty(n)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        A = np.ones((r1 - r0, K.shape[0]), bool) if allowed is None else allowed[r0:r1]
        _check_rows(A)
        S = c * (Q[r0:r1] @ K.T)
        S = np.where(A, S, -np.inf)
        mi = S.max(axis=1)
        E = np.exp(S - mi[:, None])  # exp(-inf) = 0 on masked entries
        li = E.sum(axis=1)
        Y[r0:r1] = (E @ V) / li[:, None]
        m[r0:r1] = mi
        ell[r0:r1] = li
    return Y, m, ell, m + np.log(ell)


def vjp(Q, K, V, c, allowed, G):
    """dQ, dK, dV of <G, Y> for one unit, materialising the n x n matrices."""
    Q, K, V, G = _f64(Q), _f64(K), _f64(V), _f64(G)
    A = np.ones((Q.shape[0], K.shape[0]), bool) if allowed is None else allowed
    _check_rows(A)
    S = np.where(A, c * (Q @ K.T), -np.inf)
    E = np.exp(S - S.max(axis=1, keepdims=True))
    P = E / E.sum(axis=1, keepdims=True)
    dV = P.T @ G
    dP = G @ V.T
    dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
    dQ = c * (dS @ K)
    dK = c * (dS.T @ Q)
    return dQ, dK, dV


def forward_rows(Q, K, V, c, allowed_rows, rows):
    """Y_i and L_i for the listed query rows only (same definition).

    ``allowed_rows`` is bool [len(rows), n] (None = all keys).
    """
    Q = _f64(Q)[np.asarray(rows)]
    A = allowed_rows
    Y, _, _, L = forward(Q, K, V, c, A, row_chunk=max(1, len(rows)))
    return Y, L


def grads_sampled(Q, K, V, c, allowed, G, L, Y, rows, cols):
    """dQ for sampled query rows and dK, dV for sampled key columns.

    Evaluates the reverse formulas of the alphabetamath page (reverse
    procedure: delta_i = <G_i, Y_i>, p_ij = exp(s_ij - L_i) with
    L_i = m_i + ln l_i, gamma_ij = p_ij(<G_i, V_j> - delta_i),
    dQ_i = c sum_j gamma_ij K_j, dK_j = c sum_i gamma_ij Q_i,
    dV_j = sum_i p_ij G_i) one output row or column at a time, using the
    row statistics L and the output Y of all rows (from ``forward``).

    ``allowed`` is a callable ``allowed(rows) -> bool [len(rows), n]``.
    """
    Q, K, V, G, L, Y = (_f64(a) for a in (Q, K, V, G, L, Y))
    n = Q.shape[0]
    delta = (G * Y).sum(axis=1)
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    # dQ rows: need p_ij over all keys j of row i.
    A = allowed(rows)
    S = np.where(A, c * (Q[rows] @ K.T), -np.inf)
    P = np.exp(S - L[rows, None])
    gam = P * (G[rows] @ V.T - delta[rows, None])
    dQ = c * (gam @ K)
    # dK, dV columns: need p_ij over all query rows i of key j.
    Acols = allowed(np.arange(n))[:, cols]
    Sc = np.where(Acols, c * (Q @ K[cols].T), -np.inf)
    Pc = np.exp(Sc - L[:, None])
    gc = Pc * (G @ V[cols].T - delta[:, None])
    dK = c * (gc.T @ Q)
    dV = Pc.T @ G
    return dQ, dK, dV
