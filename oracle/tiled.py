"""Key-block procedure of exact tiled softmax attention, in float64.

Test infrastructure only (see the package docstring).

Follows "Exact tiled softmax attention with block-recomputed vector-Jacobian
products" (alphabetamath page): key blocks J_t = {(t-1)b+1, ..., min(tb, n)}
(here 0-based: [t b, min((t+1) b, n))), a per-row summary that starts empty,
per-block summaries over I = J_t intersect A_i that are skipped when I is
empty, and a merge of summaries.

The page lists "Summary state and merge convention" as a section heading
but its body is missing, so the summary and merge are read from the running
max / denominator / accumulator update the other pages describe
(HarshvardhanJ/FlashAttention README, chunked forward; trentorch exercise,
the hint; maitreyasuin post, the tiled forward):

    Sigma_i(I) = (m_I, l_I, z_I)
        m_I = max_{j in I} s_ij
        l_I = sum_{j in I} exp(s_ij - m_I)
        z_I = sum_{j in I} exp(s_ij - m_I) V_j
    (m, l, z) * (m', l', z') = (M, e^{m-M} l + e^{m'-M} l', e^{m-M} z + e^{m'-M} z')
        with M = max(m, m')
    the empty summary is the identity of *.

Computation is vectorised over query rows; the Python loop runs over the
key blocks, in the page's order.
"""

from __future__ import annotations

import numpy as np


def _block_summary(S_blk, A_blk, V_blk):
    """Sigma_i(J_t intersect A_i) for every row; rows with empty I get has=False."""
    has = A_blk.any(axis=1)
    Sm = np.where(A_blk, S_blk, -np.inf)
    mI = np.where(has, Sm.max(axis=1, initial=-np.inf), 0.0)
    E = np.where(A_blk, np.exp(Sm - mI[:, None]), 0.0)
    lI = E.sum(axis=1)
    zI = E @ V_blk
    return has, mI, lI, zI


def _merge(m, l, z, m2, l2, z2):
    """The merge * of two nonempty summaries."""
    M = np.maximum(m, m2)
    a, a2 = np.exp(m - M), np.exp(m2 - M)
    return M, a * l + a2 * l2, a[:, None] * z + a2[:, None] * z2


def forward(Q, K, V, c, allowed, b):
    """Forward procedure, steps 1-4.

    Q [n,d], K [nk,d], V [nk,v]; ``allowed`` bool [n,nk] (None = all keys);
    ``b`` the key-block size.  Returns float64 Y [n,v], m [n], l [n] and
    L = m + ln l [n] (the logsumexp form of the retained statistics).
    """
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    n = Q.shape[0]
    nk = K.shape[0]
    A = np.ones((n, nk), bool) if allowed is None else np.asarray(allowed, bool)
    if not A.any(axis=1).all():
        raise ValueError("allowed-key sets must be nonempty (precondition)")
    # Step 1: every row starts from the empty summary.
    state = np.zeros(n, dtype=bool)
    m = np.zeros(n)
    ell = np.zeros(n)
    z = np.zeros((n, V.shape[1]))
    # Step 2: stream the key blocks.
    for t0 in range(0, nk, b):
        t1 = min(t0 + b, nk)
        S_blk = c * (Q @ K[t0:t1].T)
        has, mI, lI, zI = _block_summary(S_blk, A[:, t0:t1], V[t0:t1])
        copy = has & ~state  # current summary empty: copy
        merge = has & state  # otherwise merge with *
        m[copy], ell[copy], z[copy] = mI[copy], lI[copy], zI[copy]
        if merge.any():
            Mm, lm, zm = _merge(m[merge], ell[merge], z[merge],
                                mI[merge], lI[merge], zI[merge])
            m[merge], ell[merge], z[merge] = Mm, lm, zm
        state |= has  # rows with empty I are skipped and left unchanged
    # Step 3: normalise once; keep m and l.
    Y = z / ell[:, None]
    return Y, m, ell, m + np.log(ell)


def reverse(Q, K, V, c, allowed, b, Y, m, ell, G):
    """Reverse procedure: block-recomputed vector-Jacobian product.

    Given the forward's Y, m, l and the upstream G, returns dQ, dK, dV.
    delta_i = sum_a G_ia Y_ia; for every block J_t and j in J_t intersect A_i:
    p_ij = exp(s_ij - m_i) / l_i, gamma_ij = p_ij (sum_a G_ia V_ja - delta_i),
    dQ_i += c gamma_ij K_j, dK_j += c gamma_ij Q_i, dV_j += p_ij G_i.
    Only one block of scores exists at a time.
    """
    Q, K, V, Y, G = (np.asarray(a, dtype=np.float64) for a in (Q, K, V, Y, G))
    m, ell = np.asarray(m, np.float64), np.asarray(ell, np.float64)
    n, nk = Q.shape[0], K.shape[0]
    A = np.ones((n, nk), bool) if allowed is None else np.asarray(allowed, bool)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    delta = (G * Y).sum(axis=1)
    for t0 in range(0, nk, b):
        t1 = min(t0 + b, nk)
        A_blk = A[:, t0:t1]
        S_blk = c * (Q @ K[t0:t1].T)
        P = np.where(A_blk, np.exp(np.where(A_blk, S_blk, 0.0) - m[:, None]) / ell[:, None], 0.0)
        gam = P * (G @ V[t0:t1].T - delta[:, None])
        dQ += c * (gam @ K[t0:t1])
        dK[t0:t1] += c * (gam.T @ Q)
        dV[t0:t1] += P.T @ G
    return dQ, dK, dV
