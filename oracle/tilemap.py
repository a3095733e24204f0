"""Tile classification from the allowed-key sets (integer, exact).

Test infrastructure only (see the package docstring).

A blocked implementation visits (query tile, key tile) pairs.  The skip rule
of the alphabetamath page (forward step 2: a block whose intersection with
A_i is empty leaves the summary unchanged and is skipped) and the block
causal rule of the ob1 page (part 3: skip key blocks right of the query
block, mask only the diagonal block) generalise to this classification of a
tile of query rows R (the in-range rows of the tile) and key columns
C = [k0, k0 + Bk) (including any columns past n):

    EMPTY   (0)  no pair (i, j) in R x C with j < n and j in A_i
    FULL    (2)  every pair in R x C has j < n and j in A_i  (no masking needed)
    PARTIAL (1)  otherwise (some keys must be masked inside the tile)
"""

from __future__ import annotations

import numpy as np

EMPTY, PARTIAL, FULL = 0, 1, 2


def tile_map(allowed, Bq: int, Bk: int):
    """uint8 [ceil(n/Bq), ceil(n/Bk)] classification for one allowed matrix."""
    A = np.asarray(allowed, dtype=bool)
    n, nk = A.shape
    tq, tk = -(-n // Bq), -(-nk // Bk)
    out = np.empty((tq, tk), dtype=np.uint8)
    for a in range(tq):
        R = A[a * Bq:min(n, (a + 1) * Bq)]
        for t in range(tk):
            k0 = t * Bk
            blk = R[:, k0:min(nk, k0 + Bk)]
            if not blk.any():
                out[a, t] = EMPTY
            elif k0 + Bk <= nk and blk.all():
                out[a, t] = FULL
            else:
                out[a, t] = PARTIAL
    return out


def causal_tile_map(n: int, Bq: int, Bk: int):
    """Same classification for A_i = {j <= i}, from tile corners only."""
    tq, tk = -(-n // Bq), -(-n // Bk)
    out = np.empty((tq, tk), dtype=np.uint8)
    for a in range(tq):
        q_lo, q_hi = a * Bq, min(n, (a + 1) * Bq) - 1
        for t in range(tk):
            k_lo, k_hi = t * Bk, t * Bk + Bk - 1
            if k_lo > q_hi:
                out[a, t] = EMPTY
            elif k_hi <= q_lo and k_hi < n:
                out[a, t] = FULL
            else:
                out[a, t] = PARTIAL
    return out


def nonempty_tiles(tmap) -> int:
    return int((np.asarray(tmap) != EMPTY).sum())
