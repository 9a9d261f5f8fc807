"""Closed forms of causal attention for uniform queries (Q = 0), written from
the definition (test infrastructure; pinned against the oracle in
tests/test_oracle.py).

With Q = 0 every scaled score is 0, so query i attends with equal weight
P_ij = 1/(i+1) to keys j <= i, whatever the scale:
    O_i   = mean(V_0 .. V_i)                LSE_i = ln(i + 1)
    dV_j  = sum_{i >= j} dO_i / (i + 1)     dK    = s dS^T Q = 0
    dQ_i  = s/(i+1) sum_{j <= i} (dO_i . V_j - D_i) K_j,  D_i = dO_i . O_i
(dP_ij = dO_i . V_j and dS = P o (dP - D)).  Everything is O(T d) per head,
or O(i d) per sampled dQ row, so it checks any sequence length.
"""
from __future__ import annotations

import numpy as np


def uniform_q(K, V, dO, scale: float, dq_rows=None):
    """For [T, d] arrays of one head: O, LSE, dV (all rows) and dQ on the
    rows listed in dq_rows (all rows when None), in float64."""
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    T = V.shape[0]
    cnt = np.arange(1, T + 1, dtype=np.float64)[:, None]
    O = np.cumsum(V, axis=0) / cnt
    LSE = np.log(cnt[:, 0])
    dV = np.flip(np.cumsum(np.flip(dO / cnt, axis=0), axis=0), axis=0)
    rows = np.arange(T) if dq_rows is None else np.asarray(dq_rows)
    dQ = np.empty((len(rows), V.shape[1]))
    for n, i in enumerate(rows):
        Di = float(dO[i] @ O[i])
        coef = V[: i + 1] @ dO[i] - Di          # dP_ij - D_i for j <= i
        dQ[n] = scale / (i + 1) * (coef @ K[: i + 1])
    return O, LSE, dV, dQ
