"""fp64 CPU oracle for the layer products next to attention (GEMM_NT, GEMM_NN,
GEMM_TN).

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and never by the product
package.

What is computed follows the three products Forge times for its MLP
("Forge: Building an LLM Training Framework from Scratch in C++ and Metal on
Apple Silicon", section "Results", GEMM table): the forward X W^T (weights
stored [out, in]), the input gradient dY W and the weight gradient dY^T X.
Each is the plain matrix product of the exact operand values, evaluated in
float64 by numpy's matmul (a library primitive standing for the definition
C_ij = sum_k A_ik B_kj; no splitting, no reordering beyond what the library
does).  Operands are the bf16 values the device receives, widened exactly.

Pins (tests/test_oracle_gemm.py): a pure-Python triple loop over the
definition on small shapes, for each operation, and closed forms (all-ones
operands give K everywhere; an identity operand returns the other one).
"""
from __future__ import annotations

import numpy as np

OPS = ("NT", "NN", "TN")


def gemm(op: str, A, B) -> np.ndarray:
    """C = A B^T (NT: A [M,K], B [N,K]), A B (NN: A [M,K], B [K,N]) or
    A^T B (TN: A [K,M], B [K,N]) in float64."""
    A64 = np.asarray(A, dtype=np.float64)
    B64 = np.asarray(B, dtype=np.float64)
    if op == "NT":
        return A64 @ B64.T
    if op == "NN":
        return A64 @ B64
    if op == "TN":
        return A64.T @ B64
    raise ValueError("unknown op %r" % (op,))


def gemm_rows(op: str, A, B, rows) -> np.ndarray:
    """Rows `rows` of gemm(op, A, B) only (for checking large products on a
    sample of output rows)."""
    A64 = np.asarray(A, dtype=np.float64)
    B64 = np.asarray(B, dtype=np.float64)
    rows = np.asarray(rows)
    if op == "NT":
        return A64[rows] @ B64.T
    if op == "NN":
        return A64[rows] @ B64
    if op == "TN":
        return A64[:, rows].T @ B64
    raise ValueError("unknown op %r" % (op,))


def abs_product(op: str, A, B) -> np.ndarray:
    """gemm(op, |A|, |B|): the sum of |a_ik b_kj| that bounds the rounding
    error of any fp32 evaluation order of C_ij."""
    return gemm(op, np.abs(np.asarray(A, dtype=np.float64)), np.abs(np.asarray(B, dtype=np.float64)))
