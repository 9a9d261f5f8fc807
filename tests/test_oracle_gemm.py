"""Pins for the GEMM oracle (oracle/gemm.py), on the CPU: the definition
C_ij = sum_k op(A)_ik op(B)_kj written out as a pure-Python triple loop for
every operation, and closed forms.  A transposed operand or a swapped index
in the oracle fails the triple loop on these non-square shapes."""
import numpy as np
import pytest

from oracle import gemm as og


def _loop(op, An, Bn):
    A, B = An.tolist(), Bn.tolist()
    if op == "NT":
        M, K = An.shape
        N = Bn.shape[0]
        a = lambda i, k: A[i][k]
        b = lambda k, j: B[j][k]
    elif op == "NN":
        M, K = An.shape
        N = Bn.shape[1]
        a = lambda i, k: A[i][k]
        b = lambda k, j: B[k][j]
    else:  # TN
        K, M = An.shape
        N = Bn.shape[1]
        a = lambda i, k: A[k][i]
        b = lambda k, j: B[k][j]
    C = [[0.0] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = 0.0
            for k in range(K):
                s += float(a(i, k)) * float(b(k, j))
            C[i][j] = s
    return np.array(C)


def _operands(op, M, N, K, rng):
    shapes = {"NT": ((M, K), (N, K)), "NN": ((M, K), (K, N)), "TN": ((K, M), (K, N))}[op]
    return rng.standard_normal(shapes[0]), rng.standard_normal(shapes[1])


@pytest.mark.parametrize("op", og.OPS)
def test_triple_loop(op):
    rng = np.random.default_rng(11)
    A, B = _operands(op, 5, 3, 7, rng)
    C = og.gemm(op, A, B)
    assert C.shape == (5, 3)
    np.testing.assert_allclose(C, _loop(op, A, B), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("op", og.OPS)
def test_rows_sample_matches_full_product(op):
    rng = np.random.default_rng(12)
    A, B = _operands(op, 9, 4, 6, rng)
    rows = [0, 3, 8]
    np.testing.assert_array_equal(og.gemm_rows(op, A, B, rows), og.gemm(op, A, B)[rows])


@pytest.mark.parametrize("op", og.OPS)
def test_closed_forms(op):
    M, N, K = 4, 6, 8
    ones = {"NT": (np.ones((M, K)), np.ones((N, K))), "NN": (np.ones((M, K)), np.ones((K, N))),
            "TN": (np.ones((K, M)), np.ones((K, N)))}[op]
    assert np.array_equal(og.gemm(op, *ones), np.full((M, N), float(K)))
    rng = np.random.default_rng(13)
    X = rng.standard_normal((K, K))
    # an identity operand returns the other operand (transposed as op says)
    if op == "NT":
        assert np.array_equal(og.gemm(op, np.eye(K), X), X.T)
    elif op == "NN":
        assert np.array_equal(og.gemm(op, np.eye(K), X), X)
    else:
        assert np.array_equal(og.gemm(op, X, np.eye(K)), X.T)


def test_abs_product_bounds_the_product():
    rng = np.random.default_rng(14)
    A, B = _operands("NN", 7, 5, 9, rng)
    assert np.all(np.abs(og.gemm("NN", A, B)) <= og.abs_product("NN", A, B) + 1e-12)
