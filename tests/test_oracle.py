"""Pins of the fp64 CPU oracle against facts fixed by the mathematics, not by
the oracle itself (CPU only).

- Central finite differences of L = <dO, O> against the analytic dQ, dK, dV
  (Forge, section "Methodology and reproducibility": gradients are checked
  against central finite differences).
- Closed forms: uniform queries (Q = 0), equal keys, row 0 of a causal head,
  T = 1, and V = identity exposing P itself (rows sum to 1, upper triangle 0).
- Invariants: a common shift of every key, folding the scale into Q,
  causality (future keys and values cannot change a row), sum over keys of dK.
- A library routine on the same definition: torch's CPU float64
  scaled_dot_product_attention with autograd, and torch.logsumexp.
- Mutation check: planted mistakes in a copy of the oracle's C source must
  fail at least one of the pins above.
"""
import math
import os
import re
import shutil

import numpy as np
import pytest

import oracle

rng0 = np.random.default_rng(1234)


def _rand(shape, rng=None, sigma=1.0):
    rng = rng or rng0
    return rng.standard_normal(shape) * sigma


# ---------------------------------------------------------------- finite differences
def _loss(Q, K, V, dO, s, causal, lib=None):
    O, _ = oracle.attn_fwd(Q, K, V, s, causal, threads=1, lib=lib)
    return float(np.sum(O * dO))


def fd_check(T, d, causal, s, seed, lib=None):
    """Max normalised deviation of central FD from the analytic gradients."""
    rng = np.random.default_rng(seed)
    Q, K, V, dO = (rng.standard_normal((1, 1, T, d)) for _ in range(4))
    dQ, dK, dV, *_ = oracle.attn_bwd(Q, K, V, dO, s, causal, threads=1, lib=lib)
    h = 1e-6
    worst = 0.0
    for X, G in ((Q, dQ), (K, dK), (V, dV)):
        for idx in np.ndindex(X.shape):
            x0 = X[idx]
            X[idx] = x0 + h
            lp = _loss(Q, K, V, dO, s, causal, lib)
            X[idx] = x0 - h
            lm = _loss(Q, K, V, dO, s, causal, lib)
            X[idx] = x0
            fd = (lp - lm) / (2 * h)
            worst = max(worst, abs(fd - G[idx]) / max(1.0, abs(G[idx])))
    return worst


@pytest.mark.parametrize("T", [1, 2, 5, 8])
@pytest.mark.parametrize("d", [1, 3, 4])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("s", [1.0, 0.37])
def test_finite_differences(T, d, causal, s):
    assert fd_check(T, d, causal, s, seed=T * 100 + d * 10 + int(causal)) <= 1e-6


# ---------------------------------------------------------------- closed forms
def uniform_q_check(lib=None):
    T, d = 9, 3
    V, K, dO = _rand((2, T, d)), _rand((2, T, d)), _rand((2, T, d))
    Q = np.zeros((2, T, d))
    s = 0.7
    O, LSE = oracle.attn_fwd(Q, K, V, s, True, lib=lib)
    cnt = np.arange(1, T + 1, dtype=np.float64)[None, :, None]
    ok = np.allclose(O, np.cumsum(V, axis=1) / cnt, rtol=0, atol=1e-14)
    ok &= np.allclose(LSE, np.log(np.arange(1, T + 1))[None, :], rtol=0, atol=1e-14)
    dQ, dK, dV, *_ = oracle.attn_bwd(Q, K, V, dO, s, True, lib=lib)
    ok &= bool(np.all(dK == 0.0))
    # dV_j = sum_{i >= j} dO_i / (i + 1)
    w = dO / cnt
    ref_dv = np.flip(np.cumsum(np.flip(w, axis=1), axis=1), axis=1)
    ok &= np.allclose(dV, ref_dv, rtol=0, atol=1e-13)
    # non-causal: O_i = mean(V), LSE_i = ln T
    O2, LSE2 = oracle.attn_fwd(Q, K, V, s, False, lib=lib)
    ok &= np.allclose(O2, np.broadcast_to(V.mean(axis=1, keepdims=True), O2.shape), rtol=0, atol=1e-14)
    ok &= np.allclose(LSE2, math.log(T), rtol=0, atol=1e-14)
    return bool(ok)


def test_uniform_queries_closed_form():
    assert uniform_q_check()


def test_uniform_queries_closed_forms_module_matches_oracle():
    """tests/closed_forms.py (used by the long-sequence GPU test) against the
    oracle on small heads, dQ included."""
    import closed_forms

    for T, d, s in ((1, 4, 0.5), (9, 3, 0.7), (33, 8, -0.25)):
        K, V, dO = _rand((1, T, d)), _rand((1, T, d)), _rand((1, T, d))
        Q = np.zeros((1, T, d))
        dQ, dK, dV, O, LSE, _ = oracle.attn_bwd(Q, K, V, dO, s, True)
        cO, cL, cdV, cdQ = closed_forms.uniform_q(K[0], V[0], dO[0], s)
        assert np.allclose(cO, O[0], rtol=0, atol=1e-13)
        assert np.allclose(cL, LSE[0], rtol=0, atol=1e-13)
        assert np.allclose(cdV, dV[0], rtol=0, atol=1e-13)
        assert np.allclose(cdQ, dQ[0], rtol=1e-11, atol=1e-12)
        assert np.all(dK == 0.0)
        rows = [0, T // 2, T - 1]
        assert np.allclose(closed_forms.uniform_q(K[0], V[0], dO[0], s, rows)[3], dQ[0][rows], rtol=1e-11, atol=1e-12)


def equal_keys_check(lib=None):
    T, d = 7, 4
    Q, V, dO = _rand((3, T, d)), _rand((3, T, d)), _rand((3, T, d))
    k = _rand((3, 1, d))
    K = np.broadcast_to(k, (3, T, d)).copy()
    s = 0.5
    ok = True
    for causal in (True, False):
        O, _ = oracle.attn_fwd(Q, K, V, s, causal, lib=lib)
        Ou, _ = oracle.attn_fwd(np.zeros_like(Q), K, V, s, causal, lib=lib)
        ok &= np.allclose(O, Ou, rtol=0, atol=1e-13)
        dQ, *_ = oracle.attn_bwd(Q, K, V, dO, s, causal, lib=lib)
        ok &= float(np.max(np.abs(dQ))) <= 1e-13
    return bool(ok)


def test_equal_keys_closed_form():
    assert equal_keys_check()


def row0_check(lib=None):
    T, d = 6, 5
    Q, K, V = _rand((2, T, d)), _rand((2, T, d)), _rand((2, T, d))
    s = 0.3
    O, LSE = oracle.attn_fwd(Q, K, V, s, True, lib=lib)
    ok = bool(np.array_equal(O[:, 0], V[:, 0]))
    l0 = s * np.sum(Q[:, 0] * K[:, 0], axis=-1)
    ok &= np.allclose(LSE[:, 0], l0, rtol=1e-15, atol=1e-15)
    return bool(ok)


def test_row0_closed_form():
    assert row0_check()


def t1_check(lib=None):
    Q, K, V, dO = (_rand((4, 1, 3)) for _ in range(4))
    ok = True
    for causal in (True, False):
        dQ, dK, dV, O, LSE, D = oracle.attn_bwd(Q, K, V, dO, 1.3, causal, lib=lib)
        ok &= bool(np.array_equal(O, V)) and bool(np.all(dQ == 0)) and bool(np.all(dK == 0))
        ok &= bool(np.array_equal(dV, dO))
    return ok


def test_single_token():
    assert t1_check()


def identity_v_check(lib=None):
    """With V = I (d = T), O = P: rows sum to 1, P >= 0, causal upper triangle is 0."""
    T = 12
    Q, K = _rand((2, T, 5)), _rand((2, T, 5))
    V = np.broadcast_to(np.eye(T), (2, T, T)).copy()
    Qp = np.concatenate([Q, np.zeros((2, T, T - 5))], axis=-1)
    Kp = np.concatenate([K, np.zeros((2, T, T - 5))], axis=-1)
    ok = True
    for causal in (True, False):
        P, _ = oracle.attn_fwd(Qp, Kp, V, 0.8, causal, lib=lib)
        ok &= np.allclose(P.sum(-1), 1.0, rtol=0, atol=1e-14)
        ok &= bool(np.all(P >= 0))
        if causal:
            ok &= bool(np.all(np.triu(P[0], 1) == 0)) and bool(np.all(np.triu(P[1], 1) == 0))
        else:
            ok &= bool(np.all(P > 0))
    return bool(ok)


def test_softmax_rows_via_identity_values():
    assert identity_v_check()


# ---------------------------------------------------------------- invariants
def key_shift_check(lib=None):
    T, d = 10, 4
    Q, K, V, dO = (_rand((2, T, d)) for _ in range(4))
    c = _rand((1, 1, d))
    s = 0.45
    ok = True
    for causal in (True, False):
        a = oracle.attn_bwd(Q, K, V, dO, s, causal, lib=lib)
        b = oracle.attn_bwd(Q, K + c, V, dO, s, causal, lib=lib)
        for x, y in zip(a[:4], b[:4]):  # dQ, dK, dV, O unchanged
            ok &= np.allclose(x, y, rtol=0, atol=1e-12)
        ok &= np.allclose(b[4], a[4] + s * np.sum(Q * c, axis=-1), rtol=0, atol=1e-12)
    return bool(ok)


def test_key_shift_invariance():
    assert key_shift_check()


def scale_fold_check(lib=None):
    T, d = 11, 3
    Q, K, V = (_rand((2, T, d)) for _ in range(3))
    s = 0.61
    ok = True
    for causal in (True, False):
        O1, L1 = oracle.attn_fwd(Q, K, V, s, causal, lib=lib)
        O2, L2 = oracle.attn_fwd(s * Q, K, V, 1.0, causal, lib=lib)
        ok &= np.allclose(O1, O2, rtol=0, atol=1e-13) and np.allclose(L1, L2, rtol=0, atol=1e-13)
    return bool(ok)


def test_scale_fold_into_q():
    assert scale_fold_check()


def causality_check(lib=None):
    T, d = 9, 4
    Q, K, V = (_rand((1, T, d)) for _ in range(3))
    O, LSE = oracle.attn_fwd(Q, K, V, 0.9, True, lib=lib)
    ok = True
    for i in range(T - 1):
        K2, V2 = K.copy(), V.copy()
        K2[:, i + 1:] += 3.0
        V2[:, i + 1:] -= 2.0
        O2, L2 = oracle.attn_fwd(Q, K2, V2, 0.9, True, lib=lib)
        ok &= bool(np.array_equal(O2[:, : i + 1], O[:, : i + 1]))
        ok &= bool(np.array_equal(L2[:, : i + 1], LSE[:, : i + 1]))
    return ok


def test_causality_bit_identical():
    assert causality_check()


def dk_colsum_check(lib=None):
    T, d = 13, 4
    Q, K, V, dO = (_rand((3, T, d)) for _ in range(4))
    ok = True
    for causal in (True, False):
        dQ, dK, *_ = oracle.attn_bwd(Q, K, V, dO, 0.4, causal, lib=lib)
        ok &= float(np.max(np.abs(dK.sum(axis=1)))) <= 1e-12
    return ok


def test_sum_of_dk_over_keys_is_zero():
    assert dk_colsum_check()


# ---------------------------------------------------------------- library special case
def torch_check(lib=None):
    import torch

    ok = True
    for causal in (True, False):
        for (B, H, T, d, s) in ((2, 3, 17, 8, 0.35), (1, 2, 33, 16, 0.25)):
            rng = np.random.default_rng(T * 7 + d)
            Q, K, V, dO = (rng.standard_normal((B, H, T, d)) for _ in range(4))
            tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, K, V))
            o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=s)
            o.backward(torch.tensor(dO))
            sc = s * torch.tensor(Q) @ torch.tensor(K).transpose(-1, -2)
            if causal:
                sc = sc.masked_fill(torch.ones(T, T, dtype=torch.bool).triu(1), float("-inf"))
            lse = torch.logsumexp(sc, dim=-1)
            dQ, dK, dV, O, LSE, _ = oracle.attn_bwd(Q, K, V, dO, s, causal, lib=lib)
            for a, b in ((O, o), (LSE, lse), (dQ, tq.grad), (dK, tk.grad), (dV, tv.grad)):
                ok &= np.allclose(a, b.detach().numpy(), rtol=0, atol=1e-12)
    return bool(ok)


def test_against_torch_cpu_float64():
    assert torch_check()


# ---------------------------------------------------------------- threads / layout
def test_thread_count_and_head_slicing_bitwise():
    Q, K, V, dO = (_rand((2, 3, 20, 6)) for _ in range(4))
    a = oracle.attn_bwd(Q, K, V, dO, 0.5, True, threads=1)
    b = oracle.attn_bwd(Q, K, V, dO, 0.5, True, threads=4)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    # one head alone gives the same bits as inside a batch
    c = oracle.attn_bwd(Q[1:2, 2:3], K[1:2, 2:3], V[1:2, 2:3], dO[1:2, 2:3], 0.5, True, threads=1)
    for x, y in zip(a, c):
        assert np.array_equal(x[1:2, 2:3], y)
    O, L = oracle.attn_fwd(Q, K, V, 0.5, True, threads=3)
    assert np.array_equal(O, a[3]) and np.array_equal(L, a[4])


# ---------------------------------------------------------------- mutation check
MUTANTS = {
    # dK without the scale factor
    "dk_unscaled": ("dK[(size_t)j * d + c] = jb->s * acc;", "dK[(size_t)j * d + c] = acc;"),
    # dS with the wrong sign on D
    "ds_sign": ("* (dP - Di);", "* (dP + Di);"),
    # causal mask off by one (the diagonal hidden)
    "mask_off_by_one": ("const int jmax = causal ? i : T - 1;", "const int jmax = causal ? (i > 0 ? i - 1 : 0) : T - 1;"),
    # logsumexp without the max
    "lse_no_max": ("if (LSE) LSE[i] = m + log(l);", "if (LSE) LSE[i] = log(l);"),
    # dQ with K transposed in the contraction
    "dq_transposed": ("acc += dS[(size_t)i * T + j] * K[(size_t)j * d + c];",
                      "acc += dS[(size_t)j * T + i] * K[(size_t)j * d + c];"),
    # dV with P instead of P^T
    "dv_untransposed": ("acc += P[(size_t)i * T + j] * dO[(size_t)i * d + c];",
                        "acc += P[(size_t)j * T + i] * dO[(size_t)i * d + c];"),
}


def _all_pins(lib):
    return {
        "fd": all(fd_check(T, 3, c, s, 7, lib) <= 1e-6 for T in (2, 5) for c in (True, False) for s in (1.0, 0.37)),
        "uniform": uniform_q_check(lib),
        "equal_keys": equal_keys_check(lib),
        "row0": row0_check(lib),
        "t1": t1_check(lib),
        "identity_v": identity_v_check(lib),
        "key_shift": key_shift_check(lib),
        "causality": causality_check(lib),
        "torch": torch_check(lib),
    }


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name, tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, "mutation anchor missing: " + old
    mpath = tmp_path / ("mut_%s.c" % name)
    mpath.write_text(src.replace(old, new))
    lib = oracle.load_library(oracle.build(True, str(mpath), str(tmp_path / ("mut_%s.so" % name))))
    pins = _all_pins(lib)
    assert not all(pins.values()), "planted mistake %s passed every pin" % name


def test_unmutated_oracle_passes_every_pin(tmp_path):
    lib = oracle.load_library(oracle.build(True, os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c"),
                                           str(tmp_path / "plain.so")))
    pins = _all_pins(lib)
    assert all(pins.values()), pins
