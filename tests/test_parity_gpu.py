"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs, element by element.

- every configuration of the benchmark suite at full size, compared on
  sampled (batch, head) slices the oracle computes one by one;
- small shapes that span several tiles with ragged tails (T not a multiple of
  any tile), every head dimension, both dtypes, causal and non-causal, other
  scales including a negative one;
- closed forms and properties on the GPU: row 0 of a causal head returns V_0,
  uniform queries give running means of V and dK = 0, bitwise determinism;
- coverage: outputs start as NaN and none may remain; guard bands around
  every output stay untouched.
"""
import math

import numpy as np
import pytest
import torch

import attn_inputs as ai
from gpu_util import compare, log, oracle_ref, run_gpu

pytestmark = pytest.mark.gpu


def _heads(cfg, k=3):
    picks = [(0, 0), (cfg.B - 1, cfg.H - 1), (cfg.B // 2, cfg.H // 2)]
    return list(dict.fromkeys(picks))[:k]


def test_tiny_f32_full():
    cfg = ai.CONFIGS["tiny_f32"]
    inp = ai.make_inputs(cfg)
    gpu = run_gpu(inp, cfg.scale_f32, cfg.causal)
    errs = compare(gpu, oracle_ref(inp, cfg.scale_f32, cfg.causal), "f32")
    log("tiny_f32 %s" % errs)


@pytest.mark.parametrize("atomic", [False, True])
@pytest.mark.parametrize("name", ["gpt2_small", "decoder_200m", "long_4k", "wide_d128"])
def test_full_size_sampled_heads(name, atomic):
    cfg = ai.CONFIGS[name]
    inp = ai.make_inputs(cfg)
    gpu = run_gpu(inp, cfg.scale_f32, cfg.causal, label=name, atomic=atomic)
    heads = _heads(cfg)
    errs = compare(gpu, oracle_ref(inp, cfg.scale_f32, cfg.causal, heads), cfg.dtype, heads)
    log("%s %s" % (name, errs))


SMALL = []
for dtype in ("bf16", "f32"):
    for d in (32, 64, 128):
        for T in (1, 17, 63, 65, 200, 333, 1000):
            SMALL.append((dtype, d, T, True))
    for d, T in ((64, 130), (128, 77), (128, 300), (32, 260)):
        SMALL.append((dtype, d, T, False))


@pytest.mark.parametrize("dtype,d,T,causal", SMALL)
def test_small_ragged(dtype, d, T, causal):
    cfg = ai.AttnConfig("small", 2, 3, T, d, dtype, causal, None, seed=1000 + T + d)
    inp = ai.make_inputs(cfg)
    ref = oracle_ref(inp, cfg.scale_f32, causal)
    compare(run_gpu(inp, cfg.scale_f32, causal), ref, dtype)
    if dtype == "bf16":
        compare(run_gpu(inp, cfg.scale_f32, causal, atomic=True), ref, dtype)


# Ragged sequences past 2048 keys, where bf16 d = 64 takes the interleaved dQ
# kernel (its steady-tile loop, then the edge tiles), causal and not, against
# the oracle on every head.
@pytest.mark.parametrize("T,causal", [(2100, True), (2500, False), (3073, True)])
def test_long_ragged_bf16_d64(T, causal):
    cfg = ai.AttnConfig("long_ragged", 1, 2, T, 64, "bf16", causal, None, seed=3000 + T)
    inp = ai.make_inputs(cfg)
    errs = compare(run_gpu(inp, cfg.scale_f32, causal), oracle_ref(inp, cfg.scale_f32, causal), "bf16")
    log("long_ragged T=%d causal=%d %s" % (T, causal, errs))


@pytest.mark.parametrize("scale", [0.3, -0.2, 0.0])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_other_scales(scale, dtype):
    cfg = ai.AttnConfig("scale", 1, 2, 150, 64, dtype, True, scale, seed=77)
    inp = ai.make_inputs(cfg)
    s = float(np.float32(scale))
    gpu = run_gpu(inp, s, True)
    compare(gpu, oracle_ref(inp, s, True), dtype)


def test_row0_returns_v0_exactly():
    cfg = ai.AttnConfig("row0", 2, 2, 96, 64, "bf16", True, seed=5)
    inp = ai.make_inputs(cfg)
    gpu = run_gpu(inp, cfg.scale_f32, True, backward=False)
    O = gpu["O"].view.float().cpu().numpy()
    assert np.array_equal(O[:, :, 0, :], inp.V[:, :, 0, :])


def test_uniform_queries_on_gpu():
    cfg = ai.AttnConfig("uniform", 1, 2, 300, 64, "bf16", True, seed=6)
    inp = ai.make_inputs(cfg)
    inp.store["Q"][:] = 0
    inp.Q[:] = 0
    gpu = run_gpu(inp, cfg.scale_f32, True)
    cnt = np.arange(1, cfg.T + 1, dtype=np.float64)[None, None, :, None]
    ref_O = np.cumsum(inp.V.astype(np.float64), axis=2) / cnt
    O = gpu["O"].numpy64()
    assert np.max(np.abs(O - ref_O)) <= 2e-2 * np.max(np.abs(ref_O))
    L = gpu["LSE"].numpy64()
    assert np.max(np.abs(L - np.log(np.arange(1, cfg.T + 1))[None, None])) <= 1e-5
    assert float(np.max(np.abs(gpu["dK"].numpy64()))) == 0.0


def test_bitwise_deterministic():
    cfg = ai.with_shape(ai.CONFIGS["gpt2_small"], B=2, H=4)
    inp = ai.make_inputs(cfg)
    a = run_gpu(inp, cfg.scale_f32, True)
    b = run_gpu(inp, cfg.scale_f32, True)
    for n in ("O", "LSE", "dQ", "dK", "dV"):
        assert torch.equal(a[n].view, b[n].view), n


def test_atomic_path_repeatability():
    """The atomic-dQ backward: dK and dV bitwise equal across runs and equal to
    attn_bwd's; dQ within fp32 reordering of its sums."""
    cfg = ai.with_shape(ai.CONFIGS["gpt2_small"], B=2, H=4)
    inp = ai.make_inputs(cfg)
    a = run_gpu(inp, cfg.scale_f32, True, atomic=True)
    b = run_gpu(inp, cfg.scale_f32, True, atomic=True)
    c = run_gpu(inp, cfg.scale_f32, True)
    for n in ("O", "LSE", "dK", "dV"):
        assert torch.equal(a[n].view, b[n].view), n
        assert torch.equal(a[n].view, c[n].view), n
    da, db, dc = (x["dQ"].view.float() for x in (a, b, c))
    scale = float(dc.abs().max())
    assert float((da - db).abs().max()) <= 1e-2 * scale
    assert float((da - dc).abs().max()) <= 1e-2 * scale


def test_general_dkdv_kernel_matches_steady():
    """B16 H8 T1024 d64 has 1024 key blocks of 128: two full rounds of the
    steady dK/dV kernel's resident workgroups (two per compute unit on 256),
    so attn_bwd runs the three-wave general kernel there, while the atomic
    path keeps the steady tile loop.  Their dK and dV must agree bit for bit."""
    cfg = ai.with_shape(ai.CONFIGS["gpt2_small"], B=16, H=8)
    inp = ai.make_inputs(cfg)
    a = run_gpu(inp, cfg.scale_f32, True)
    c = run_gpu(inp, cfg.scale_f32, True, atomic=True)
    for n in ("dK", "dV"):
        assert torch.equal(a[n].view, c[n].view), n


@pytest.mark.parametrize("dtype,T,d", [("bf16", 65553, 64), ("bf16", 32785, 128), ("f32", 16401, 64)])
def test_long_sequence_uniform_queries(dtype, T, d):
    """Sequence lengths far past the workloads (ragged: not a multiple of any
    tile), checked against the closed forms for Q = 0 (tests/closed_forms.py):
    O and LSE on every row, dV on every key, dK = 0 exactly, dQ on sampled
    rows."""
    import closed_forms

    cfg = ai.AttnConfig("long_uniform", 1, 2, T, d, dtype, True, None, sigma_do=0.1, seed=17)
    inp = ai.make_inputs(cfg)
    inp.store["Q"][:] = 0
    inp.Q[:] = 0
    gpu = run_gpu(inp, cfg.scale_f32, True, label="long_uniform")
    rows = [0, 1, 63, 64, 1000, T // 2, T - 2, T - 1]
    ref = {"O": [], "LSE": [], "dV": [], "dQ": []}
    for h in range(cfg.H):
        O, LSE, dV, dQ = closed_forms.uniform_q(inp.K[0, h], inp.V[0, h], inp.dO[0, h], cfg.scale_f32, rows)
        for n, x in (("O", O), ("LSE", LSE), ("dV", dV), ("dQ", dQ)):
            ref[n].append(x)
    tol = 1e-4 if dtype == "f32" else 2e-2
    for n in ("O", "LSE", "dV", "dQ"):
        g = gpu[n]
        assert g.guards_intact(), n
        x = g.numpy64()[0]
        if n == "dQ":
            x = x[:, rows]
        r = np.stack(ref[n])
        assert not np.isnan(x).any(), n
        err = float(np.max(np.abs(x - r)))
        bar = tol if dtype == "f32" else tol * float(np.max(np.abs(r)))
        log("long_uniform %s T=%d d=%d %s: max abs err %.3g (bar %.3g)" % (dtype, T, d, n, err, bar))
        assert err <= bar, (n, err, bar)
    assert float(np.max(np.abs(gpu["dK"].numpy64()))) == 0.0


@pytest.mark.parametrize("name", ["forge_gpt10m_f32", "forge_gpt25m_f32"])
def test_forge_shapes_f32_sampled_heads(name):
    """Random fp32 inputs at Forge's attention-backward shapes (its Table 2,
    all-float), the launch the fp32 bench times, against the oracle on three
    heads at the fp32 bar (max abs error <= 1e-4)."""
    cfg = ai.CONFIGS[name]
    inp = ai.make_inputs(cfg)
    gpu = run_gpu(inp, cfg.scale_f32, cfg.causal, label=name)
    heads = _heads(cfg)
    errs = compare(gpu, oracle_ref(inp, cfg.scale_f32, cfg.causal, heads), "f32", heads)
    log("%s %s" % (name, errs))


def _equal_keys(cfg):
    inp = ai.make_inputs(cfg)
    # every key of a head equal to its key 0 (the stored values, so both sides
    # see the same numbers)
    inp.store["K"][:] = inp.store["K"][:, :, :1, :]
    inp.K[:] = inp.K[:, :, :1, :]
    return inp


@pytest.mark.parametrize("dtype,d,T", [("bf16", 64, 1000), ("bf16", 128, 333), ("f32", 64, 300)])
def test_equal_keys_give_zero_dq(dtype, d, T):
    """Equal keys (k_j = k for every j): the probabilities do not depend on
    the query, so sum_j dS_ij = sum_j P_ij dP_ij - D_i = 0 and dQ_i =
    s (sum_j dS_ij) k = 0 exactly.  On the GPU what is left is rounding: dS is
    rounded to the element type before its product with K (relative 2^-8 in
    bf16, at most), and D is formed from the stored O; the bound per row is
    2^-7 s max|k| (sum_j |dS_ij| + sum_c |dO_ic O_ic|) with the oracle's fp64
    values (2^-12 for fp32, whose LSE and D carry fp32 rounding).  O, LSE, dK,
    dV stay at the usual parity bar."""
    cfg = ai.AttnConfig("equal_keys", 1, 3, T, d, dtype, True, None, sigma_do=0.1, seed=4000 + T)
    inp = _equal_keys(cfg)
    s = cfg.scale_f32
    gpu = run_gpu(inp, s, True, label="equal_keys")
    ref = oracle_ref(inp, s, True)
    compare(gpu, ref, dtype, names=("O", "LSE", "dK", "dV"))
    dq = gpu["dQ"].numpy64()
    assert not np.isnan(dq).any()
    assert float(np.max(np.abs(ref["dQ"]))) <= 1e-9 * float(np.max(np.abs(ref["dV"])))  # the oracle's own zero
    eps = 2.0 ** -7 if dtype == "bf16" else 2.0 ** -12
    for h in range(cfg.H):
        k = inp.K[0, h, 0].astype(np.float64)
        V, dO, O = (x[0, h].astype(np.float64) for x in (inp.V, inp.dO, ref["O"]))
        D = ref["D"][0, h]
        dp = dO @ V.T                                   # dP_ij = dO_i . V_j
        P = np.tril(np.ones((T, T))) / np.arange(1, T + 1)[:, None]  # uniform over j <= i
        bound = eps * s * np.max(np.abs(k)) * (np.sum(np.abs(P * (dp - D[:, None])), axis=1)
                                               + np.sum(np.abs(dO * O), axis=1))
        err = np.max(np.abs(dq[0, h]), axis=1)
        log("equal_keys %s d=%d T=%d head %d: max |dQ| %.3g, max bound %.3g" % (
            dtype, d, T, h, float(err.max()), float(bound.max())))
        assert np.all(err <= bound), "row %d: |dQ| %.3g > %.3g" % (int(np.argmax(err - bound)), err.max(), bound.max())


@pytest.mark.parametrize("dtype,d,T", [("bf16", 64, 1000), ("bf16", 128, 513), ("f32", 32, 257)])
def test_key_gradients_sum_to_zero(dtype, d, T):
    """sum_j dK_j = s sum_i (sum_j dS_ij) q_i = 0 for every (b, h), because
    every row of dS sums to zero.  The GPU's column sums of dK must vanish to
    within 2^-6 (bf16; 1e-4 for fp32) of the oracle's sum_j |dK_jc|."""
    cfg = ai.AttnConfig("dk_sum", 2, 2, T, d, dtype, True, None, sigma_do=0.1, seed=5000 + T)
    inp = ai.make_inputs(cfg)
    gpu = run_gpu(inp, cfg.scale_f32, True, label="dk_sum")
    ref = oracle_ref(inp, cfg.scale_f32, True)
    compare(gpu, ref, dtype)
    dk = gpu["dK"].numpy64()
    rel = 2.0 ** -6 if dtype == "bf16" else 1e-4
    for b in range(cfg.B):
        for h in range(cfg.H):
            colsum = np.abs(dk[b, h].sum(axis=0))
            scale = np.abs(ref["dK"][b, h]).sum(axis=0).max()
            log("dk_sum %s d=%d T=%d (%d,%d): max |sum_j dK_j| %.3g of sum|dK| %.3g" % (
                dtype, d, T, b, h, float(colsum.max()), float(scale)))
            assert float(colsum.max()) <= rel * float(scale)
