"""GPU parity of the strided entry points, through the C ABI.

Q, K and V are read straight out of one packed [B, T, 3, H, d] buffer (the
output layout of a fused QKV projection), O and dO live as [B, T, H, d]
(= [B, T, H*d]), and dQ, dK, dV are written into one packed [B, T, 3, H, d]
gradient buffer.  Each case is compared with the fp64 oracle and, bit for
bit, with the contiguous entry points on the same values (the kernels run the
same arithmetic; only addresses change).  Every buffer is NaN-prefilled with
guard bands: no output may stay NaN, and no byte outside the views (guards,
row padding) may change.
"""
import numpy as np
import pytest
import torch

import attn_inputs as ai
import causal_attention_attn_amd as ca
from gpu_util import Guarded, compare, log, oracle_ref, run_gpu, to_device

pytestmark = pytest.mark.gpu


class ViewOut:
    """A [B, H, T, d] view into a guarded buffer, shaped like gpu_util's outputs."""

    def __init__(self, g: Guarded, view: torch.Tensor):
        self.g, self.view = g, view

    def guards_intact(self) -> bool:
        return self.g.guards_intact()

    def numpy64(self) -> np.ndarray:
        return self.view.float().cpu().numpy().astype(np.float64)


def _packed_inputs(inp, dt):
    """Q, K, V as views of one packed [B, T, 3, H, d] device buffer."""
    cfg = inp.cfg
    qkv = torch.empty((cfg.B, cfg.T, 3, cfg.H, cfg.d), dtype=dt, device="cuda")
    for i, n in enumerate(("Q", "K", "V")):
        qkv[:, :, i] = to_device(inp, n).permute(0, 2, 1, 3)
    return [qkv[:, :, i].permute(0, 2, 1, 3) for i in range(3)]


def run_packed(inp, scale, causal, atomic=False, pad=0):
    """Forward and backward on packed/strided views.  pad > 0 adds `pad`
    elements of padding after every token row of O, dO and the gradients."""
    cfg = inp.cfg
    B, H, T, d = cfg.B, cfg.H, cfg.T, cfg.d
    log("[gpu] packed B=%d H=%d T=%d d=%d %s causal=%d atomic=%d pad=%d" % (B, H, T, d, cfg.dtype, causal, atomic,
                                                                           pad))
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    Q, K, V = _packed_inputs(inp, dt)
    row = H * d + pad
    Og = Guarded((B, T, row), dt)
    O = Og.view[:, :, :H * d].unflatten(2, (H, d)).permute(0, 2, 1, 3)
    Lg = Guarded((B, H, T), torch.float32)
    ca.attn_fwd_strided(Q, K, V, O, Lg.view, scale, causal)
    dO_full = torch.full((B, T, row), float("nan"), dtype=dt, device="cuda")
    dO = dO_full[:, :, :H * d].unflatten(2, (H, d)).permute(0, 2, 1, 3)
    dO.copy_(to_device(inp, "dO"))
    dtc = ca.ATTN_BF16 if cfg.dtype == "bf16" else ca.ATTN_F32
    nbytes = (ca.attn_bwd_atomic_workspace_bytes if atomic else ca.attn_bwd_workspace_bytes)(dtc, B, H, T, d, causal)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    Gg = Guarded((B, T, 3 * H * d + pad), dt)
    G = Gg.view[:, :, :3 * H * d].unflatten(2, (3, H, d))
    dQ, dK, dV = (G[:, :, i].permute(0, 2, 1, 3) for i in range(3))
    fn = ca.attn_bwd_atomic_strided if atomic else ca.attn_bwd_strided
    fn(Q, K, V, O, dO, Lg.view, dQ, dK, dV, ws, scale, causal)
    torch.cuda.synchronize()
    if pad:
        assert bool(torch.isnan(Og.view[:, :, H * d:]).all()), "O row padding written"
        assert bool(torch.isnan(Gg.view[:, :, 3 * H * d:]).all()), "gradient row padding written"
    return {"O": ViewOut(Og, O), "LSE": Lg, "dQ": ViewOut(Gg, dQ), "dK": ViewOut(Gg, dK), "dV": ViewOut(Gg, dV)}


def _bitwise(a, b, names):
    for n in names:
        assert torch.equal(a[n].view.contiguous(), b[n].view.contiguous()), n + " differs from the contiguous path"


CASES = [
    ("bf16", 64, 200, True), ("bf16", 128, 333, True), ("bf16", 32, 65, True), ("bf16", 64, 130, False),
    ("f32", 64, 200, True), ("f32", 32, 17, True), ("f32", 128, 77, False),
]


@pytest.mark.parametrize("dtype,d,T,causal", CASES)
def test_packed_small(dtype, d, T, causal):
    cfg = ai.AttnConfig("packed", 2, 3, T, d, dtype, causal, None, seed=4000 + T + d)
    inp = ai.make_inputs(cfg)
    ref = oracle_ref(inp, cfg.scale_f32, causal)
    got = run_packed(inp, cfg.scale_f32, causal)
    compare(got, ref, dtype)
    _bitwise(got, run_gpu(inp, cfg.scale_f32, causal), ("O", "LSE", "dQ", "dK", "dV"))
    if dtype == "bf16":
        got_a = run_packed(inp, cfg.scale_f32, causal, atomic=True, pad=64)
        compare(got_a, ref, dtype)
        _bitwise(got_a, got, ("O", "LSE", "dK", "dV"))


def test_packed_full_size_gpt2_small():
    """The benchmark's shape (B 8, H 12, T 1024, d 64, bf16) in the packed
    layout: bit-equal to the contiguous path everywhere, and within the bf16
    bar of the oracle on sampled heads."""
    cfg = ai.CONFIGS["gpt2_small"]
    inp = ai.make_inputs(cfg)
    got = run_packed(inp, cfg.scale_f32, cfg.causal)
    _bitwise(got, run_gpu(inp, cfg.scale_f32, cfg.causal, label="gpt2_small contiguous"),
             ("O", "LSE", "dQ", "dK", "dV"))
    heads = [(0, 0), (cfg.B - 1, cfg.H - 1), (3, 5)]
    log("packed gpt2_small %s" % compare(got, oracle_ref(inp, cfg.scale_f32, cfg.causal, heads), "bf16", heads))


def test_broadcast_kv_heads():
    """K and V with head stride 0 (one key/value head shared by all query
    heads): equal to the contiguous path on K, V expanded over heads."""
    cfg = ai.AttnConfig("bcast", 2, 4, 150, 64, "bf16", True, None, seed=91)
    inp = ai.make_inputs(cfg)
    for n in ("K", "V"):  # make every head hold head 0's values
        inp.store[n][:] = inp.store[n][:, :1]
        getattr(inp, n)[:] = getattr(inp, n)[:, :1]
    ref = run_gpu(inp, cfg.scale_f32, True, label="bcast contiguous")
    Q, dO = to_device(inp, "Q"), to_device(inp, "dO")
    K1, V1 = (to_device(inp, n)[:, :1].expand(-1, cfg.H, -1, -1) for n in ("K", "V"))
    assert K1.stride(1) == 0
    shape = (cfg.B, cfg.H, cfg.T, cfg.d)
    O, L = Guarded(shape, torch.bfloat16), Guarded(shape[:3], torch.float32)
    ca.attn_fwd_strided(Q, K1, V1, O.view, L.view, cfg.scale_f32, True)
    ws = torch.empty(ca.attn_bwd_workspace_bytes(ca.ATTN_BF16, *shape), dtype=torch.uint8, device="cuda")
    dQ, dK, dV = (Guarded(shape, torch.bfloat16) for _ in range(3))
    ca.attn_bwd_strided(Q, K1, V1, O.view, dO, L.view, dQ.view, dK.view, dV.view, ws, cfg.scale_f32, True)
    torch.cuda.synchronize()
    got = {"O": O, "LSE": L, "dQ": dQ, "dK": dK, "dV": dV}
    for n, g in got.items():
        assert g.guards_intact(), n
    _bitwise(got, ref, ("O", "LSE", "dQ", "dK", "dV"))
