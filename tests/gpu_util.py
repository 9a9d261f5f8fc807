"""Helpers shared by the GPU tests: upload seeded inputs, run the HIP path
through the C ABI with NaN-prefilled outputs and guard bands, and compare with
the fp64 oracle.  Parity bars: fp32 inputs -> max |gpu - ref| <= 1e-4 per
output tensor (the Forge paper's float parity bar, section "Methodology and
reproducibility"); bf16 inputs -> max |gpu - ref| / max |ref| <= 2e-2 per
output tensor."""
from __future__ import annotations

import json
import os
import sys

import numpy as np
import torch

import attn_inputs as ai
import causal_attention_attn_amd as ca
import oracle

GUARD = 4096  # elements of sentinel on each side of every output buffer
TOL_F32_ABS = 1e-4
TOL_BF16_REL = 2e-2


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def to_device(inp: ai.AttnInputs, name: str) -> torch.Tensor:
    x = inp.store[name]
    if inp.cfg.dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to("cuda")


class Guarded:
    """A device buffer with NaN (float) or 0x7FC1 (bf16 NaN) sentinels around
    and inside it; ``view`` is the [shape] tensor handed to the library."""

    def __init__(self, shape, dtype):
        n = int(np.prod(shape))
        self.full = torch.full((n + 2 * GUARD,), float("nan"), dtype=dtype, device="cuda")
        self.view = self.full[GUARD:GUARD + n].view(*shape)
        self.n = n

    def guards_intact(self) -> bool:
        g = torch.cat([self.full[:GUARD], self.full[GUARD + self.n:]])
        return bool(torch.isnan(g).all())

    def numpy64(self) -> np.ndarray:
        return self.view.float().cpu().numpy().astype(np.float64)


def run_gpu(inp: ai.AttnInputs, scale: float, causal: bool, backward: bool = True, label: str = "",
            atomic: bool = False):
    cfg = inp.cfg
    log("[gpu] %s B=%d H=%d T=%d d=%d %s causal=%d scale=%g atomic=%d" % (
        label or cfg.name, cfg.B, cfg.H, cfg.T, cfg.d, cfg.dtype, causal, scale, atomic))
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    shape = (cfg.B, cfg.H, cfg.T, cfg.d)
    Q, K, V = (to_device(inp, n) for n in ("Q", "K", "V"))
    O = Guarded(shape, dt)
    L = Guarded(shape[:3], torch.float32)
    ca.attn_fwd(Q, K, V, O.view, L.view, scale, causal)
    out = {"O": O, "LSE": L}
    if backward:
        dO = to_device(inp, "dO")
        dtc = ca.ATTN_BF16 if cfg.dtype == "bf16" else ca.ATTN_F32
        nbytes = (ca.attn_bwd_atomic_workspace_bytes if atomic else ca.attn_bwd_workspace_bytes)(dtc, *shape, causal)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        dQ, dK, dV = (Guarded(shape, dt) for _ in range(3))
        bwd = ca.attn_bwd_atomic if atomic else ca.attn_bwd
        bwd(Q, K, V, O.view, dO, L.view, dQ.view, dK.view, dV.view, ws, scale, causal)
        out.update(dQ=dQ, dK=dK, dV=dV)
    torch.cuda.synchronize()
    return out


def oracle_ref(inp: ai.AttnInputs, scale: float, causal: bool, heads=None):
    """Oracle outputs (float64) on all heads, or on the listed (b, h) pairs."""
    def sel(x):
        if heads is None:
            return x
        return np.stack([x[b, h] for (b, h) in heads])[None]

    dQ, dK, dV, O, LSE, D = oracle.attn_bwd(sel(inp.Q), sel(inp.K), sel(inp.V), sel(inp.dO), scale, causal)
    return {"O": O, "LSE": LSE, "dQ": dQ, "dK": dK, "dV": dV, "D": D}


def compare(gpu: dict, ref: dict, dtype: str, heads=None, names=("O", "LSE", "dQ", "dK", "dV")):
    """Per-tensor errors; raises AssertionError naming every tensor off the bar."""
    errs, bad = {}, []
    for n in names:
        if n not in gpu:
            continue
        g = gpu[n]
        assert g.guards_intact(), "%s: guard band overwritten" % n
        x = g.numpy64()
        if heads is not None:
            x = np.stack([x[b, h] for (b, h) in heads])[None]
        assert not np.isnan(x).any(), "%s: %d outputs never written (NaN sentinel left)" % (n, int(np.isnan(x).sum()))
        r = ref[n]
        amax = float(np.max(np.abs(x - r)))
        rmax = float(np.max(np.abs(r)))
        rel = amax / rmax if rmax > 0 else amax
        frob = float(np.linalg.norm(x - r) / max(np.linalg.norm(r), 1e-300))
        errs[n] = {"max_abs": amax, "max_rel": rel, "frob_rel": frob}
        ok = amax <= TOL_F32_ABS if dtype == "f32" else rel <= TOL_BF16_REL
        if not ok:
            bad.append("%s max_abs=%.3g max_rel=%.3g" % (n, amax, rel))
    rec_path = os.environ.get("ATTN_PARITY_LOG")
    if rec_path:
        with open(rec_path, "a") as f:
            f.write(json.dumps({"test": os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], "dtype": dtype,
                                "errors": errs, "ok": not bad}) + "\n")
    assert not bad, "; ".join(bad)
    return errs
