"""Seeded synthetic inputs for causal attention, shared by the oracle side and
the GPU side of every test and of the benchmark.

This module holds no attention arithmetic: it only draws Gaussian tensors in a
fixed order and rounds them to the storage type.  Both the CPU oracle and the
HIP library receive exactly the values produced here (the oracle as float64
upcasts of the rounded values), following the Forge paper's practice of
comparing a fast low-precision path against a reference fed identically rounded
inputs (Forge, section "The same operands through matmul2d").

The workloads stand in for GPT training activations (Forge trains on
TinyStories, section "End-to-end training run"; the SwiftTransformer article
trains a 12-layer, 12-head, d_model 768 GPT): i.i.d. Gaussian Q, K, V and dO of
the layer shapes below.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class AttnConfig:
    name: str
    B: int
    H: int
    T: int
    d: int
    dtype: str  # "f32" or "bf16"
    causal: bool = True
    scale: float | None = None  # None: 1/sqrt(d)
    sigma_qk: float = 1.0
    sigma_v: float = 1.0
    sigma_do: float = 1.0
    seed: int = 0

    @property
    def scale_f32(self) -> float:
        s = (1.0 / math.sqrt(self.d)) if self.scale is None else self.scale
        return float(np.float32(s))

    @property
    def bh(self) -> int:
        return self.B * self.H


# dO ~ N(0, 1e-2) is read as variance 1e-2 (sigma 0.1); "scaled by 2" multiplies
# the N(0,1) draws of Q and K by 2 before rounding.
CONFIGS = {
    "tiny_f32": AttnConfig("tiny_f32", 1, 2, 64, 32, "f32", True, 1.0 / math.sqrt(32), seed=1),
    "gpt2_small": AttnConfig("gpt2_small", 8, 12, 1024, 64, "bf16", True, sigma_do=0.1, seed=2),
    "decoder_200m": AttnConfig("decoder_200m", 8, 16, 1024, 64, "bf16", True, sigma_do=0.1, seed=3),
    "long_4k": AttnConfig("long_4k", 2, 12, 4096, 64, "bf16", True, sigma_qk=2.0, seed=4),
    "wide_d128": AttnConfig("wide_d128", 4, 32, 2048, 128, "bf16", True, sigma_do=0.1, seed=5),
    # Forge's two attention-backward shapes (its Table 2: gpt-10m, B=64 T=512
    # H=6 d=64; gpt-25m, B=64 T=1024 H=8 d=64), for context only; Forge runs
    # them in fp32, so both precisions are listed
    "forge_gpt10m": AttnConfig("forge_gpt10m", 64, 6, 512, 64, "bf16", True, sigma_do=0.1, seed=6),
    "forge_gpt25m": AttnConfig("forge_gpt25m", 64, 8, 1024, 64, "bf16", True, sigma_do=0.1, seed=7),
    "forge_gpt10m_f32": AttnConfig("forge_gpt10m_f32", 64, 6, 512, 64, "f32", True, sigma_do=0.1, seed=6),
    "forge_gpt25m_f32": AttnConfig("forge_gpt25m_f32", 64, 8, 1024, 64, "f32", True, sigma_do=0.1, seed=7),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits.
    Inputs are finite (no NaN handling needed for Gaussian draws)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class AttnInputs:
    cfg: AttnConfig
    # values as the device receives them, widened to float32 (exact)
    Q: np.ndarray
    K: np.ndarray
    V: np.ndarray
    dO: np.ndarray
    # storage bits: float32 arrays in "f32" mode, uint16 bf16 bits in "bf16" mode
    store: dict = field(default_factory=dict)


def make_inputs(cfg: AttnConfig, seed: int | None = None, with_do: bool = True) -> AttnInputs:
    """Draw Q, K, V, dO (in that order) as float64 standard normals of shape
    [B,H,T,d] from numpy's PCG64 generator, multiply by their sigma, cast to
    float32 and, in bf16 mode, round to bfloat16."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    shape = (cfg.B, cfg.H, cfg.T, cfg.d)
    sig = {"Q": cfg.sigma_qk, "K": cfg.sigma_qk, "V": cfg.sigma_v, "dO": cfg.sigma_do}
    vals, store = {}, {}
    for name in ("Q", "K", "V", "dO"):
        if name == "dO" and not with_do:
            continue
        x = (rng.standard_normal(shape) * sig[name]).astype(np.float32)
        if cfg.dtype == "bf16":
            bits = f32_to_bf16_bits(x)
            store[name] = bits
            vals[name] = bf16_bits_to_f32(bits)
        else:
            store[name] = x
            vals[name] = x
    return AttnInputs(cfg, vals["Q"], vals["K"], vals["V"], vals.get("dO"), store)


def with_shape(cfg: AttnConfig, **kw) -> AttnConfig:
    """A copy of ``cfg`` with some fields replaced (e.g. a smaller T for tests)."""
    d = dict(cfg.__dict__)
    d.update(kw)
    return AttnConfig(**d)


# ---- layer-GEMM operands ------------------------------------------------------
# GPT-2-small MLP products at B=8, T=1024 (C = 768, hidden 3072): the forward
# X W1^T, the input gradient dY W1 and the weight gradient dY^T X, whose
# contraction runs over the B*T = 8192 tokens.
GEMM_WORKLOADS = {
    # name: (op, M, N, K)
    "mlp_fwd": ("NT", 8192, 3072, 768),
    "mlp_dx": ("NN", 8192, 768, 3072),
    "mlp_dw": ("TN", 3072, 768, 8192),
    "square_4096": ("NT", 4096, 4096, 4096),
}


def gemm_operand_shapes(op: str, M: int, N: int, K: int):
    """Shapes of A and B for C[M, N] = op(A) op(B)."""
    return {"NT": ((M, K), (N, K)), "NN": ((M, K), (K, N)), "TN": ((K, M), (K, N))}[op]


def make_matrix(shape, seed: int, sigma: float = 1.0):
    """float64 standard normals times sigma from PCG64(seed), rounded to
    bfloat16; returns (uint16 bits, float32 values)."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(shape) * sigma).astype(np.float32)
    bits = f32_to_bf16_bits(x)
    return bits, bf16_bits_to_f32(bits)
