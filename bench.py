"""Benchmark: fused causal attention forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gpt2_small]
                    [--layout contiguous|packed] [--bwd deterministic|atomic]
                    [--no-cpu-baseline]
    python bench.py --gemm [all|mlp_fwd|mlp_dx|mlp_dw|square_4096] [--split-k S]

A step is one attn_fwd plus one attn_bwd (every kernel of the path: forward,
D preprocess, dK/dV, dQ) over the workload's device-resident synthetic inputs.
W untimed steps, then K steps bracketed by synchronisations and HIP events on
the stream the library launches on.  The printed JSON line carries:
  value      causal-adjusted TFLOP/s of the whole step, 7 B H T^2 d / time
             (forward 2 B H T^2 d, backward 5 B H T^2 d: every T x T x d
             product counted over the lower triangle only);
  roofline   the dominant kernel's algorithmic FLOPs per launch over its
             average event-measured duration, against the bf16 dense MFMA peak;
  cpu_baseline  the fp64 CPU oracle timed on the host cores on a sample of the
             same workload (test infrastructure, reported for context only).
Inputs stay resident in HBM during the timed region; numbers are warm-cache
(the whole working set fits in the 256 MB Infinity Cache).
--layout packed runs the same step through the strided entry points on the
layouts of a GPT-2 layer: Q, K, V read from one [B, T, 3, H, d] projection
output, O and dO as [B, T, H*d], dQ, dK, dV written into one packed
[B, T, 3, H, d] gradient buffer.
--gemm times the layer products instead (gemm_bf16: the GPT-2-small MLP
forward X W1^T, input gradient dY W1 and weight gradient dY^T X at B=8 T=1024,
and a 4096^3 square product), one JSON line per product, with the fp64
oracle timed on a sample of output rows as the CPU baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal attn fwd+bwd TFLOP/s (and % bf16 MFMA peak), B8 H12 T1024 d64, 1 GPU"
PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
WARMUP_S = 0.5

# Algorithmic T^2 d "units" (one causal-adjusted product: B H T^2 d multiply-adds
# over the lower triangle = 2 B H T^2 d / 2 flops) executed for the method by
# each kernel.  The dQ kernel recomputes S and dP (2 units) that are not
# counted: only its dQ product is algorithmic.  The dK/dV kernel (one wave or,
# at d = 128, a wave pair per key block) forms S, dP, dV and dK.
UNITS = {"attn_fwd": 2, "attn_bwd_dkdv": 4, "attn_bwd_dq": 1}
CSRC = os.path.join(ROOT, "causal_attention_attn_amd", "csrc")


def flops_units(cfg, units: float) -> float:
    f = 2.0 * cfg.B * cfg.H * cfg.T * cfg.T * cfg.d * units
    return f / 2 if cfg.causal else f


def fwd_bytes(cfg) -> float:
    """Algorithmic bytes of the forward: read Q, K, V, write O and LSE."""
    e = 2 if cfg.dtype == "bf16" else 4
    return 4.0 * cfg.B * cfg.H * cfg.T * cfg.d * e + 4.0 * cfg.B * cfg.H * cfg.T


def bwd_bytes(cfg) -> float:
    """Algorithmic bytes of the backward: read Q, K, V, O, dO and LSE, write
    dQ, dK, dV, write and read D."""
    e = 2 if cfg.dtype == "bf16" else 4
    return 8.0 * cfg.B * cfg.H * cfg.T * cfg.d * e + 12.0 * cfg.B * cfg.H * cfg.T


def sclk_mhz():
    """Current shader clock of the first GPU from sysfs (the DPM level marked
    active), or None where it cannot be read."""
    import glob
    import re

    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            for ln in open(f):
                if ln.rstrip().endswith("*"):
                    m = re.search(r"(\d+)\s*Mhz", ln, re.I)
                    if m:
                        return int(m.group(1))
        except OSError:
            continue
    return None


def _code_only(text: str) -> str:
    """C++ source with its comments removed and each line stripped of outer
    whitespace (blank lines dropped); string and character literals are kept
    as written."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return "\n".join(line.strip() for line in "".join(out).split("\n") if line.strip())


def kernel_source_sha() -> str:
    """sha256[:16] of the kernel sources' code (comments and layout removed),
    which keys the committed counter summaries: a change to the comments
    alone keeps them."""
    h = hashlib.sha256()
    for n in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, n), encoding="utf-8") as f:
            h.update(n.encode() + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_for(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is absent or was taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get("kernels", {}).get(kernel)
    if not rec or t.get("source_sha") != kernel_source_sha():
        return None
    return (rec["fetch_kib"] * t["fetch_scale"] + rec["write_kib"] * t["write_scale"]) * 1024.0


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, inp, heads: int, threads: int, gpu_out=None, one_thread: bool = True):
    """The fp64 oracle, forward then backward, on the first `heads` (b, h)
    heads of the bench inputs, timed on the host cores.  When the GPU outputs
    of the same inputs are given, also reports their per-tensor error against
    the oracle (max |gpu - ref| and that over max |ref|) on those heads."""
    import numpy as np

    import oracle

    d = cfg.d
    flat = lambda x: np.ascontiguousarray(x.reshape(cfg.B * cfg.H, cfg.T, d)[:heads])
    Q, K, V, dO = flat(inp.Q), flat(inp.K), flat(inp.V), flat(inp.dO)
    oracle.attn_bwd(Q[:1, :64], K[:1, :64], V[:1, :64], dO[:1, :64], cfg.scale_f32, cfg.causal,
                    threads=1)  # loads the library
    t0 = time.perf_counter()
    O, LSE = oracle.attn_fwd(Q, K, V, cfg.scale_f32, cfg.causal, threads=threads)
    dQ, dK, dV, _, _, _ = oracle.attn_bwd(Q, K, V, dO, cfg.scale_f32, cfg.causal, threads=threads)
    dt = time.perf_counter() - t0
    used = min(threads, heads)
    one = None
    if one_thread:
        # the same sample on one thread, head after head (progress on stderr)
        t1 = time.perf_counter()
        for i in range(heads):
            oracle.attn_fwd(Q[i:i + 1], K[i:i + 1], V[i:i + 1], cfg.scale_f32, cfg.causal, threads=1)
            oracle.attn_bwd(Q[i:i + 1], K[i:i + 1], V[i:i + 1], dO[i:i + 1], cfg.scale_f32, cfg.causal, threads=1)
            if (i + 1) % 16 == 0 or i + 1 == heads:
                print("[bench] one-thread oracle: %d of %d heads, %.1f s" % (i + 1, heads, time.perf_counter() - t1),
                      file=sys.stderr, flush=True)
        one = (time.perf_counter() - t1) * 1e3
    sub = __import__("attn_inputs").with_shape(cfg, B=1, H=heads)
    res = {
        "value": flops_units(sub, 7) / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": used,
        "kind": "oracle",
        "sample": "%d of %d (b,h) heads of %s (T=%d, d=%d), fp64 oracle forward then backward, %.2f s wall"
                  % (heads, cfg.B * cfg.H, cfg.name, cfg.T, cfg.d, dt),
        "cpu_ms_total": dt * 1e3,
        "cpu_threads": used,
        "cpu_ms_total_one_thread": one,
        "nproc": os.cpu_count(),
        "cpu_model": cpu_model(),
    }
    if gpu_out is not None:
        ref = {"O": O, "LSE": LSE, "dQ": dQ, "dK": dK, "dV": dV}
        par = {}
        for n, r in ref.items():
            g = gpu_out[n].reshape((cfg.B * cfg.H,) + r.shape[1:])[:heads].astype(np.float64)
            e = float(np.max(np.abs(g - r)))
            par[n] = {"max_abs": e, "max_rel": e / max(float(np.max(np.abs(r))), 1e-300)}
        res["parity"] = par
    return res


def cpu_tiny_f32(threads: int, runs: int = 5):
    """The fp64 oracle, forward then backward, on the whole tiny fp32
    configuration (B1 H2 T64 d32): median, min and max of `runs` runs with one
    thread per head, and one run on a single thread."""
    import attn_inputs as ai
    import oracle

    cfg = ai.CONFIGS["tiny_f32"]
    inp = ai.make_inputs(cfg)

    def once(nthreads):
        t0 = time.perf_counter()
        oracle.attn_fwd(inp.Q, inp.K, inp.V, cfg.scale_f32, cfg.causal, threads=nthreads)
        oracle.attn_bwd(inp.Q, inp.K, inp.V, inp.dO, cfg.scale_f32, cfg.causal, threads=nthreads)
        return (time.perf_counter() - t0) * 1e3

    once(1)  # loads the library
    used = min(threads, cfg.B * cfg.H)
    xs = sorted(once(used) for _ in range(runs))
    return {"workload": "tiny_f32: B=1 H=2 T=64 head_dim=32 f32, fp64 oracle forward then backward",
            "threads": used, "runs": runs, "median_ms": xs[len(xs) // 2], "min_ms": xs[0], "max_ms": xs[-1],
            "one_thread_ms": once(1)}


def blas_threads():
    """Threads of the BLAS behind numpy's matmul (None if unknown)."""
    try:
        from threadpoolctl import threadpool_info

        n = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
        return int(n[0]) if n else None
    except Exception:
        return None


def bench_gemm(a) -> int:
    """One JSON line per layer GEMM: W untimed calls (and at least WARMUP_S s),
    then K calls between HIP events on the launch stream."""
    import numpy as np
    import torch

    import attn_inputs as ai
    import causal_attention_attn_amd as ca

    opc = {"NT": ca.GEMM_NT, "NN": ca.GEMM_NN, "TN": ca.GEMM_TN}
    names = list(ai.GEMM_WORKLOADS) if a.gemm == "all" else [a.gemm]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    for name in names:
        op, M, N, K = ai.GEMM_WORKLOADS[name]
        sa, sb = ai.gemm_operand_shapes(op, M, N, K)
        Ab, Af = ai.make_matrix(sa, seed=300)
        Bb, Bf = ai.make_matrix(sb, seed=301)
        A = torch.from_numpy(Ab.view(np.int16)).view(torch.bfloat16).to(dev)
        B = torch.from_numpy(Bb.view(np.int16)).view(torch.bfloat16).to(dev)
        C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        nb = ca.gemm_workspace_bytes(opc[op], M, N, K, a.split_k)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None

        def call():
            ca.gemm(opc[op], A, B, C, a.split_k, ws, stream)

        t0 = time.perf_counter()
        n = 0
        while n < a.warmup or time.perf_counter() - t0 < WARMUP_S:
            call()
            n += 1
            if n % 50 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        ca.attn_prof_enable(2 * a.steps + 8)
        ca.attn_prof_read()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(a.steps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / a.steps
        kern = ca.attn_prof_read()
        ca.attn_prof_enable(0)
        flops = 2.0 * M * N * K
        kernels = {k: {"launches": c, "avg_us": 1000.0 * t / c} for k, (c, t) in kern.items()}
        ach = flops / (kernels["gemm"]["avg_us"] * 1e-6) / 1e12
        out = {
            "metric": "layer GEMM TFLOP/s (bf16 operands, fp32 accumulation), 1 GPU",
            "value": flops / (ms * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps,
            "warmup": a.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "%s: %s M=%d N=%d K=%d" % (name, op, M, N, K), "op": op, "M": M, "N": N, "K": K,
                       "split_k": a.split_k, "workspace_bytes": nb},
            "kernels": kernels,
            "roofline": {"bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": ach / PEAK_BF16_TFLOPS, "kernel": "gemm", "traffic": None},
            "cpu_baseline": None,
        }
        # the same product through torch.matmul (the vendor BLAS library), timed
        # the same way: context for the kernel's number, not part of the path
        f = {"NT": lambda: A @ B.t(), "NN": lambda: A @ B, "TN": lambda: A.t() @ B}[op]
        for _ in range(max(a.warmup, 10)):
            f()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(a.steps):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_vendor = e0.elapsed_time(e1) / a.steps
        out["vendor_blas"] = {"call": "torch.matmul", "ms": ms_vendor, "value": flops / (ms_vendor * 1e-3) / 1e12,
                              "unit": "TFLOP/s"}
        if not a.no_cpu_baseline:
            from oracle import gemm as og

            rows = np.arange(0, M, max(1, M // 64))[:64]
            t1 = time.perf_counter()
            og.gemm_rows(op, Af, Bf, rows)
            dt = time.perf_counter() - t1
            out["cpu_baseline"] = {"value": 2.0 * len(rows) * N * K / dt / 1e12, "unit": "TFLOP/s",
                                   "cores": blas_threads(),
                                   "kind": "oracle",
                                   "sample": "%d of %d output rows, fp64 numpy matmul, %.3f s wall" % (len(rows), M, dt)}
        print(json.dumps(out), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="gpt2_small",
                    help="an attention configuration of attn_inputs.CONFIGS, or 'all' for one line per benchmark configuration")
    ap.add_argument("--layout", choices=("contiguous", "packed"), default="contiguous")
    ap.add_argument("--bwd", choices=("deterministic", "atomic"), default="deterministic",
                    help="backward path: attn_bwd (default) or attn_bwd_atomic (bf16 only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=0, help="heads in the CPU sample (0: all)")
    ap.add_argument("--cpu-threads", type=int, default=16)
    ap.add_argument("--no-cpu-one-thread", action="store_true",
                    help="skip the single-thread oracle run over the whole sample (tiny_f32 and gpt2_small)")
    ap.add_argument("--gemm", default=None, metavar="WORKLOAD",
                    help="time the layer GEMMs instead of attention: 'all' or one workload name")
    ap.add_argument("--split-k", type=int, default=0, help="split_k for --gemm (0: chosen from the shape)")
    ap.add_argument("--repeats", type=int, default=5,
                    help="extra timed regions of K passes each for the fwd/bwd/step spread (median, min, max)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (HBM counter calibration)")
    a = ap.parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(every (batch, head) pair is independent, so B or H would shard with no exchange); "
              "run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    if a.copy_calibration:
        n = a.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 4 * n, "dispatches": 3}), flush=True)
        return 0

    import attn_inputs as ai
    import causal_attention_attn_amd as ca

    if a.gemm:
        return bench_gemm(a)
    if a.workload == "all":  # one line per benchmark configuration (reported, not the headline)
        for name in ("tiny_f32", "gpt2_small", "decoder_200m", "long_4k", "wide_d128"):
            bench_attention(a, name, cpu_heads=a.cpu_heads or {"long_4k": 6, "wide_d128": 8}.get(name, 0))
        return 0
    return bench_attention(a, a.workload, a.cpu_heads)


def bench_attention(a, workload: str, cpu_heads: int = 0) -> int:
    import numpy as np
    import torch

    import attn_inputs as ai
    import causal_attention_attn_amd as ca

    cfg = ai.CONFIGS[workload]
    inp = ai.make_inputs(cfg)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    import numpy as np

    def up(name):
        x = inp.store[name]
        if cfg.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    Q, K, V, dO = (up(n) for n in ("Q", "K", "V", "dO"))
    packed = a.layout == "packed"
    atomic = a.bwd == "atomic"
    if packed:  # [B, H, T, d] views of GPT-2 layer buffers (see the module docstring)
        qkv = torch.stack([Q, K, V], dim=0).permute(1, 3, 0, 2, 4).contiguous()  # [B, T, 3, H, d]
        Q, K, V = (qkv[:, :, i].permute(0, 2, 1, 3) for i in range(3))
        dO = dO.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        O = torch.empty_like(dO.permute(0, 2, 1, 3)).permute(0, 2, 1, 3)
        dqkv = torch.empty_like(qkv)
        dQ, dK, dV = (dqkv[:, :, i].permute(0, 2, 1, 3) for i in range(3))
    else:
        O = torch.empty_like(Q)
        dQ, dK, dV = torch.empty_like(Q), torch.empty_like(Q), torch.empty_like(Q)
    LSE = torch.empty(Q.shape[:3], dtype=torch.float32, device=dev)
    fwd_fn = ca.attn_fwd_strided if packed else ca.attn_fwd
    bwd_fn = {(False, False): ca.attn_bwd, (False, True): ca.attn_bwd_atomic,
              (True, False): ca.attn_bwd_strided, (True, True): ca.attn_bwd_atomic_strided}[(packed, atomic)]
    dtc = ca.ATTN_BF16 if cfg.dtype == "bf16" else ca.ATTN_F32
    ws_fn = ca.attn_bwd_atomic_workspace_bytes if atomic else ca.attn_bwd_workspace_bytes
    ws = torch.empty(ws_fn(dtc, cfg.B, cfg.H, cfg.T, cfg.d, cfg.causal), dtype=torch.uint8, device=dev)
    s = cfg.scale_f32
    stream = torch.cuda.current_stream()

    def fwd():
        fwd_fn(Q, K, V, O, LSE, s, cfg.causal, stream)

    def bwd():
        bwd_fn(Q, K, V, O, dO, LSE, dQ, dK, dV, ws, s, cfg.causal, stream)

    def step():
        fwd()
        bwd()

    def timed(fn, n):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # untimed warm-up: W steps, and at least WARMUP_S seconds of steps so the
    # GPU has left its idle clock state (short runs can otherwise be timed in
    # a reduced performance state)
    t0 = time.perf_counter()
    nwarm = 0
    while nwarm < a.warmup or time.perf_counter() - t0 < WARMUP_S:
        step()
        nwarm += 1
        if nwarm % 50 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    warm_s = time.perf_counter() - t0
    print("[bench] warmup done (%d steps, %.2f s), timing %d steps of %s" % (nwarm, warm_s, a.steps, cfg.name),
          file=sys.stderr, flush=True)

    # the timed region: K whole steps, each kernel bracketed by a HIP event pair
    # on the launch stream so the dominant kernel's duration is measured live
    ca.attn_prof_enable(4 * a.steps + 8)
    ca.attn_prof_read()
    wall0 = time.perf_counter()
    ms_step = timed(step, a.steps)
    wall = time.perf_counter() - wall0
    kern = ca.attn_prof_read()
    ca.attn_prof_enable(0)
    # forward-only and backward-only passes, without per-kernel events
    ms_fwd = timed(fwd, a.steps)
    ms_bwd = timed(bwd, a.steps)
    ms_step_noev = timed(step, a.steps)
    sclk = sclk_mhz()
    print("[bench] timed: %.4f ms/step (events), %.4f ms/step (no events)" % (ms_step, ms_step_noev),
          file=sys.stderr, flush=True)
    # spread over repeated regions (reported, not the value): each region runs
    # at least K passes and at least 50 ms of them
    spread = {}
    for name, fn, ms1 in (("fwd", fwd, ms_fwd), ("bwd", bwd, ms_bwd), ("step", step, ms_step_noev)):
        n = max(a.steps, int(math.ceil(50.0 / max(ms1, 1e-6))))
        xs = sorted(timed(fn, n) for _ in range(max(a.repeats, 0)))
        if xs:
            spread[name] = {"median_ms": xs[len(xs) // 2], "min_ms": xs[0], "max_ms": xs[-1], "regions": len(xs),
                            "passes_per_region": n}

    tot = flops_units(cfg, 7)
    kernels = {k: {"launches": n, "avg_us": 1000.0 * t / n} for k, (n, t) in kern.items()}
    dom = max(kernels, key=lambda k: kernels[k]["avg_us"])
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    units = dict(UNITS)
    if atomic:  # the dK/dV kernel also forms dQ = s dS K
        units["attn_bwd_dkdv"] = 5
    if dom in units:
        ach = flops_units(cfg, units[dom]) / (kernels[dom]["avg_us"] * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s", "frac": ach / peak}
    else:  # the HBM-bound preprocess: read O and dO, write D
        nbytes = 2 * cfg.B * cfg.H * cfg.T * cfg.d * (2 if cfg.dtype == "bf16" else 4) + 4 * cfg.B * cfg.H * cfg.T
        ach = nbytes / (kernels[dom]["avg_us"] * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS}
    roof["kernel"] = dom
    tr = traffic_for(dom)
    roof["traffic"] = tr

    out = {
        "metric": METRIC,
        "value": tot / (ms_step_noev * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "warmup_steps_run": nwarm,
        "ms_per_step": ms_step_noev,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": "%s: causal attention fwd+bwd B=%d H=%d T=%d head_dim=%d %s, fp32 accumulation"
                               % (cfg.name, cfg.B, cfg.H, cfg.T, cfg.d, cfg.dtype),
                   "B": cfg.B, "H": cfg.H, "T": cfg.T, "head_dim": cfg.d, "causal": cfg.causal,
                   "scale": cfg.scale_f32, "seed": cfg.seed, "layout": a.layout, "bwd": a.bwd},
        "pct_peak": tot / (ms_step_noev * 1e-3) / 1e12 / peak,
        "ms_fwd": ms_fwd,
        "ms_bwd": ms_bwd,
        "tflops_fwd": flops_units(cfg, 2) / (ms_fwd * 1e-3) / 1e12,
        "tflops_bwd": flops_units(cfg, 5) / (ms_bwd * 1e-3) / 1e12,
        "pct_peak_fwd": flops_units(cfg, 2) / (ms_fwd * 1e-3) / 1e12 / peak,
        "pct_peak_bwd": flops_units(cfg, 5) / (ms_bwd * 1e-3) / 1e12 / peak,
        "gbps_fwd": fwd_bytes(cfg) / (ms_fwd * 1e-3) / 1e9,
        "gbps_bwd": bwd_bytes(cfg) / (ms_bwd * 1e-3) / 1e9,
        "spread": spread,
        "sclk_mhz": sclk,
        "cache": "warm: the step's working set fits the 256 MB Infinity Cache",
        "ms_per_step_with_kernel_events": ms_step,
        "kernels": kernels,
        "wall_s_timed_region": wall,
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not a.no_cpu_baseline:
        heads = cpu_heads or cfg.B * cfg.H
        print("[bench] CPU oracle baseline on %d heads, %d threads" % (heads, a.cpu_threads),
              file=sys.stderr, flush=True)
        gpu_out = {n: t.float().cpu().numpy() for n, t in
                   (("O", O), ("LSE", LSE), ("dQ", dQ), ("dK", dK), ("dV", dV))}
        one = not a.no_cpu_one_thread and heads == cfg.B * cfg.H and cfg.name in ("tiny_f32", "gpt2_small")
        out["cpu_baseline"] = cpu_baseline(cfg, inp, heads, a.cpu_threads, gpu_out, one_thread=one)
        if cfg.name != "tiny_f32":
            out["cpu_baseline"]["tiny_f32"] = cpu_tiny_f32(a.cpu_threads)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
