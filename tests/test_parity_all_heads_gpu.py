"""Every (batch, head) pair of the long-context and the wide-head workloads
against the fp64 oracle, on the launch the benchmark times (bf16, max |gpu -
ref| / max |ref| <= 2e-2 per output tensor over all heads).  The oracle runs
in chunks of heads so that progress is printed as it goes."""
import numpy as np
import pytest

import attn_inputs as ai
import oracle
from gpu_util import compare, log, run_gpu

pytestmark = pytest.mark.gpu


# the oracle over every head takes minutes of host time (it prints each chunk)
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["long_4k", "wide_d128"])
def test_all_heads_against_oracle(name):
    cfg = ai.CONFIGS[name]
    inp = ai.make_inputs(cfg)
    gpu = run_gpu(inp, cfg.scale_f32, cfg.causal, label=name)
    flat = lambda x: x.reshape(cfg.B * cfg.H, cfg.T, cfg.d)
    Q, K, V, dO = flat(inp.Q), flat(inp.K), flat(inp.V), flat(inp.dO)
    ref = {n: [] for n in ("dQ", "dK", "dV", "O", "LSE")}
    chunk = 16
    for i in range(0, cfg.B * cfg.H, chunk):
        dQ, dK, dV, O, LSE, _ = oracle.attn_bwd(Q[i:i + chunk], K[i:i + chunk], V[i:i + chunk], dO[i:i + chunk],
                                                cfg.scale_f32, cfg.causal, threads=16)
        for n, x in (("dQ", dQ), ("dK", dK), ("dV", dV), ("O", O), ("LSE", LSE)):
            ref[n].append(x)
        log("%s: oracle heads %d..%d done" % (name, i, min(i + chunk, cfg.B * cfg.H) - 1))
    shape = (cfg.B, cfg.H, cfg.T)
    full = {n: np.concatenate(v).reshape(shape + ((cfg.d,) if n != "LSE" else ())) for n, v in ref.items()}
    errs = compare(gpu, full, cfg.dtype)
    log("%s all %d heads: %s" % (name, cfg.B * cfg.H, errs))
