"""The seeded input generator: determinism, shapes, and bfloat16 rounding
(round to nearest, ties to even) checked against torch's own float32 ->
bfloat16 conversion (CPU only)."""
import numpy as np
import torch

import attn_inputs as ai


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 3,
        # exact ties: low 16 bits == 0x8000, both parities of bit 16
        (np.arange(1000, dtype=np.uint32) << 17 | 0x3F808000).view(np.float32),
        (np.arange(1000, dtype=np.uint32) << 17 | 0x3F818000).view(np.float32),
        np.array([0.0, -0.0, 1e-40, -1e-40, 3.3e38], dtype=np.float32),
    ])
    ours = ai.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = ai.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_inputs_are_seeded_and_shaped():
    cfg = ai.with_shape(ai.CONFIGS["gpt2_small"], B=1, H=2, T=40)
    a, b = ai.make_inputs(cfg), ai.make_inputs(cfg)
    for n in ("Q", "K", "V", "dO"):
        x, y = getattr(a, n), getattr(b, n)
        assert x.shape == (1, 2, 40, 64) and x.dtype == np.float32
        assert np.array_equal(x, y)
        assert a.store[n].dtype == np.uint16
        assert np.array_equal(ai.bf16_bits_to_f32(a.store[n]), x)
    c = ai.make_inputs(cfg, seed=99)
    assert not np.array_equal(a.Q, c.Q)
    # dO is drawn with sigma 0.1 for this workload
    assert 0.05 < float(np.std(a.dO)) < 0.2 and 0.8 < float(np.std(a.Q)) < 1.2


def test_tiny_config_is_f32_and_exact():
    cfg = ai.CONFIGS["tiny_f32"]
    a = ai.make_inputs(cfg)
    assert a.Q.dtype == np.float32 and a.store["Q"].dtype == np.float32
    assert cfg.scale_f32 == float(np.float32(1 / np.sqrt(32)))


def test_long_context_qk_scaled_by_two():
    cfg = ai.with_shape(ai.CONFIGS["long_4k"], B=1, H=1, T=2048)
    a = ai.make_inputs(cfg)
    assert 1.8 < float(np.std(a.Q)) < 2.2 and 1.8 < float(np.std(a.K)) < 2.2
    assert 0.9 < float(np.std(a.V)) < 1.1
