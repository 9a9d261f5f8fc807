"""Host-side validation of the strided entry points (no GPU): packed QKV
views are accepted, and every output view that could share an element with
another argument is refused.  Accepted calls return ATTN_ELAUNCH here (no HIP
device), so they run only where no GPU is present; refused ones fail before
any HIP call, with fake, never dereferenced addresses.

The overlap rule is a sufficient test; a randomised check compares its
verdicts with brute-force enumeration of the addresses each view touches:
whatever it accepts must be truly disjoint."""
import ctypes
import itertools

import numpy as np
import pytest

import causal_attention_attn_amd as ca

L = ca.lib
MB = 1 << 20
BASE = [0x100000000 + i * 256 * MB for i in range(12)]


def _no_gpu():
    import torch

    return not torch.cuda.is_available()


accepted_only_without_gpu = pytest.mark.skipif(not _no_gpu(), reason="fake pointers must not reach a real launch")


def ll(vals):
    return (ctypes.c_longlong * len(vals))(*vals)


def fwd_s(ptrs, strides, B=2, H=3, T=100, d=64, dt=ca.ATTN_BF16, LSE=BASE[10]):
    Q, K, V, O = ptrs
    st = ll(strides) if strides is not None else None
    return L.attn_fwd_strided(dt, Q, K, V, O, LSE, st, B, H, T, d, ctypes.c_float(0.125), 1, None)


def bwd_s(ptrs, strides, B=2, H=3, T=100, d=64, dt=ca.ATTN_BF16, atomic=False):
    Q, K, V, O, dO, dQ, dK, dV = ptrs
    ws_fn = ca.attn_bwd_atomic_workspace_bytes if atomic else ca.attn_bwd_workspace_bytes
    fn = L.attn_bwd_atomic_strided if atomic else L.attn_bwd_strided
    st = ll(strides) if strides is not None else None
    return fn(dt, Q, K, V, O, dO, BASE[10], dQ, dK, dV, BASE[11], ws_fn(dt, B, H, T, d), st, B, H, T, d,
              ctypes.c_float(0.125), 1, None)


def packed(B, H, T, d, eb, base):
    """Q, K, V views of one [B, T, 3, H, d] buffer: pointers and strides."""
    s = [T * 3 * H * d, d, 3 * H * d]
    return [base + i * H * d * eb for i in range(3)], s * 3


def bthd(B, H, T, d):
    return [T * H * d, d, H * d]  # [B, T, H, d], i.e. O as [B, T, H*d]


@accepted_only_without_gpu
@pytest.mark.parametrize("atomic", [False, True])
def test_packed_qkv_and_packed_gradients_are_accepted(atomic):
    B, H, T, d, eb = 2, 3, 100, 64, 2
    qkv, s_qkv = packed(B, H, T, d, eb, BASE[0])
    assert fwd_s(qkv + [BASE[1]], s_qkv + bthd(B, H, T, d)) == ca.ATTN_ELAUNCH
    dqkv, s_dqkv = packed(B, H, T, d, eb, BASE[4])
    ptrs = qkv + [BASE[1], BASE[2]] + dqkv
    assert bwd_s(ptrs, s_qkv + bthd(B, H, T, d) * 2 + s_dqkv, atomic=atomic) == ca.ATTN_ELAUNCH


@accepted_only_without_gpu
def test_contiguous_strides_and_ignored_extent_one_strides_are_accepted():
    B, H, T, d = 2, 3, 100, 64
    c = [H * T * d, T * d, d]
    assert fwd_s(BASE[:4], c * 4) == ca.ATTN_ELAUNCH
    # B = 1: the batch stride never multiplies a non-zero index, any value passes
    assert fwd_s(BASE[:4], [-7, T * d, d] * 4, B=1) == ca.ATTN_ELAUNCH
    # broadcast inputs (one K/V head shared by every query head) are allowed
    kv = [T * d, 0, d]
    assert fwd_s(BASE[:4], c + kv + kv + c) == ca.ATTN_ELAUNCH


@accepted_only_without_gpu
def test_output_interleaved_with_inputs_in_one_buffer_is_accepted():
    # [B, T, 4, H, d]: q, k, v and o slices of one buffer
    B, H, T, d, eb = 2, 3, 100, 64, 2
    s = [T * 4 * H * d, d, 4 * H * d]
    ptrs = [BASE[0] + i * H * d * eb for i in range(4)]
    assert fwd_s(ptrs, s * 4) == ca.ATTN_ELAUNCH


def test_null_strides():
    assert fwd_s(BASE[:4], None) == ca.ATTN_EINVAL
    assert "strides is null" in ca.attn_last_error()
    assert bwd_s(BASE[:8], None) == ca.ATTN_EINVAL
    assert "strides is null" in ca.attn_last_error()


@pytest.mark.parametrize("mutate,msg", [
    (lambda s: s.__setitem__(2, -64), "negative stride"),
    (lambda s: s.__setitem__(5, 68), "multiple of 16 bytes"),       # 136 bytes in bf16
    (lambda s: s.__setitem__(11, 0), "several elements to one address"),  # O token stride 0
    (lambda s: s.__setitem__(10, 32), "several elements to one address"),  # O heads 32 apart, d = 64
    (lambda s: s.__setitem__(9, 1 << 62), "overflows"),
])
def test_fwd_stride_errors(mutate, msg):
    B, H, T, d = 2, 3, 100, 64
    s = [H * T * d, T * d, d] * 4
    mutate(s)
    assert fwd_s(BASE[:4], s) == ca.ATTN_EINVAL
    assert msg in ca.attn_last_error()


def test_packed_gradients_that_collide_are_refused():
    B, H, T, d, eb = 2, 3, 100, 64, 2
    qkv, s_qkv = packed(B, H, T, d, eb, BASE[0])
    dqkv, s_dqkv = packed(B, H, T, d, eb, BASE[4])
    o2 = bthd(B, H, T, d) * 2
    # dK on top of dQ
    ptrs = qkv + [BASE[1], BASE[2], dqkv[0], dqkv[0], dqkv[2]]
    assert bwd_s(ptrs, s_qkv + o2 + s_dqkv) == ca.ATTN_EINVAL
    assert "output dQ overlaps output dK" in ca.attn_last_error()
    # dK half a head row after dQ: the slices interleave element-wise
    ptrs = qkv + [BASE[1], BASE[2], dqkv[0], dqkv[0] + 32 * eb, dqkv[2]]
    assert bwd_s(ptrs, s_qkv + o2 + s_dqkv) == ca.ATTN_EINVAL
    assert "output dQ overlaps output dK" in ca.attn_last_error()
    # gradients written in place over the packed inputs
    ptrs = qkv + [BASE[1], BASE[2]] + qkv
    assert bwd_s(ptrs, s_qkv + o2 + s_qkv) == ca.ATTN_EINVAL
    assert "output dQ overlaps input Q" in ca.attn_last_error()
    # same buffer, different strides: refused even where a finer test might accept
    ptrs = qkv + [BASE[1], BASE[2], dqkv[0], dqkv[1], dqkv[2]]
    s = s_qkv + o2 + s_dqkv
    s[18:21] = [T * 3 * H * d, d, 3 * H * d + 0]  # dK as given
    s[15:18] = [T * 3 * H * d, 3 * d, 3 * H * d]  # dQ heads spread out: strides differ from dK's
    assert bwd_s(ptrs, s) == ca.ATTN_EINVAL
    assert "overlaps" in ca.attn_last_error()


def test_workspace_and_lse_stay_contiguous_and_are_checked_against_views():
    B, H, T, d, eb = 2, 3, 100, 64, 2
    qkv, s_qkv = packed(B, H, T, d, eb, BASE[0])
    # O starts inside LSE's range
    assert L.attn_fwd_strided(ca.ATTN_BF16, qkv[0], qkv[1], qkv[2], BASE[10] + 256, BASE[10],
                              ll(s_qkv + bthd(B, H, T, d)), B, H, T, d, ctypes.c_float(0.1), 1, None) == ca.ATTN_EINVAL
    assert "overlaps output LSE" in ca.attn_last_error()


# ---- the overlap rule against brute force ------------------------------------

def _offsets(base_el, s, B, H, T, d):
    b, h, t, c = np.meshgrid(np.arange(B), np.arange(H), np.arange(T), np.arange(d), indexing="ij")
    return (base_el + b * s[0] + h * s[1] + t * s[2] + c).ravel()


@accepted_only_without_gpu
def test_overlap_rule_is_sound_against_enumeration():
    """Random small views, fp32 (strides in multiples of 4 elements): every
    output the library accepts is injective, and every accepted pair of
    outputs (and output/input) is disjoint."""
    rng = np.random.default_rng(20260731)
    d = 32
    cands = [0, 4, 8, 16, 32, 64, 96, 128, 192, 256, 384, 512]
    n_accept = 0
    for trial in range(400):
        B, H, T = (int(x) for x in rng.integers(1, 4, size=3))
        s = [int(rng.choice(cands)) for _ in range(12)]
        ptr_el = [0] + [int(rng.choice([0, 32, 64, 96, 128, 512, 4096])) for _ in range(3)]
        # Q, K, V, O all in one region of fake memory, offsets in elements
        ptrs = [BASE[0] + 4 * p for p in ptr_el]
        st = fwd_s(ptrs, s, B=B, H=H, T=T, d=d, dt=ca.ATTN_F32, LSE=BASE[10])
        o = _offsets(ptr_el[3], s[9:12], B, H, T, d)
        truly_ok = len(np.unique(o)) == o.size
        for i in range(3):
            truly_ok = truly_ok and not np.intersect1d(o, _offsets(ptr_el[i], s[3 * i:3 * i + 3], B, H, T, d)).size
        if st == ca.ATTN_ELAUNCH:
            n_accept += 1
            assert truly_ok, (B, H, T, s, ptr_el)
        else:
            assert st == ca.ATTN_EINVAL
    assert n_accept > 20  # the random draws exercise the accepting branch too


def test_token_stride_beyond_32bit_row_offsets_is_unsupported():
    # packed QKV rows of 3*H*d = 2304 elements over 2^20 tokens: slab offsets pass 2^31
    B, H, T, d, eb = 1, 12, 1 << 20, 64, 2
    qkv, s_qkv = packed(B, H, T, d, eb, BASE[0])
    assert fwd_s(qkv + [BASE[1]], s_qkv + bthd(B, H, T, d), B=B, H=H, T=T, d=d) == ca.ATTN_EUNSUPPORTED
    assert "2^31-1" in ca.attn_last_error()
