"""Pins for the oracle's rotary embedding (non-NeoX, interleaved pairs) and
the RoPE-fused cache write: complex multiplication in float64, exact special
angles, norm preservation, position 0, and the write's layout (kv_c columns
as the plain write, k_pe columns rotated, padded tokens skipped)."""

import math

import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from mla_paged_decode_concat_amd import workloads as W


def test_rotation_is_complex_multiplication_of_interleaved_pairs():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((50, 64)).astype(np.float32)
    ang = rng.uniform(-math.pi, math.pi, (50, 32))
    c = np.cos(ang).astype(np.float32)
    s = np.sin(ang).astype(np.float32)
    got = O.rope_rotate_f32(x, c, s).astype(np.float64)
    z = x[:, 0::2].astype(np.float64) + 1j * x[:, 1::2].astype(np.float64)
    want = z * (c.astype(np.float64) + 1j * s.astype(np.float64))
    bound = 2.0 ** -23 * (np.abs(x[:, 0::2]) + np.abs(x[:, 1::2])).astype(np.float64) + 1e-45
    assert np.all(np.abs(got[:, 0::2] - want.real) <= bound)
    assert np.all(np.abs(got[:, 1::2] - want.imag) <= bound)


def test_exact_angles():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((8, 64)).astype(np.float32)
    one, zero = np.ones((8, 32), np.float32), np.zeros((8, 32), np.float32)
    assert np.array_equal(O.rope_rotate_f32(x, one, zero), x)              # angle 0
    r90 = O.rope_rotate_f32(x, zero, one)                                   # a quarter turn
    assert np.array_equal(r90[:, 0::2], -x[:, 1::2]) and np.array_equal(r90[:, 1::2], x[:, 0::2])
    r180 = O.rope_rotate_f32(x, -one, zero)
    assert np.array_equal(r180, -x)


def test_norm_and_inverse():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((30, 64)).astype(np.float32)
    ang = rng.uniform(0, 2 * math.pi, (30, 32))
    c, s = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    y = O.rope_rotate_f32(x, c, s)
    n0 = np.hypot(x[:, 0::2].astype(np.float64), x[:, 1::2].astype(np.float64))
    n1 = np.hypot(y[:, 0::2].astype(np.float64), y[:, 1::2].astype(np.float64))
    assert np.max(np.abs(n1 - n0) / np.maximum(n0, 1e-30)) < 1e-6
    back = O.rope_rotate_f32(y, c, -s)
    assert np.max(np.abs(back - x)) < 1e-5


def test_table_layout_and_position_zero():
    tab = W.rope_table(100, 64).numpy()
    assert tab.shape == (100, 64) and np.all(tab[0, :32] == 1) and np.all(tab[0, 32:] == 0)
    c, s = O.rope_table_rows(tab, np.array([0, 7]), 64)
    assert np.allclose(c[1] ** 2 + s[1] ** 2, 1, atol=1e-6)
    assert abs(c[1, 0] - math.cos(7.0)) < 1e-7 and abs(s[1, 1] - math.sin(7.0 * 10000 ** (-2 / 64))) < 1e-7


@pytest.mark.parametrize("in_dtype,cache_dtype", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "fp8"), ("f32", "fp8")])
def test_cache_write_rope_layout(in_dtype, cache_dtype):
    rng = np.random.default_rng(8)
    nb, bs, R, P, T = 4, 4, 512, 64, 9
    if in_dtype == "f32":
        kv_c = rng.standard_normal((T, R)).astype(np.float32)
        k_pe = rng.standard_normal((T, P)).astype(np.float32)
    else:
        kv_c = O.f32_to_bf16_bits_rne(rng.standard_normal((T, R)).astype(np.float32))
        k_pe = O.f32_to_bf16_bits_rne(rng.standard_normal((T, P)).astype(np.float32))
    slots = np.array([3, -1, 0, 15, 8, -1, 1, 12, 5], dtype=np.int64)
    pos = np.array([0, 999, 5, 17, 2, 999, 40, 63, 1], dtype=np.int64)   # 999: never read
    tab = W.rope_table(64, P).numpy()
    fill = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "fp8": np.uint8(0x7F)}[cache_dtype]
    dt = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[cache_dtype]
    cache = np.full((nb, bs, R + P), fill, dtype=dt)
    scale = 0.01 if cache_dtype == "fp8" else None
    plain = O.cache_write(cache, kv_c, k_pe, slots, in_dtype, cache_dtype, scale)
    out = O.cache_write_rope(cache, kv_c, k_pe, pos, tab, slots, in_dtype, cache_dtype, scale)
    assert np.array_equal(out[..., :R].view(np.uint8), plain[..., :R].view(np.uint8))
    for t, sl in enumerate(slots):
        row = out[sl // bs, sl % bs, R:] if sl >= 0 else None
        if sl < 0:
            continue
        x = O.to_f32_exact(k_pe[t], in_dtype).astype(np.float64)
        ang = pos[t] * 10000.0 ** (-np.arange(0, P, 2) / P)
        z = (x[0::2] + 1j * x[1::2]) * np.exp(1j * ang)
        want = np.empty(P)
        want[0::2], want[1::2] = z.real, z.imag
        got = O.to_f64(row, cache_dtype) * (scale if cache_dtype == "fp8" else 1.0)
        tol = {"f32": 1e-5, "bf16": 2.0 ** -7 * 4, "fp8": 0.5 * 4}[cache_dtype]
        assert np.max(np.abs(got - want)) <= tol * (1 if cache_dtype != "fp8" else scale * 64)
    written = np.zeros((nb, bs), bool)
    written[slots[slots >= 0] // bs, slots[slots >= 0] % bs] = True
    assert np.array_equal(out[~written].view(np.uint8), cache[~written].view(np.uint8))


def test_rope_q_touches_only_the_rope_part():
    rng = np.random.default_rng(9)
    q = O.f32_to_bf16_bits_rne(rng.standard_normal((3, 4, 576)).astype(np.float32))
    tab = W.rope_table(32, 64).numpy()
    pos = np.array([0, 31, 4])
    out = O.rope_q(q, pos, tab, "bf16", 512)
    assert np.array_equal(out[..., :512], q[..., :512])
    assert np.array_equal(out[0], q[0])                      # position 0: identity
    x = O.bf16_bits_to_f64(q[1, 2, 512:])
    ang = 31 * 10000.0 ** (-np.arange(0, 64, 2) / 64)
    z = (x[0::2] + 1j * x[1::2]) * np.exp(1j * ang)
    got = O.bf16_bits_to_f64(out[1, 2, 512:])
    assert np.max(np.abs(got[0::2] - z.real)) < 2.0 ** -6 and np.max(np.abs(got[1::2] - z.imag)) < 2.0 ** -6
