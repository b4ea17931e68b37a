"""Pins for the oracle's E4M3 codec: the OFP8 definition (hand-derived golden
values), exhaustive round trips, rounding at every midpoint, and torch's own
float32 -> float8_e4m3fn cast as an independent library routine."""

import os

import numpy as np
import pytest
import torch

from oracle import mla_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_e4m3_examples.txt")


def _torch_cast(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_golden_hand_derived_codes():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        v, code = line.split()[:2]
        rows.append((float(v), int(code, 16)))
    assert len(rows) >= 15
    for v, code in rows:
        got = int(O.fp8_e4m3fn_encode(np.array([v], dtype=np.float32))[0])
        assert got == code, (v, hex(got), hex(code))


def test_decode_table_matches_torch_and_definition():
    table = O.fp8_e4m3fn_decode_table()
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(table), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(table[~nan], ref[~nan])
    assert table[0x7E] == 448.0 and table[0x08] == 2.0 ** -6 and table[0x01] == 2.0 ** -9
    assert table[0x38] == 1.0 and table[0x80] == 0.0 and np.signbit(table[0x80])


def test_round_trip_every_code():
    table = O.fp8_e4m3fn_decode_table()
    codes = np.array([c for c in range(256) if not np.isnan(table[c])], dtype=np.uint8)
    vals = table[codes].astype(np.float32)
    assert np.array_equal(O.fp8_e4m3fn_encode(vals), codes)


def test_midpoints_round_to_even_and_neighbours_to_nearest():
    table = O.fp8_e4m3fn_decode_table()
    pos = table[:0x7F]
    for c in range(0x7E):
        lo, hi = pos[c], pos[c + 1]
        mid = np.float32((lo + hi) / 2)          # exact: one more bit than E4M3 has
        assert float(mid) == (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert O.fp8_e4m3fn_encode(np.array([mid]))[0] == even
        assert O.fp8_e4m3fn_encode(np.array([-mid]))[0] == (even | 0x80)
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(1e9))
        assert O.fp8_e4m3fn_encode(np.array([below]))[0] == c
        assert O.fp8_e4m3fn_encode(np.array([above]))[0] == c + 1


def test_random_fp32_matches_torch_below_464():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(400_000).astype(np.float32) * 100,
        rng.standard_normal(200_000).astype(np.float32) * 0.01,
        rng.uniform(-463.9, 463.9, 200_000).astype(np.float32),
        (rng.standard_normal(200_000) * 2.0 ** rng.integers(-20, 9, 200_000)).astype(np.float32),
    ])
    x = x[np.abs(x) < 464]
    assert np.array_equal(O.fp8_e4m3fn_encode(x), _torch_cast(x))


def test_every_bf16_pattern_divided_by_scale_matches_torch():
    # all 65536 bf16 patterns as the fp8 write sees them: x_f32 / scale_f32
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = O.bf16_bits_to_f64(bits).astype(np.float32)
    for scale in [np.float32(1.0), np.float32(9.5 / 448.0), np.float32(0.0213), np.float32(3.7)]:
        with np.errstate(invalid="ignore", over="ignore"):
            y = x / scale
        finite = np.isfinite(y) & (np.abs(y) < 464)
        assert np.array_equal(O.fp8_e4m3fn_encode(y[finite]), _torch_cast(y[finite]))
        big = np.isfinite(y) & (np.abs(y) >= 464)
        got = O.fp8_e4m3fn_encode(y[big])
        assert np.all((got & 0x7F) == 0x7E)
        assert np.array_equal(got >> 7, np.signbit(y[big]).astype(np.uint8))


def test_saturation_and_nan():
    x = np.array([448.0, 463.99, 464.0, 1e6, np.inf, -np.inf, -470.0, np.nan, -np.nan], dtype=np.float32)
    got = O.fp8_e4m3fn_encode(x)
    assert got.tolist()[:7] == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert got[7] & 0x7F == 0x7F


def test_bf16_helpers_match_torch():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(100_000) * 10.0 ** rng.integers(-30, 30, 100_000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_bf16_bits_rne(x), ref)
    back = O.bf16_bits_to_f64(ref)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy())
