"""Pins of the oracle's FP8 (E4M3) codec and quantiser.  CPU only.

The oracle's table is built from the format's definition; here it is
checked against torch's float8_e4m3fn (a library implementation the oracle
does not call), against hand-worked values, and its rounding against exact
midpoints and brute force."""

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8


def test_code_values_match_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = fp8.E4M3_VALUES
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_hand_worked_values():
    v = fp8.E4M3_VALUES
    assert v[0x38] == 1.0           # exponent 7 (bias 7), mantissa 0
    assert v[0x7E] == 448.0         # 1.75 * 2^8, the largest finite value
    assert v[0x08] == 2.0**-6       # smallest normal
    assert v[0x01] == 2.0**-9       # smallest subnormal
    assert v[0x07] == 7 * 2.0**-9   # largest subnormal
    assert v[0x3C] == 1.5
    assert v[0xC0] == -2.0
    assert v[0x80] == 0.0 and np.signbit(v[0x80])
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.count_nonzero(np.isnan(v)) == 2  # no infinities, two NaNs


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(fp8.fp8_encode(fp8.E4M3_VALUES[codes]), codes)


def test_midpoints_round_to_even_codes():
    pos = fp8.E4M3_VALUES[:0x7F]
    for c in range(0x7E):
        mid = (pos[c] + pos[c + 1]) / 2  # exact in float64
        even = c if c % 2 == 0 else c + 1
        assert fp8.fp8_encode(mid) == even, hex(c)
        assert fp8.fp8_encode(-mid) == (even | 0x80)
        assert fp8.fp8_encode(np.nextafter(mid, 0)) == c
        assert fp8.fp8_encode(np.nextafter(mid, np.inf)) == c + 1


def test_encode_matches_brute_force_nearest():
    rng = np.random.default_rng(0)
    y = np.concatenate([rng.standard_normal(3000) * 30, np.exp2(rng.uniform(-12, 8.8, 3000)) * rng.choice([-1, 1], 3000)])
    pos = fp8.E4M3_VALUES[:0x7F]
    for v in y:
        a = min(abs(v), 448.0)
        d = np.abs(pos - a)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert fp8.fp8_encode(v) == (want | (0x80 if v < 0 else 0))


def test_encode_matches_torch_in_range():
    # torch's float32 -> float8_e4m3fn conversion rounds to nearest even; it
    # does not saturate, so only magnitudes <= 448 are compared.
    rng = np.random.default_rng(1)
    pos = fp8.E4M3_VALUES[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    y = np.concatenate([
        rng.standard_normal(20000) * 40,
        np.exp2(rng.uniform(-14, 8.8, 20000)) * rng.choice([-1, 1], 20000),
        mids, -mids, pos, -pos,
    ]).astype(np.float32)
    y = y[np.abs(y) <= 448]
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.fp8_encode(y), ref)


def test_saturation_nan_and_signed_zero():
    enc = fp8.fp8_encode
    for v in (448.0, 449.0, 463.99, 464.0, 480.0, 1e6, np.inf):
        assert enc(v) == 0x7E and enc(-v) == 0xFE
    assert enc(np.nan) == 0x7F
    assert enc(0.0) == 0x00 and enc(-0.0) == 0x80
    assert enc(2.0**-10) == 0x00          # tie between 0 and 2^-9 -> even (0)
    assert enc(3 * 2.0**-10) == 0x02      # tie between 0x01 and 0x02 -> 0x02
    assert enc(-1e-30) == 0x80            # underflow keeps the sign


def test_quantiser_error_bound_and_power_of_two_scale():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(50000)).astype(np.float16)
    for s in (2.0**-6, 0.0123, 0.37):
        q = fp8.fp8_quantize(x, s)
        back = fp8.fp8_dequantize(q, s)
        xf = x.astype(np.float64)
        sf = float(np.float32(s))
        y = np.abs(xf / sf)
        inside = y <= 448
        # half a unit in the last place: 2^-4 relative for normals, 2^-10 absolute below 2^-6
        bound = np.maximum(np.abs(xf) * 2.0**-4, 2.0**-10 * sf) * (1 + 1e-6)
        assert np.all(np.abs(back - xf)[inside] <= bound[inside])
        assert np.all(np.abs(back[~inside]) == 448 * sf)
    # A power-of-two scale only moves the exponent: quantising x with scale
    # 2^-6 is encoding 64 x.
    assert np.array_equal(fp8.fp8_quantize(x, 2.0**-6), fp8.fp8_encode(x.astype(np.float64) * 64))


def test_fp8_scatter_writes_quantised_codes():
    rng = np.random.default_rng(3)
    NB, H, B, D = 4, 2, 16, 8
    kc = np.full((NB, H, 2, B, D // 2), 0x55, np.uint8)  # key tiles in 4-code chunks
    vc = np.full((NB, H, D, B), 0x55, np.uint8)
    key = rng.standard_normal((3, H, D)).astype(np.float16)
    val = rng.standard_normal((3, H, D)).astype(np.float16)
    slots = np.array([5, -1, 40])
    fp8.reshape_and_cache_fp8(kc, vc, key, val, slots, 0.05, 0.02)
    assert np.array_equal(kc[0, :, :, 5].reshape(H, D), fp8.fp8_quantize(key[0], 0.05))
    assert np.array_equal(vc[2, :, :, 8], fp8.fp8_quantize(val[2], 0.02))
    assert np.count_nonzero(kc != 0x55) <= 2 * H * D  # the padding token wrote nothing
