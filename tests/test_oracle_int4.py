"""Pins for the int4 KV codec oracle (CPU only).

Checked against: hand-derived worked examples (tests/golden: a 0.25 grid, half-even
ties, a range whose fifteenth is not an fp32 number so the scale's fp32-then-fp16
rounding decides a code, and a minimum that rounds to an fp16 zero of -0), a
brute-force nearest code search, exact rational arithmetic for the dequantised value,
the error bound the format implies, and degenerate inputs.  Planted mistakes (wrong
nibble order, round half away from zero, scale left in fp32, zero not rounded to
fp16) are shown to fail a pin.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from mixed_head_kv_amd.inputs import f32_to_bf16_bits, bf16_bits_to_f32
from oracle import int4 as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "int4_worked_example.json")


def _bf16(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_golden_worked_examples():
    for c in json.load(open(GOLDEN))["cases"]:
        bits = _bf16(c["x"])
        assert np.array_equal(bf16_bits_to_f32(bits), np.asarray(c["x"], np.float32)), "fixture not bf16-exact"
        codes, s, z = Q.quantize(bits)
        assert int(s.view(np.uint16)) == c["scale_bits"], c["name"]
        assert int(z.view(np.uint16)) == c["zero_bits"], c["name"]
        assert codes.tolist() == c["codes"], c["name"]


def test_grid_example_round_trips_exactly():
    c = json.load(open(GOLDEN))["cases"][0]
    codes, s, z = Q.quantize(_bf16(c["x"]))
    assert np.array_equal(Q.dequantize(codes, s, z), np.asarray(c["x"], np.float32))


def _rand_bits(seed, n, scale=1.0):
    rng = np.random.default_rng(seed)
    return _bf16(rng.standard_normal((n, 128)).astype(np.float32) * np.float32(scale))


@pytest.mark.parametrize("scale", [1.0, 1e-3, 300.0])
def test_codes_in_range_and_error_bound(scale):
    bits = _rand_bits(1, 500, scale)
    codes, s, z = Q.quantize(bits)
    q = Q.unpack(codes)
    assert q.max() <= 15 and codes.shape == (500, 64)
    x = bf16_bits_to_f32(bits).astype(np.float64)
    xh = Q.dequantize(codes, s, z).astype(np.float64)
    s64 = s.astype(np.float64)[:, None]
    mn = x.min(axis=1, keepdims=True)
    # half a step, plus the fp16 rounding of the zero, plus the clamp at the top end
    # (the fp16 scale can round 15*s below the range by at most 15 * half an fp16 ulp of s)
    bound = 0.5 * s64 + np.abs(z.astype(np.float64)[:, None] - mn) + 15 * s64 * 2.0 ** -11 + 1e-30
    assert np.all(np.abs(xh - x) <= bound * (1 + 1e-6))


def test_codes_are_nearest_grid_points():
    """Brute force over all 16 codes on the grid (x - z)/s, in fp32 as the format fixes."""
    bits = _rand_bits(2, 200)
    codes, s, z = Q.quantize(bits)
    q = Q.unpack(codes).astype(np.int64)
    x = bf16_bits_to_f32(bits)
    t = ((x - z.astype(np.float32)[:, None]).astype(np.float32) / s.astype(np.float32)[:, None]).astype(np.float64)
    for r in range(x.shape[0]):
        for k in range(128):
            dist = [abs(t[r, k] - c) for c in range(16)]
            best = min(dist)
            cands = [c for c in range(16) if dist[c] == best]
            if len(cands) == 1:
                assert q[r, k] == cands[0]
            else:
                assert q[r, k] in cands and q[r, k] % 2 == 0


def test_degenerate_vector_gives_zero_codes():
    bits = _bf16(np.full(128, 0.7, np.float32))
    codes, s, z = Q.quantize(bits[None])
    assert float(s[0]) == 0.0 and not codes.any()
    assert np.all(Q.dequantize(codes, s, z) == np.float32(np.float16(bf16_bits_to_f32(bits)[0])))


def test_tiny_range_rounds_scale_to_zero_or_subnormal():
    x = np.zeros(128, np.float32)
    x[5] = np.float32(2.0 ** -40)
    codes, s, z = Q.quantize(_bf16(x)[None])
    assert float(s[0]) == 0.0 and not codes.any()
    x[5] = np.float32(2.0 ** -20)  # 2^-20/15 is an fp16 subnormal
    codes, s, z = Q.quantize(_bf16(x)[None])
    assert 0 < float(s[0]) < 6.2e-5
    assert Q.unpack(codes)[0, 5] == 15


def _rn_f32(fr: Fraction) -> np.float32:
    """Exact round-to-nearest-even of a rational to float32."""
    c = np.float32(float(fr))
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - fr)
        key = (d, int(np.float32(cand).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return np.float32(best[1])


def test_dequant_equals_exact_rounding_of_q_s_plus_z():
    """x_hat = RN_fp32(q*s + z) computed exactly with rationals, over every code and a
    sweep of fp16 scales and zeros (normal and subnormal).  This is the exactness
    argument: q*s is exact, so FMA and multiply-then-add agree."""
    rng = np.random.default_rng(3)
    s_vals = np.concatenate([np.array([2.0 ** -24, 2.0 ** -20, 6.0e-5, 1.0, 0.25, 3.0e4]),
                             np.abs(rng.standard_normal(40)) * 0.5]).astype(np.float16)
    z_vals = np.concatenate([np.array([0.0, -1.0, 2.0 ** -24, -6.0e4]),
                             rng.standard_normal(40) * 3]).astype(np.float16)
    for s in s_vals:
        for z in z_vals:
            codes = np.array([[k | ((k + 1) % 16) << 4 for k in range(0, 16, 2)] * 8], np.uint8)
            xh = Q.dequantize(codes, np.array([s]), np.array([z]))[0]
            q = Q.unpack(codes)[0]
            for k in range(16):
                exact = Fraction(int(q[k])) * Fraction(float(s)) + Fraction(float(z))
                assert xh[k] == _rn_f32(exact)


def test_nibble_order_is_low_then_high():
    x = np.zeros(128, np.float32)
    x[0], x[1] = -1.0, 2.75      # s = 0.25, z = -1
    x[2] = 2.75                  # element 2 -> code 15 in the low nibble of byte 1
    codes, s, z = Q.quantize(_bf16(x)[None])
    assert codes[0, 0] == (0 | (15 << 4))
    assert codes[0, 1] == (15 | (4 << 4))


# --- planted mistakes -------------------------------------------------------------

def test_planted_round_half_away_is_caught(monkeypatch):
    monkeypatch.setattr(Q.np, "rint", lambda t: np.floor(t + 0.5))
    c = json.load(open(GOLDEN))["cases"][1]
    codes, _, _ = Q.quantize(_bf16(c["x"]))
    assert codes.tolist() != c["codes"]


def test_planted_nibble_swap_is_caught():
    c = json.load(open(GOLDEN))["cases"][0]
    codes, s, z = Q.quantize(_bf16(c["x"]))
    swapped = ((codes >> 4) | (codes << 4)).astype(np.uint8)
    assert swapped.tolist() != c["codes"]
    assert not np.array_equal(Q.dequantize(swapped, s, z), np.asarray(c["x"], np.float32))


def _golden(name):
    return next(c for c in json.load(open(GOLDEN))["cases"] if c["name"] == name)


def test_planted_scale_left_in_fp32_is_caught(monkeypatch):
    """A quantiser that divides by the fp32 quotient instead of its fp16 rounding puts
    x = 0 of the inexact-range example in code 7 instead of 8."""
    c = _golden("inexact_range_over_15")
    monkeypatch.setattr(Q, "_scale_fp16", lambda s32: np.asarray(s32, dtype=np.float32))
    codes, _, _ = Q.quantize(_bf16(c["x"]))
    assert codes.tolist() != c["codes"]


def test_planted_zero_not_rounded_to_fp16_is_caught(monkeypatch):
    """A quantiser that subtracts the unrounded minimum moves every code of the
    subnormal-grid example up by one."""
    c = _golden("zero_rounds_to_fp16_subnormal_grid")
    monkeypatch.setattr(Q, "_zero_fp16", lambda mn: np.asarray(mn, dtype=np.float32))
    codes, _, _ = Q.quantize(_bf16(c["x"]))
    assert codes.tolist() != c["codes"]
