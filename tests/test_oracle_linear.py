"""Pins for the projection / rotary-encoding oracle (CPU only).

Checked against: exact integer arithmetic in pure Python (the 8-bit linear layer),
closed-form rotations (a quarter turn moves dim d onto dim d + D/2), the frequencies'
closed forms, the complex-number form of the rotation (a different routine: NumPy
complex exponentials), and the invariants that define a rotary encoding (identity at
position 0, norms kept, scores depend only on the relative position).  Planted
mistakes (interleaved pairing, reversed rotation, unrotated keys, swapped K/V
sections) are shown to fail a pin.
"""

from fractions import Fraction

import numpy as np
import pytest

from mixed_head_kv_amd import inputs as I
from oracle import linear as L


def test_w8_linear_matches_exact_integer_arithmetic():
    rng = np.random.default_rng(0)
    M, K, N = 5, 37, 11
    x = rng.integers(-8, 9, (M, K)).astype(np.float64) / 4          # exact quarter steps
    codes = rng.integers(-127, 128, (N, K)).astype(np.int8)
    scales = 2.0 ** rng.integers(-12, -2, N).astype(np.float64)     # powers of two
    got = L.w8_linear(x, codes, scales.astype(np.float32))
    for m in range(M):
        for n in range(N):
            ref = sum(Fraction(x[m, k]) * int(codes[n, k]) for k in range(K)) * Fraction(scales[n])
            assert Fraction(got[m, n]) == ref, (m, n)


def test_w8_linear_uses_each_channel_scale_on_its_own_row():
    codes = np.array([[1, 0], [0, 1], [1, 1]], dtype=np.int8)
    y = L.w8_linear(np.array([[3.0, 5.0]]), codes, np.array([2.0, 0.5, 0.25], dtype=np.float32))
    assert y.tolist() == [[6.0, 2.5, 2.0]]


def test_frequencies_closed_forms():
    th = L.rope_frequencies(128, 10000.0)
    assert th.shape == (64,)
    assert th[0] == 1.0
    assert th[32] == pytest.approx(0.01, rel=1e-15)                  # 10000 ** -0.5
    assert th[16] == pytest.approx(0.1, rel=1e-15)                   # 10000 ** -0.25
    th3 = L.rope_frequencies(128, 500000.0)
    assert th3[32] == pytest.approx(1.0 / np.sqrt(500000.0), rel=1e-15)
    assert np.allclose(th[1:] / th[:-1], 10000.0 ** (-2.0 / 128), rtol=1e-14)


def test_quarter_turn_moves_d_onto_d_plus_half():
    # D = 4, theta = (1, base^-1/2); position pi/2 turns pair (0, 2) by a quarter
    D = 4
    e = np.eye(D)[:, None, :]                                        # 4 tokens, 1 head
    out = L.rope(e, np.full(4, np.pi / 2), 100.0)[:, 0, :]
    assert np.allclose(out[0], [0, 0, 1, 0], atol=1e-15)             # e0 -> e2
    assert np.allclose(out[2], [-1, 0, 0, 0], atol=1e-15)            # e2 -> -e0
    a = np.pi / 2 * 0.1                                              # pair (1, 3) at theta_1 = 0.1
    assert np.allclose(out[1], [0, np.cos(a), 0, np.sin(a)], atol=1e-15)


def _complex_rope(x, positions, base):
    D = x.shape[-1]
    h = D // 2
    z = x[..., :h] + 1j * x[..., h:]
    th = np.exp(-np.log(base) * 2.0 * np.arange(h) / D)
    z = z * np.exp(1j * np.outer(positions, th))[:, None, :]
    return np.concatenate([z.real, z.imag], axis=-1)


def test_matches_complex_multiplication():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 3, 128))
    pos = rng.integers(0, 3_400_000, 50)
    assert np.allclose(L.rope(x, pos, 500000.0), _complex_rope(x, pos, 500000.0), atol=1e-9)


def test_invariants_identity_norm_relative_position():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 2, 64))
    k = rng.standard_normal((1, 2, 64))
    assert np.array_equal(L.rope(q, [0], 10000.0), q)
    r = L.rope(q, [12345], 10000.0)
    assert np.allclose(r[..., :32] ** 2 + r[..., 32:] ** 2, q[..., :32] ** 2 + q[..., 32:] ** 2)
    for m, n in ((7, 3), (1000, 999), (40000, 17)):
        s_mn = np.sum(L.rope(q, [m], 10000.0) * L.rope(k, [n], 10000.0), axis=-1)
        s_rel = np.sum(L.rope(q, [m - n], 10000.0) * k, axis=-1)
        assert np.allclose(s_mn, s_rel, atol=1e-9)


def _identity_qkv(Hq, Hkv, D):
    n = (Hq + 2 * Hkv) * D
    return np.eye(n, dtype=np.int8) * 127, np.full(n, 1.0 / 127, dtype=np.float64)


def test_qkv_sections_and_which_heads_rotate():
    Hq, Hkv, D = 4, 2, 8
    codes, scales = _identity_qkv(Hq, Hkv, D)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((6, (Hq + 2 * Hkv) * D))
    pos = np.array([0, 1, 5, 100, 7, 9])
    q, k, v = L.qkv_rope(x, codes, scales, Hq, Hkv, D, pos, 10000.0)
    xq = x[:, :Hq * D].reshape(6, Hq, D)
    xk = x[:, Hq * D:(Hq + Hkv) * D].reshape(6, Hkv, D)
    xv = x[:, (Hq + Hkv) * D:].reshape(6, Hkv, D)
    assert np.allclose(q, _complex_rope(xq, pos, 10000.0), atol=1e-13)
    assert np.allclose(k, _complex_rope(xk, pos, 10000.0), atol=1e-13)
    assert np.allclose(v, xv, atol=1e-14)


def test_weight_generator_codes_and_scales():
    c = I.weight_codes(7, 1, "o", 3, 5, 300)
    assert c.dtype == np.int8 and c.shape == (5, 300) and np.abs(c.astype(int)).max() <= 111
    assert np.array_equal(c, I.weight_codes(7, 1, "o", 0, 8, 300)[3:])
    x32 = I.values_f32(7, I.weight_stream(1, "o"), np.arange(3 * 300, 4 * 300, dtype=np.uint64))
    assert np.array_equal(c[0], np.rint(x32.astype(np.float64) * 32).astype(np.int8))
    s = I.weight_scales(7, 1, "o", 64, 4096)
    assert s.dtype == np.float32 and np.all(s > 0.1 / (32 * 64)) and np.all(s < 2.0 / (32 * 64))


# ---- planted mistakes: each variant must fail one of the pins above ------------------

def _interleaved(x, positions, base):
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    a = np.asarray(positions, dtype=np.float64)[:, None] * L.rope_frequencies(D, base)[None, :]
    c, s = np.cos(a)[:, None, :], np.sin(a)[:, None, :]
    ev, od = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = ev * c - od * s
    out[..., 1::2] = od * c + ev * s
    return out


def _reversed(x, positions, base):
    return L.rope(x, -np.asarray(positions, dtype=np.float64), base)


@pytest.mark.parametrize("variant", [_interleaved, _reversed])
def test_planted_rotation_mistakes_fail_the_pins(variant):
    e = np.eye(4)[:, None, :]
    bad_quarter = not np.allclose(variant(e, np.full(4, np.pi / 2), 100.0)[0, 0], [0, 0, 1, 0], atol=1e-12)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 1, 16))
    pos = rng.integers(0, 1000, 5)
    bad_complex = not np.allclose(variant(x, pos, 10000.0), _complex_rope(x, pos, 10000.0), atol=1e-9)
    assert bad_quarter and bad_complex


def test_planted_section_mistakes_fail_the_pins():
    Hq, Hkv, D = 2, 1, 4
    codes, scales = _identity_qkv(Hq, Hkv, D)
    x = np.random.default_rng(4).standard_normal((3, 16))
    pos = np.array([1, 2, 3])
    y = L.w8_linear(x, codes, scales)
    # keys left unrotated, and K / V sections swapped
    k_plain = y[:, Hq * D:(Hq + Hkv) * D].reshape(3, Hkv, D)
    v_as_k = L.rope(y[:, (Hq + Hkv) * D:].reshape(3, Hkv, D), pos, 10000.0)
    xk = x[:, Hq * D:(Hq + Hkv) * D].reshape(3, Hkv, D)
    ref = _complex_rope(xk, pos, 10000.0)
    assert not np.allclose(k_plain, ref, atol=1e-6)
    assert not np.allclose(v_as_k, ref, atol=1e-6)
