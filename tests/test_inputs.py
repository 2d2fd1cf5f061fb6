"""The seeded input generator (CPU): published SplitMix64 test vector, determinism,
slice consistency and the moments of the value distribution."""

import numpy as np

from mixed_head_kv_amd import inputs as I


def test_splitmix64_known_answer():
    # First five outputs of SplitMix64 from state 1234567 (the reference test vector
    # published with the generator's C implementation).
    st = np.uint64(1234567)
    with np.errstate(over="ignore"):
        got = [int(I._mix64(st + np.uint64(n + 1) * I.GAMMA)) for n in range(5)]
    assert got == [6457827717110365317, 3203168211198807973, 9817491932198370423,
                   4593380528125082431, 16408922859458223821]


def test_chunk_and_head_slices_agree():
    full = I.synth(7, 0, "k", 0, 50, 3, 16, "bf16")
    part = I.synth(7, 0, "k", 20, 10, 3, 16, "bf16")
    assert np.array_equal(full[20:30], part)
    head = I.synth_head(7, 0, "k", [3, 20, 49], 2, 3, 16, "bf16")
    assert np.array_equal(head, full[[3, 20, 49], 2])


def test_moments_and_support():
    x = I.values_f32(3, 2, np.arange(1 << 20, dtype=np.uint64))
    assert abs(float(x.mean())) < 5e-3
    assert abs(float(x.var()) - 1.0) < 5e-3
    assert np.abs(x).max() <= np.float32(131070) * I.SCALE_F32


def test_streams_differ():
    a = I.synth(1, 0, "q", 0, 4, 2, 8, "f32")
    b = I.synth(1, 0, "k", 0, 4, 2, 8, "f32")
    c = I.synth(1, 1, "q", 0, 4, 2, 8, "f32")
    assert not np.array_equal(a, b) and not np.array_equal(a, c)


def test_bf16_rounding_nearest_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20], np.float32)
    assert I.f32_to_bf16_bits(x).tolist() == [0x3F80, 0x3F82, 0xC020, 0x3F81]


def test_masks():
    w = I.WORKLOADS["llama2_7b_mha_32k"]
    m = w.mask(0)
    assert m.sum() == 8 and m.shape == (32,)
    t = I.WORKLOADS["tiny_mha_f32_512"]
    assert t.mask(0).tolist() == [True, False, True, False]
    s = I.WORKLOADS["llama3_8b_gqa_32layer_1m"].masks()
    assert s.shape == (32, 8) and (s.sum(axis=1) == 4).all()


def test_host_c_twin_matches_numpy_definition():
    """The C twin of the generator (libduo_inputs.so) gives the NumPy definition's
    values bit for bit: contiguous ranges and strided head rows, fp32 and bf16."""
    if I._host_lib() is None:
        import pytest
        pytest.skip("libduo_inputs.so not built")
    rng = np.random.default_rng(5)
    for dtype in ("f32", "bf16"):
        for seed, layer, kind, pos0, T, H, D in [(3, 0, "k", 0, 37, 8, 128), (5, 31, "v", 3_299_990, 9, 8, 128),
                                                 (1, 2, "q", 123, 5, 32, 64)]:
            a = I.synth(seed, layer, kind, pos0, T, H, D, dtype)
            b = I.synth(seed, layer, kind, pos0, T, H, D, dtype, use_host_lib=False)
            assert a.dtype == b.dtype and np.array_equal(a, b)
        pos = rng.integers(0, 3_300_000, 300)
        a = I.synth_head(4, 17, "k", pos, 5, 8, 128, dtype)
        b = I.synth_head(4, 17, "k", pos, 5, 8, 128, dtype, use_host_lib=False)
        assert a.dtype == b.dtype and np.array_equal(a, b)
