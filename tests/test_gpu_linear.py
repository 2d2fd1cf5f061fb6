"""GPU parity of the 8-bit-weight linear layers (output projection; fused QKV projection
with the rotary encoding) against the fp64 oracle on the same seeded inputs.

Bar: |got - ref| <= 2^-8 |ref| + 2^-12 per element.  The output is rounded once to
bfloat16 (relative error <= 2^-9); the fp32 accumulation of K products and the
rotation's fp32 sine and cosine add errors orders of magnitude below that for these
unit-scale outputs; the absolute floor covers outputs near zero.
"""

import numpy as np
import pytest

from mixed_head_kv_amd import inputs as I
from oracle import linear as OL
from oracle.attention import upcast

from parity_util import say

pytestmark = pytest.mark.gpu
SEED = 5


def bar(name, got, ref):
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), name
    excess = np.abs(got - ref) - (2.0 ** -8 * np.abs(ref) + 2.0 ** -12)
    worst = float(np.max(np.abs(got - ref) / (np.abs(ref) + 2.0 ** -4)))
    say(f"  {name}: worst relative error {worst:.2e} over {got.size} values")
    assert excess.max() <= 0, f"{name}: {int((excess > 0).sum())} values outside the bar"


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def device_x(torch, M, K, layer=0, pos0=0):
    from mixed_head_kv_amd import binding as B
    t = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    B.duo_synth_fill(t, B.DUO_DTYPE_BF16, SEED, layer * 4 + I.KIND_STREAM["x"], pos0 * K, M * K)
    return t


def host_x(M, K, layer=0, pos0=0):
    return upcast(I.synth(SEED, layer, "x", pos0, M, 1, K, "bf16").reshape(M, K), "bf16")


def device_weights(torch, which, N, K, layer=0):
    from mixed_head_kv_amd import binding as B
    w = torch.empty((N, K), dtype=torch.int8, device="cuda")
    B.duo_synth_fill(w, B.DUO_SYNTH_INT8, SEED, I.weight_stream(layer, which), 0, N * K)
    s = torch.from_numpy(I.weight_scales(SEED, layer, which, N, K)).cuda()
    return w, s


def to64(t):
    return t.float().cpu().numpy().astype(np.float64)


def test_device_int8_codes_match_host_generator(torch_cuda):
    w, _ = device_weights(torch_cuda, "qkv", 256, 384)
    assert np.array_equal(w.cpu().numpy(), I.weight_codes(SEED, 0, "qkv", 0, 256, 384))


# M: the decoding kernel's token blocks (1, 16 | 17, 32 | 33, 64) and the tiled kernel with
# ragged row tiles; N: one column tile (row-major tile order) and 8 (XCD bands).
@pytest.mark.parametrize("M", [1, 5, 16, 17, 33, 64, 65, 300, 513])
@pytest.mark.parametrize("K,N", [(128, 256), (384, 2048)])
def test_linear_w8_matches_oracle(torch_cuda, M, K, N):
    from mixed_head_kv_amd import binding as B
    say(f"linear_w8 M={M} K={K} N={N}")
    x = device_x(torch_cuda, M, K)
    w, s = device_weights(torch_cuda, "o", N, K)
    y = B.linear_w8(x, w, s)
    torch_cuda.cuda.synchronize()
    ref = OL.w8_linear(host_x(M, K), I.weight_codes(SEED, 0, "o", 0, N, K), I.weight_scales(SEED, 0, "o", N, K))
    bar(f"linear M={M} K={K} N={N}", to64(y), ref)


def _positions(M, rng, far):
    base = 3_300_000 if far else 0
    return np.sort(rng.integers(base, base + 50_000, M)).astype(np.int64)


@pytest.mark.parametrize("M", [1, 7, 64, 200])
@pytest.mark.parametrize("far", [False, True])
def test_qkv_rope_w8_matches_oracle(torch_cuda, M, far):
    """4 query heads, 2 KV heads of 128 dims, hidden 256; positions near 0 or past 3.3M
    (the angle reduction), with the Llama-3 base."""
    import torch
    from mixed_head_kv_amd import binding as B
    Hq, Hkv, D, hidden, base = 4, 2, 128, 256, 500000.0
    N = (Hq + 2 * Hkv) * D
    say(f"qkv_rope M={M} far={far}")
    pos = _positions(M, np.random.default_rng(M), far)
    x = device_x(torch, M, hidden)
    w, s = device_weights(torch, "qkv", N, hidden)
    q, k, v = B.qkv_rope_w8(x, torch.from_numpy(pos).cuda(), w, s, Hq, Hkv, D, base)
    torch.cuda.synchronize()
    rq, rk, rv = OL.qkv_rope(host_x(M, hidden), I.weight_codes(SEED, 0, "qkv", 0, N, hidden),
                             I.weight_scales(SEED, 0, "qkv", N, hidden), Hq, Hkv, D, pos, base)
    bar("q", to64(q), rq)
    bar("k", to64(k), rk)
    bar("v", to64(v), rv)


@pytest.mark.parametrize("model", ["llama2_7b", "llama3_8b"])
@pytest.mark.parametrize("M", [1, 16, 4096])
def test_full_size_qkv_and_output_projection(torch_cuda, model, M):
    """The shapes of the measured workloads: hidden 4096, 32 query heads, 32 (Llama-2-7B,
    base 10^4) or 8 (Llama-3-8B, base 5 * 10^5) KV heads; a decoding step (M = 1 or a batch
    of 16) and a 4096-token pre-filling chunk at positions 28672.. (the 32K workload's last
    chunk).  Every output channel of 64 sampled tokens (all tokens when M <= 64) is checked."""
    import torch
    from mixed_head_kv_amd import binding as B
    Hq, D, hidden = 32, 128, 4096
    Hkv, base = (32, 10000.0) if model == "llama2_7b" else (8, 500000.0)
    N = (Hq + 2 * Hkv) * D
    say(f"full-size {model} M={M}")
    pos = np.arange(28672, 28672 + M, dtype=np.int64)
    x = device_x(torch, M, hidden)
    w, s = device_weights(torch, "qkv", N, hidden)
    q, k, v = B.qkv_rope_w8(x, torch.from_numpy(pos).cuda(), w, s, Hq, Hkv, D, base)
    wo, so = device_weights(torch, "o", hidden, Hq * D)
    o_in = device_x(torch, M, Hq * D, layer=1)
    y = B.linear_w8(o_in, wo, so)
    torch.cuda.synchronize()
    rows = np.arange(M) if M <= 64 else np.unique(np.concatenate(
        [np.arange(8), np.arange(M - 8, M), np.random.default_rng(0).integers(0, M, 48)]))
    xs = host_x(M, hidden)[rows]
    rq, rk, rv = OL.qkv_rope(xs, I.weight_codes(SEED, 0, "qkv", 0, N, hidden),
                             I.weight_scales(SEED, 0, "qkv", N, hidden), Hq, Hkv, D, pos[rows], base)
    bar(f"{model} q", to64(q)[rows], rq)
    bar(f"{model} k", to64(k)[rows], rk)
    bar(f"{model} v", to64(v)[rows], rv)
    ry = OL.w8_linear(host_x(M, Hq * D, layer=1)[rows], I.weight_codes(SEED, 0, "o", 0, hidden, Hq * D),
                      I.weight_scales(SEED, 0, "o", hidden, Hq * D))
    bar(f"{model} o-proj", to64(y)[rows], ry)


def test_linear_outputs_are_bitwise_repeatable(torch_cuda):
    from mixed_head_kv_amd import binding as B
    x = device_x(torch_cuda, 300, 384)
    w, s = device_weights(torch_cuda, "o", 512, 384)
    a = B.linear_w8(x, w, s)
    b = B.linear_w8(x, w, s)
    x1 = x[:3].contiguous()
    c = B.linear_w8(x1, w, s)
    d = B.linear_w8(x1, w, s)
    torch_cuda.cuda.synchronize()
    assert torch_cuda.equal(a, b) and torch_cuda.equal(c, d)
