"""The algorithmic work bench.py divides by (CPU only): flops of a pre-filling chunk and
bytes of a decode launch, checked by counting visible (query, key) pairs and cached
vectors with the oracle's visibility rule, and the extras' grid arithmetic against the
launch shapes of the library's kernels."""

import os
import sys

import numpy as np
import pytest

from mixed_head_kv_amd import inputs as I
from oracle.attention import visible

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def W(hq, hkv, S, R, nr, fmt="same", io="bf16"):
    return I.Workload("w", 3, 1, hq, hkv, 128, io, fmt, S, R, 100, 0, 1, nr, None)


@pytest.mark.parametrize("retrieval", [True, False])
@pytest.mark.parametrize("t0,T", [(0, 37), (50, 70), (5, 1)])
def test_prefill_flops_count_visible_pairs(retrieval, t0, T):
    w = W(8, 4, 4, 9, 2)
    mask = w.mask(0)
    i = np.arange(t0, t0 + T)[:, None]
    j = np.arange(t0 + T)[None, :]
    pairs = 0
    for g in range(w.n_kv_heads):
        if bool(mask[g]) == retrieval:
            pairs += int(visible(i, j, bool(mask[g]), w.sink, w.recent).sum()) * w.group
    assert bench.prefill_flops(w, t0, T, retrieval) == 4 * w.head_dim * pairs


@pytest.mark.parametrize("fmt,io", [("same", "bf16"), ("same", "f32"), ("int4", "bf16")])
@pytest.mark.parametrize("t", [0, 3, 12, 40])
def test_decode_bytes_count_cached_vectors(fmt, io, t):
    w = W(8, 4, 4, 9, 2, fmt, io)
    mask = w.mask(0)
    vec = 68 if fmt == "int4" else 128 * (4 if io == "f32" else 2)
    vectors = 0
    for g in range(w.n_kv_heads):  # once per KV head: the G query heads share its keys
        vectors += int(visible(t, np.arange(t + 1), bool(mask[g]), w.sink, w.recent).sum())
    qo = 2 * w.n_q_heads * 128 * (4 if io == "f32" else 2)
    assert bench.decode_bytes(w, t) == 2 * vec * vectors + qo


def test_extras_grids_match_the_launch_shapes():
    k = bench.extra_kernels("llama2_7b_mha_32k")
    assert k["qkv_rope_decode"] == ("k_w8_gemv<1>", 12288 // 16 * 512)
    assert k["out_proj_decode"] == ("k_w8_gemv<1>", 4096 // 16 * 512)
    assert k["qkv_rope_prefill"] == ("k_w8_gemm<", 16 * 48 * 512)
    assert k["out_proj_prefill"] == ("k_w8_gemm<", 16 * 16 * 512)
    k3 = bench.extra_kernels("llama3_8b_gqa_32layer_1m")
    assert k3["qkv_rope_decode"][1] == 6144 // 16 * 512 and "qkv_rope_prefill" not in k3


def test_launch_kinds_follow_the_prefill_grid_rules():
    """The prefill launches are told apart by grid in the profile summaries: the chunk's
    streaming-only launches use 4-wavefront workgroups of 128 / pack queries x pack heads
    (pack = 4 for the 128K GQA layer: 4 head groups x 128 blocks x 256 threads), every
    other k_prefill_mfma launch is the chunk's main launch; a 4096-token chunk (32K MHA
    layer) has no streaming-only launch."""
    assert bench.streaming_only_grid("llama3_8b_gqa_128k") == 4 * (4096 // 32) * 256
    assert bench.streaming_only_grid("llama2_7b_mha_32k") is None
    name = "duo::(anonymous namespace)::k_prefill_mfma<4>(duo::(anonymous namespace)::PrefillArgs)"
    assert bench.launch_kind(name, 131072, "llama3_8b_gqa_128k") == "prefill_streaming_attention"
    main = name.replace("<4>", "<8>")
    assert bench.launch_kind(main, (512 + 256) * 512, "llama3_8b_gqa_128k") == "prefill_attention"
    assert bench.launch_kind("duo::k_decode_mfma(args)", 1, "llama3_8b_gqa_128k") == "decode_attention"
    assert bench.launch_kind("duo::k_synth<1>(args)", 1, "llama3_8b_gqa_128k") is None


def test_traffic_digest_covers_source_and_build_flags(monkeypatch):
    """Stored HBM traffic counts for a kernel only while both its source file and the hipcc
    flags that file builds with are unchanged."""
    from mixed_head_kv_amd import build
    before = bench.source_digest("prefill_attention")
    assert before == bench.source_digest("prefill_attention")
    assert "-fno-honor-nans" in build.flags_for("prefill_mfma.hip")
    assert "-fno-honor-nans" not in build.flags_for("decode_mfma.hip")
    monkeypatch.setitem(build.FILE_FLAGS, "prefill_mfma.hip", [])
    assert bench.source_digest("prefill_attention") != before
    monkeypatch.undo()
    assert bench.source_digest("prefill_attention") == before
