"""Seeded synthetic inputs and the workload shapes, shared by the tests, the bench and
the oracle checks.

This module holds no attention arithmetic and imports neither the HIP binding nor the
oracle.  It defines:

* the five workload shapes (head counts, head size, dtypes, sink / recent sizes,
  context lengths, chunking);
* the per-layer retrieval masks (a seeded choice of KV heads);
* a counter-based generator for Q, K and V, so that any slice of a multi-gigabyte
  input can be produced independently on the host (this module, NumPy, or its C twin
  inputs_host.c when built) or on the device (a HIP fill kernel implementing the same
  published definition), bit for bit.

Generator definition (SplitMix64, Steele, Lea and Flood, "Fast Splittable
Pseudorandom Number Generators", OOPSLA 2014): with GAMMA = 0x9E3779B97F4A7C15 and the
SplitMix64 finaliser mix64(z) = z3 where
    z1 = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9,
    z2 = (z1 ^ (z1 >> 27)) * 0x94D049BB133111EB,
    z3 = z2 ^ (z2 >> 31)            (all mod 2^64),
the stream key is key = mix64((seed << 32) | stream) and the n-th word of the stream is
w(n) = mix64(key + (n + 1) * GAMMA).  A value is the sum S of the four 16-bit fields of
w(n) (Irwin-Hall with four uniforms), centred and scaled to unit variance:
    x = fp32(S - 131070) * fp32(sqrt(3) / 65536)       (one fp32 multiply, RN),
then rounded to nearest even into the I/O dtype.  Every step is exact integer work or a
single correctly rounded fp32 operation, so host and device agree bit for bit.  x has
mean 0, variance 1 (to 1 part in 2^32) and support [-3.47, 3.47]: a stand-in for the
workloads' N(0, 1) that costs the attention path exactly the same work.

Streams: stream = layer * 4 + {Q: 0, K: 1, V: 2, X: 3} (X: a layer's hidden-state input,
[T, hidden], counter n = pos * hidden + e).  Counters index the whole sequence by
absolute position: Q at (pos, head, d) uses n = (pos * Hq + head) * D + d and K/V at
(pos, kv_head, d) use n = (pos * Hkv + kv_head) * D + d, so a prefill chunk
[pos0, pos0 + T) is the contiguous counter range starting at pos0 * H * D and decode
step t uses position t.
"""

from __future__ import annotations

import dataclasses
import math
import os

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
SCALE_F32 = np.float32(math.sqrt(3.0) / 65536.0)
CENTER = 131070
KIND_STREAM = {"q": 0, "k": 1, "v": 2, "x": 3}
# Synthetic 8-bit weights of the linear layers around the attention: codes of weight
# `which` of `layer` use stream WEIGHT_BASE + layer * 8 + WEIGHT_STREAM[which] with
# counter n * K + k for (output channel n, input k); the per-channel scales use that
# stream + 4 with counter n.
WEIGHT_BASE = 1 << 16
WEIGHT_STREAM = {"qkv": 0, "o": 1}
CODE_MULT = np.float32(32.0)

_CHUNK = 1 << 22  # counters per NumPy pass (bounds host memory)

# The same generator in C (inputs_host.c, OpenMP), used when built: identical values,
# far faster for the multi-gigabyte histories of the long-context workloads.
_HOST_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libduo_inputs.so")
_host = None


def _host_lib():
    global _host
    if _host is None:
        _host = False
        if os.path.exists(_HOST_LIB):
            import ctypes
            L = ctypes.CDLL(_HOST_LIB)
            vp = ctypes.c_void_p
            L.duo_inputs_head_rows.argtypes = [ctypes.c_uint64, ctypes.c_uint32, vp, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_int64, ctypes.c_int64, ctypes.c_float, vp, vp]
            L.duo_inputs_range.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int64,
                                           ctypes.c_float, vp, vp]
            _host = L
    return _host or None


def _mix64(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, stream: int) -> np.uint64:
    return _mix64(np.array([(int(seed) << 32) | (int(stream) & 0xFFFFFFFF)], dtype=np.uint64))[0]


def words(seed: int, stream: int, counters: np.ndarray) -> np.ndarray:
    key = stream_key(seed, stream)
    c = np.asarray(counters, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64(key + (c + np.uint64(1)) * GAMMA)


def _fill(seed: int, stream: int, flat_c: np.ndarray, flat_o: np.ndarray, a: int) -> None:
    m16 = np.uint64(0xFFFF)
    w = words(seed, stream, flat_c[a:a + _CHUNK])
    s = (w & m16) + ((w >> np.uint64(16)) & m16) + ((w >> np.uint64(32)) & m16) + (w >> np.uint64(48))
    flat_o[a:a + _CHUNK] = (s.astype(np.int64) - CENTER).astype(np.float32) * SCALE_F32


def values_f32(seed: int, stream: int, counters: np.ndarray) -> np.ndarray:
    """fp32 values for the given counters (any shape).  Large requests are split over
    threads (NumPy releases the GIL inside these array operations)."""
    counters = np.asarray(counters, dtype=np.uint64)
    out = np.empty(counters.shape, dtype=np.float32)
    flat_c = counters.reshape(-1)
    flat_o = out.reshape(-1)
    starts = range(0, flat_c.size, _CHUNK)
    if flat_c.size <= 2 * _CHUNK:
        for a in starts:
            _fill(seed, stream, flat_c, flat_o, a)
        return out
    import concurrent.futures as cf
    workers = max(1, min(16, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda a: _fill(seed, stream, flat_c, flat_o, a), starts))
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, nearest even; returns the uint16 bit patterns.
    (Finite inputs only, which is all the generator produces.)"""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _cast(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def synth(seed: int, layer: int, kind: str, pos0: int, T: int, H: int, D: int, dtype: str,
          use_host_lib: bool = True) -> np.ndarray:
    """Tensor [T, H, D] for positions [pos0, pos0 + T) of one layer.

    dtype "f32" -> float32; "bf16" -> uint16 bf16 bit patterns."""
    stream = layer * 4 + KIND_STREAM[kind]
    L = _host_lib() if use_host_lib else None
    if L is not None and dtype in ("f32", "bf16"):
        out = np.empty((T, H, D), dtype=np.float32 if dtype == "f32" else np.uint16)
        ptr = out.ctypes.data
        L.duo_inputs_range(seed, stream, pos0 * H * D, T * H * D, float(SCALE_F32),
                           ptr if dtype == "f32" else None, ptr if dtype == "bf16" else None)
        return out
    c0 = np.uint64(pos0) * np.uint64(H * D)
    counters = c0 + np.arange(T * H * D, dtype=np.uint64)
    return _cast(values_f32(seed, stream, counters), dtype).reshape(T, H, D)


def synth_head(seed: int, layer: int, kind: str, positions, head: int, H: int, D: int, dtype: str,
               use_host_lib: bool = True) -> np.ndarray:
    """Rows [n, D] of one head at the given absolute positions (strided counters)."""
    stream = layer * 4 + KIND_STREAM[kind]
    L = _host_lib() if use_host_lib else None
    if L is not None and dtype in ("f32", "bf16"):
        pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int64).reshape(-1))
        out = np.empty((len(pos), D), dtype=np.float32 if dtype == "f32" else np.uint16)
        ptr = out.ctypes.data
        L.duo_inputs_head_rows(seed, stream, pos.ctypes.data, len(pos), head, H, D, float(SCALE_F32),
                               ptr if dtype == "f32" else None, ptr if dtype == "bf16" else None)
        return out
    pos = np.asarray(positions, dtype=np.uint64).reshape(-1)
    counters = (pos[:, None] * np.uint64(H) + np.uint64(head)) * np.uint64(D) + np.arange(D, dtype=np.uint64)[None, :]
    return _cast(values_f32(seed, stream, counters), dtype)


def retrieval_mask(seed: int, layer: int, n_kv: int, n_retrieval: int, fixed=None) -> np.ndarray:
    """Per-KV-head labels of one layer, True = retrieval.  A fixed list wins; otherwise
    ``numpy.random.default_rng(seed + layer).choice(n_kv, n_retrieval, replace=False)``."""
    m = np.zeros(n_kv, dtype=bool)
    if fixed is not None:
        m[list(fixed)] = True
        return m
    rng = np.random.default_rng(seed + layer)
    m[np.sort(rng.choice(n_kv, n_retrieval, replace=False))] = True
    return m


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    io_dtype: str            # "f32" | "bf16"
    kv_format: str           # "same" | "int4"
    sink: int
    recent: int
    context: int             # tokens before decode starts
    prefill_chunk: int       # 0 = caches are bulk-filled with kv_append instead of prefill
    decode_steps: int
    n_retrieval: int
    fixed_retrieval: tuple | None = None

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def max_context(self) -> int:
        return self.context + self.decode_steps

    def mask(self, layer: int) -> np.ndarray:
        return retrieval_mask(self.seed, layer if self.n_layers > 1 else 0, self.n_kv_heads,
                              self.n_retrieval, self.fixed_retrieval)

    def masks(self) -> np.ndarray:
        return np.stack([self.mask(l) for l in range(self.n_layers)])

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny_mha_f32_512": Workload("tiny_mha_f32_512", 1, 1, 4, 4, 64, "f32", "same", 4, 64,
                                 512, 512, 16, 2, fixed_retrieval=(0, 2)),
    "llama2_7b_mha_32k": Workload("llama2_7b_mha_32k", 2, 1, 32, 32, 128, "bf16", "same", 64, 256,
                                  32768, 4096, 128, 8),
    "llama3_8b_gqa_128k": Workload("llama3_8b_gqa_128k", 3, 1, 32, 8, 128, "bf16", "same", 64, 256,
                                   131072, 8192, 256, 4),
    "llama3_8b_gqa_32layer_1m": Workload("llama3_8b_gqa_32layer_1m", 4, 32, 32, 8, 128, "bf16", "same",
                                         64, 256, 1048576, 0, 36, 4),
    "llama3_8b_gqa_32layer_int4_3p3m": Workload("llama3_8b_gqa_32layer_int4_3p3m", 5, 32, 32, 8, 128,
                                                "bf16", "int4", 64, 256, 3300000, 0, 36, 4),
}
WORKLOAD_ORDER = list(WORKLOADS)


def weight_stream(layer: int, which: str) -> int:
    return WEIGHT_BASE + layer * 8 + WEIGHT_STREAM[which]


def weight_codes(seed: int, layer: int, which: str, n0: int, n: int, K: int) -> np.ndarray:
    """int8 codes [n, K] of output channels [n0, n0 + n): the generator's fp32 value times
    32 (exact), rounded to nearest even (|code| <= 111).  The device fill
    (duo_synth_fill with DUO_SYNTH_INT8) computes the same."""
    counters = np.uint64(n0) * np.uint64(K) + np.arange(n * K, dtype=np.uint64)
    x = values_f32(seed, weight_stream(layer, which), counters) * CODE_MULT
    return np.rint(x).astype(np.int8).reshape(n, K)


def weight_codes_rows(seed: int, layer: int, which: str, rows, K: int) -> np.ndarray:
    """Codes [len(rows), K] of the given output channels (for sampled checks)."""
    rows = np.asarray(rows, dtype=np.uint64).reshape(-1)
    counters = rows[:, None] * np.uint64(K) + np.arange(K, dtype=np.uint64)[None, :]
    x = values_f32(seed, weight_stream(layer, which), counters) * CODE_MULT
    return np.rint(x).astype(np.int8)


def weight_scales(seed: int, layer: int, which: str, N: int, K: int) -> np.ndarray:
    """fp32 scales [N]: (1 + x / 4) / (32 sqrt(K)) rounded once to fp32, x from the
    generator, so that a layer fed unit-variance inputs gives outputs of standard
    deviation 1 + x / 4 (between 0.13 and 1.87)."""
    x = values_f32(seed, weight_stream(layer, which) + 4, np.arange(N, dtype=np.uint64)).astype(np.float64)
    return ((1.0 + 0.25 * x) / (32.0 * math.sqrt(K))).astype(np.float32)
