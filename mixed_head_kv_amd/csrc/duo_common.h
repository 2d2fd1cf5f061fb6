// Internal definitions shared by the host library and the HIP kernels of
// libduo_attn.so: workspace geometry, cache addressing, element conversions.
//
// Cache layout in HBM (per layer, per sequence b, per KV head of one kind):
//   retrieval K : rows of D values, row = absolute position.  bf16 with D = 128 stores
//                 them in 32-key tiles (8 KB) whose 16-byte chunks are ordered for the
//                 MFMA K operand (k_tiled): chunk c = dims 8c..8c+7 of key kk of the tile
//                 sits at chunk ((t*4 + c%4)*4 + c/4)*16 + r with t = (kk>>2)&1 and
//                 r = 4*(kk>>3) + (kk&3), so each 1 KB of the tile is exactly what one
//                 load instruction of a wavefront needs.  Other shapes are row-major.
//   retrieval V : 8-row tiles stored d-major, [cap/8][D][8]; element (row, d) sits at
//                 ((row & ~7) * D + d * 8 + (row & 7)).  Eight consecutive keys of one
//                 dimension are contiguous, which is the operand order the MFMA
//                 products P*V read (the key index is the contraction index there).
//   streaming K/V: the same two layouts over `nslot` slots; slot s < sink holds sink
//                 position s, slot sink + ((p - sink) mod recent) holds recent position p.
//   int4 (group 128): K codes in 32-key tiles of 2 KB (byte b of key kk at
//                 (t*64 + (b/16)*16 + r)*16 + b%16, same t, r as above; byte b holds
//                 codes 2b | 2b+1 << 4),
//                 V codes in 8-row tiles [cap/8][D][8 nibbles = 4 bytes] (nibble r of the
//                 dword = row r of the tile), and per row a uint16 pair (scale, zero)
//                 of fp16 bit patterns, [cap][2] for K and for V.
// cap and nslot are multiples of 64 so whole 64-row tiles are always in bounds.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/duo_attn.h"
#include "../../include/duo_synth.h"

namespace duo {

constexpr int kMaxSplits = 2048;    // split-K partial slots per query head (decode; prefill reuses the buffer)
constexpr int kPrefillCounters = 1 << 16;  // arrival counters for split prefill query blocks
constexpr int kRowAlign = 64;       // cache rows are allocated in multiples of this
constexpr int kStageTokens = 4096;  // queries per streaming-head prefill launch (staging capacity)
constexpr int kKindRetrieval = 1;
constexpr int kKindStreaming = 0;

// Where one kind of cache of one layer lives.  `rows` = rows per cache (cap or nslot).
struct CacheRegion {
  char* k;          // K values or int4 codes
  char* v;          // V values or int4 codes
  uint16_t* k_meta; // int4: (scale, zero) per row; else null
  uint16_t* v_meta;
  int64_t rows;
  int k_tiled;      // K rows in MFMA-ordered 32-key tiles (bf16, D = 128)
};

// Everything a kernel needs to know about one layer of one handle.
struct LayerView {
  CacheRegion ret;
  CacheRegion str;
  int n_ret;                             // retrieval KV heads per sequence
  int n_str;                             // streaming KV heads per sequence
  int kind[DUO_MAX_KV_HEADS];            // per KV head: kKindRetrieval / kKindStreaming
  int slot[DUO_MAX_KV_HEADS];            // per KV head: index among heads of its kind
  int ret_kv[DUO_MAX_KV_HEADS];          // retrieval index -> KV head
  int str_kv[DUO_MAX_KV_HEADS];          // streaming index -> KV head
};

struct Geom {
  int B, Hq, Hkv, G, D, S, R;
  int io;          // DUO_DTYPE_*
  int kvfmt;       // DUO_KV_*
  float scale;     // softmax scale
  float scale_log2;// scale * log2(e): scores are kept in the base-2 domain
};

// ---- element conversions -------------------------------------------------------

__host__ __device__ inline float bf16_to_f32(uint16_t b) {
  union { uint32_t u; float f; } x;
  x.u = static_cast<uint32_t>(b) << 16;
  return x.f;
}

__host__ __device__ inline uint16_t f32_to_bf16(float f) {
  union { uint32_t u; float f; } x;
  x.f = f;
  if ((x.u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;  // NaN stays NaN
  return static_cast<uint16_t>((x.u + 0x7fffu + ((x.u >> 16) & 1u)) >> 16);
}

template <int IO> struct IoType;
template <> struct IoType<DUO_DTYPE_F32> { using T = float; };
template <> struct IoType<DUO_DTYPE_BF16> { using T = uint16_t; };
template <> struct IoType<DUO_SYNTH_INT8> { using T = int8_t; };

template <int IO>
__device__ inline float io_load(const void* p, int64_t i) {
  if constexpr (IO == DUO_DTYPE_F32) return static_cast<const float*>(p)[i];
  else return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}

template <int IO>
__device__ inline void io_store(void* p, int64_t i, float v) {
  if constexpr (IO == DUO_DTYPE_F32) static_cast<float*>(p)[i] = v;
  else static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
}

// ---- cache addressing ----------------------------------------------------------

// Element offset of 16-byte chunk c (dims 8c..8c+7) of global K row `grow` in an
// MFMA-ordered 32-key tile (bf16, D = 128).
__host__ __device__ inline int64_t k_chunk_tiled(int64_t grow, int c) {
  const int kk = static_cast<int>(grow & 31);
  const int t = (kk >> 2) & 1;
  const int r = ((kk >> 3) << 2) | (kk & 3);
  return (grow >> 5) * 4096 + static_cast<int64_t>(((t * 4 + (c & 3)) * 4 + (c >> 2)) * 16 + r) * 8;
}

// Byte offset of code byte b (0..63) of global int4 K row `grow` (32-key tiles of 2 KB).
__host__ __device__ inline int64_t k_code_byte(int64_t grow, int b) {
  const int kk = static_cast<int>(grow & 31);
  const int t = (kk >> 2) & 1;
  const int r = ((kk >> 3) << 2) | (kk & 3);
  return (grow >> 5) * 2048 + static_cast<int64_t>((t * 64 + (b >> 4) * 16 + r) * 16 + (b & 15));
}

__device__ inline int64_t k_index(const CacheRegion& c, int64_t cache, int64_t row, int D, int d) {
  const int64_t grow = cache * c.rows + row;
  return c.k_tiled ? k_chunk_tiled(grow, d >> 3) + (d & 7) : grow * D + d;
}
__device__ inline int64_t v_index(int64_t cache, int64_t rows, int64_t row, int D, int d) {
  return (cache * rows + (row & ~int64_t(7))) * D + int64_t(d) * 8 + (row & 7);
}

// Dequantised int4 element: fp32(q * s + z); q * s is exact, so this is one rounding.
__device__ inline float int4_value(uint32_t q, uint16_t s_bits, uint16_t z_bits) {
  float s = __half2float(__ushort_as_half(s_bits));
  float z = __half2float(__ushort_as_half(z_bits));
  return fmaf(static_cast<float>(q), s, z);
}

// Stored K element (cache row `row`, dimension d) of one cache, as fp32.
template <int IO, int KVF>
__device__ inline float cache_k(const CacheRegion& c, int64_t cache, int64_t row, int D, int d) {
  if constexpr (KVF == DUO_KV_INT4_G128) {
    const uint32_t byte = reinterpret_cast<const uint8_t*>(c.k)[k_code_byte(cache * c.rows + row, d >> 1)];
    uint32_t q = (d & 1) ? (byte >> 4) : (byte & 15u);
    const uint16_t* m = c.k_meta + (cache * c.rows + row) * 2;
    return int4_value(q, m[0], m[1]);
  } else {
    return io_load<IO>(c.k, k_index(c, cache, row, D, d));
  }
}

template <int IO, int KVF>
__device__ inline float cache_v(const CacheRegion& c, int64_t cache, int64_t row, int D, int d) {
  if constexpr (KVF == DUO_KV_INT4_G128) {
    const uint32_t* words = reinterpret_cast<const uint32_t*>(c.v) + (cache * c.rows + (row & ~int64_t(7))) / 8 * D;
    uint32_t q = (words[d] >> (4 * (row & 7))) & 15u;
    const uint16_t* m = c.v_meta + (cache * c.rows + row) * 2;
    return int4_value(q, m[0], m[1]);
  } else {
    return io_load<IO>(c.v, v_index(cache, c.rows, row, D, d));
  }
}

// Source token of destination row `row` for a bf16 append, with the ring position
// precomputed on the host: ring_lo = max(t0, S, t0 + T - R) is the first chunk
// position that survives in the ring, ring_have = (ring_lo - S) mod R its ring index.
__host__ __device__ inline int source_token_fast(bool streaming, int64_t row, int64_t t0, int T, int S, int R,
                                        int64_t ring_lo, int ring_have) {
  if (!streaming || row < S) {
    if (streaming && row >= S + R) return -1;
    const int64_t t = row - t0;
    return (t >= 0 && t < T) ? static_cast<int>(t) : -1;
  }
  if (row >= S + R || ring_lo >= t0 + T) return -1;
  int d = static_cast<int>(row - S) - ring_have;
  if (d < 0) d += R;
  const int64_t p = ring_lo + d;
  return p < t0 + T ? static_cast<int>(p - t0) : -1;
}

// Streaming-head prefill staging (one region per streaming cache, shared by the layers):
// sink rows [0, Sp), then window rows covering the W positions before a launch's first
// query (W >= R - 1, so every window key of its queries is there) and its queries.
__host__ __device__ inline int stage_sink_rows(int S) { return (S + kRowAlign - 1) / kRowAlign * kRowAlign; }
__host__ __device__ inline int stage_window_rows(int R) { return (R - 1 + kRowAlign - 1) / kRowAlign * kRowAlign; }

__device__ inline float wave_min(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fminf(x, __shfl_xor(x, o));
  return x;
}
__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// int4 group-128 quantisation of one vector held two values per lane (d = 2*lane,
// 2*lane + 1).  Steps and rounding are those of the format: fp32 range, fp32 divide
// by 15, fp16 round of scale and zero, fp32 (x - z) / s, round half to even, clamp.
struct Q4 {
  uint32_t q0, q1;
  uint16_t s_bits, z_bits;
};
__device__ inline Q4 quantize_pair(float x0, float x1) {
  const float mn = wave_min(fminf(x0, x1));
  const float mx = wave_max(fmaxf(x0, x1));
  const float s32 = __fdiv_rn(__fsub_rn(mx, mn), 15.0f);
  const __half sh = __float2half_rn(s32);
  const __half zh = __float2half_rn(mn);
  const float s = __half2float(sh);
  const float z = __half2float(zh);
  Q4 r;
  r.s_bits = __half_as_ushort(sh);
  r.z_bits = __half_as_ushort(zh);
  if (s == 0.0f) {
    r.q0 = r.q1 = 0;
  } else {
    const float a = fminf(fmaxf(rintf(__fdiv_rn(__fsub_rn(x0, z), s)), 0.0f), 15.0f);
    const float c = fminf(fmaxf(rintf(__fdiv_rn(__fsub_rn(x1, z), s)), 0.0f), 15.0f);
    r.q0 = static_cast<uint32_t>(a);
    r.q1 = static_cast<uint32_t>(c);
  }
  return r;
}

// Streaming slot of an absolute position that the constant-length cache holds.
__host__ __device__ inline int64_t stream_slot(int64_t p, int S, int R) {
  return p < S ? p : S + (p - S) % R;
}

}  // namespace duo
