// Internal definitions shared by the host library and the HIP kernels of
// libduo_attn.so: workspace geometry, cache addressing, element conversions.
//
// Cache layout in HBM (per layer, per sequence b, per KV head of one kind):
//   retrieval K : row-major rows [cap][D]; row = absolute position.
//   retrieval V : 8-row tiles stored d-major, [cap/8][D][8]; element (row, d) sits at
//                 ((row & ~7) * D + d * 8 + (row & 7)).  Eight consecutive keys of one
//                 dimension are contiguous, which is the operand order the MFMA
//                 products P*V read (the key index is the contraction index there).
//   streaming K/V: the same two layouts over `nslot` slots; slot s < sink holds sink
//                 position s, slot sink + ((p - sink) mod recent) holds recent position p.
//   int4 (group 128): K codes row-major [cap][D/2] bytes (byte k = codes 2k | 2k+1 << 4),
//                 V codes in 8-row tiles [cap/8][D][8 nibbles = 4 bytes] (nibble r of the
//                 dword = row r of the tile), and per row a uint16 pair (scale, zero)
//                 of fp16 bit patterns, [cap][2] for K and for V.
// cap and nslot are multiples of 64 so whole 64-row tiles are always in bounds.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/duo_attn.h"

namespace duo {

constexpr int kMaxSplits = 2048;    // split-K partial slots per query head (decode; prefill reuses the buffer)
constexpr int kPrefillCounters = 1 << 16;  // arrival counters for split prefill query blocks
constexpr int kMergeScratchFloats = 4 * 16 * 129;  // LDS the MFMA decode merge may use
constexpr int kRowAlign = 64;       // cache rows are allocated in multiples of this
constexpr int kKindRetrieval = 1;
constexpr int kKindStreaming = 0;

// Where one kind of cache of one layer lives.  `rows` = rows per cache (cap or nslot).
struct CacheRegion {
  char* k;          // K values or int4 codes
  char* v;          // V values or int4 codes
  uint16_t* k_meta; // int4: (scale, zero) per row; else null
  uint16_t* v_meta;
  int64_t rows;
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

__device__ inline int64_t k_index(int64_t cache, int64_t rows, int64_t row, int D, int d) {
  return (cache * rows + row) * D + d;
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
    const uint8_t* codes = reinterpret_cast<const uint8_t*>(c.k) + (cache * c.rows + row) * (D / 2);
    uint32_t byte = codes[d >> 1];
    uint32_t q = (d & 1) ? (byte >> 4) : (byte & 15u);
    const uint16_t* m = c.k_meta + (cache * c.rows + row) * 2;
    return int4_value(q, m[0], m[1]);
  } else {
    return io_load<IO>(c.k, k_index(cache, c.rows, row, D, d));
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

// Streaming slot of an absolute position that the constant-length cache holds.
__host__ __device__ inline int64_t stream_slot(int64_t p, int S, int R) {
  return p < S ? p : S + (p - S) % R;
}

}  // namespace duo
