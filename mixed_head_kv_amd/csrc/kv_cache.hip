// KV-cache kernels: fused append/evict (with int4 quantisation), inspection reads,
// counter clearing and the seeded synthetic fill.
//
// Append/evict follows the cache split of the hotpaper.ai page "DuoAttention:
// Efficient Long-Context LLM Inference with Retrieval and Streaming Heads" (abstract
// and technical-approach section): a retrieval head keeps every token, a streaming
// head keeps a constant-length cache of the attention sinks and the recent tokens.
#include "duo_kernels.h"

namespace duo {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Source token (index into the chunk) that lands in destination row `row`, or -1.
// Retrieval rows are absolute positions.  Streaming slot s < S holds sink position s;
// a ring slot holds the unique position p >= S with p = S + (s - S) mod R that is
// among the last R tokens of the sequence after the chunk.
__device__ inline int source_token(bool streaming, int64_t row, int64_t t0, int T, int S, int R) {
  if (!streaming) {
    int64_t t = row - t0;
    return (t >= 0 && t < T) ? static_cast<int>(t) : -1;
  }
  if (row >= S + R) return -1;
  if (row < S) {
    int64_t t = row - t0;
    return (t >= 0 && t < T) ? static_cast<int>(t) : -1;
  }
  int64_t hi = t0 + T;
  int64_t lo = t0;
  if (lo < S) lo = S;
  if (lo < hi - R) lo = hi - R;
  if (lo >= hi) return -1;
  int64_t want = row - S;                      // ring index of this slot
  int64_t have = (lo - S) % R;                 // ring index of position lo
  int64_t p = lo + ((want - have) % R + R) % R;
  return p < hi ? static_cast<int>(p - t0) : -1;
}

// One thread per (8-row tile, dimension d).  K rows are copied element by element
// (coalesced across d); the 8 V values of the tile are gathered and written as one
// contiguous 8-element run of the d-major tile layout.
template <typename T>
__global__ void __launch_bounds__(256) k_append(Geom g, LayerView lv, const T* __restrict__ k,
                                                const T* __restrict__ v, int T_, int64_t t0, int which,
                                                int64_t ret_tile0, int ret_tiles, int str_tiles) {
  const int D = g.D;
  const int per_block = 256 / D;
  const int d = threadIdx.x % D;
  const int local = threadIdx.x / D;
  const int nret = g.B * lv.n_ret;
  const int y = blockIdx.y;
  const bool streaming = y >= nret;
  if (streaming && !(which & 2)) return;
  if (!streaming && !(which & 1)) return;
  const int cache = streaming ? y - nret : y;
  const int b = streaming ? cache / lv.n_str : cache / lv.n_ret;
  const int idx = streaming ? cache % lv.n_str : cache % lv.n_ret;
  const int kvh = streaming ? lv.str_kv[idx] : lv.ret_kv[idx];
  const CacheRegion& c = streaming ? lv.str : lv.ret;
  const int tile = blockIdx.x * per_block + local;
  if (tile >= (streaming ? str_tiles : ret_tiles)) return;
  const int64_t row0 = (streaming ? int64_t(tile) : ret_tile0 + tile) * 8;
  T* K = reinterpret_cast<T*>(c.k);
  T* V = reinterpret_cast<T*>(c.v);
  T vbuf[8];
  int nvalid = 0;
  for (int r = 0; r < 8; ++r) {
    const int64_t row = row0 + r;
    const int t = source_token(streaming, row, t0, T_, g.S, g.R);
    if (t >= 0) {
      const int64_t src = ((int64_t(b) * T_ + t) * g.Hkv + kvh) * D + d;
      K[k_index(c, cache, row, D, d)] = k[src];
      vbuf[r] = v[src];
      ++nvalid;
    }
  }
  if (nvalid == 8) {
    T* dst = V + v_index(cache, c.rows, row0, D, d);
#pragma unroll
    for (int r = 0; r < 8; ++r) dst[r] = vbuf[r];
  } else if (nvalid) {
    for (int r = 0; r < 8; ++r) {
      const int64_t row = row0 + r;
      if (source_token(streaming, row, t0, T_, g.S, g.R) >= 0) V[v_index(cache, c.rows, row, D, d)] = vbuf[r];
    }
  }
}

// bf16 append, one thread per (8-row tile, 8-dim chunk): eight 16-byte K row pieces are
// copied as they are, and the 8x8 block of V is transposed in registers (byte
// permutes) into eight 16-byte runs of the d-major tile layout.  Tiles with rows that
// receive no token (range edges, evicted ring slots) write row by row.
__global__ void __launch_bounds__(256) k_append_bf16(Geom g, LayerView lv, const uint16_t* __restrict__ k,
                                                     const uint16_t* __restrict__ v, int T_, int64_t t0, int which,
                                                     int64_t ret_tile0, int ret_tiles, int str_tiles,
                                                     int64_t ring_lo, int ring_have) {
  const int D = g.D;
  const int nchunk = D / 8;
  const int nret = g.B * lv.n_ret;
  const int y = blockIdx.y;
  const bool streaming = y >= nret;
  if (streaming && !(which & 2)) return;
  if (!streaming && !(which & 1)) return;
  const int task = blockIdx.x * 256 + threadIdx.x;
  const int tile = task / nchunk, ch = task % nchunk;
  if (tile >= (streaming ? str_tiles : ret_tiles)) return;
  const int cache = streaming ? y - nret : y;
  const int b = streaming ? cache / lv.n_str : cache / lv.n_ret;
  const int idx = streaming ? cache % lv.n_str : cache % lv.n_ret;
  const int kvh = streaming ? lv.str_kv[idx] : lv.ret_kv[idx];
  const CacheRegion& c = streaming ? lv.str : lv.ret;
  const int64_t row0 = (streaming ? int64_t(tile) : ret_tile0 + tile) * 8;
  uint16_t* K = reinterpret_cast<uint16_t*>(c.k);
  uint16_t* V = reinterpret_cast<uint16_t*>(c.v);
  int src[8];
  int nvalid = 0;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    src[r] = source_token_fast(streaming, row0 + r, t0, T_, g.S, g.R, ring_lo, ring_have);
    nvalid += src[r] >= 0;
  }
  if (nvalid == 0) return;
  const int64_t in0 = (int64_t(b) * T_) * g.Hkv + kvh;  // input row of token t: in0 + t * Hkv
  // Every row loads unconditionally (a row without a token reads token 0 and drops it):
  // loads under a branch whose other side writes the same registers are each waited for
  // before the next row's, one memory round trip per row.
  // (The empty asm statements consume the K values where they stand, so the compiler
  // cannot sink each K load into its row's conditional store.)
  u32x4 kr[8];
  uint4 vr[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int64_t off = (in0 + int64_t(src[r] < 0 ? 0 : src[r]) * g.Hkv) * D + 8 * ch;
    kr[r] = *reinterpret_cast<const u32x4*>(k + off);
    vr[r] = *reinterpret_cast<const uint4*>(v + off);
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) asm volatile("" : "+v"(kr[r]));
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    if (src[r] < 0) continue;
    const int64_t grow = int64_t(cache) * c.rows + row0 + r;
    *reinterpret_cast<u32x4*>(K + (c.k_tiled ? k_chunk_tiled(grow, ch) : grow * D + 8 * ch)) = kr[r];
  }
  // V tile: element (row r, dim 8ch + e) goes to tile[8ch + e][r]
  uint16_t* vt = V + (int64_t(cache) * c.rows + row0) * D + 8 * ch * 8;
  if (nvalid == 8) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(vr);  // w[4r + e/2] holds dims e, e+1 of row r
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      uint4 out;
      out.x = __builtin_amdgcn_perm(w[4 * 1 + e / 2], w[4 * 0 + e / 2], sel);
      out.y = __builtin_amdgcn_perm(w[4 * 3 + e / 2], w[4 * 2 + e / 2], sel);
      out.z = __builtin_amdgcn_perm(w[4 * 5 + e / 2], w[4 * 4 + e / 2], sel);
      out.w = __builtin_amdgcn_perm(w[4 * 7 + e / 2], w[4 * 6 + e / 2], sel);
      *reinterpret_cast<uint4*>(vt + e * 8) = out;
    }
  } else {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (src[r] < 0) continue;
      const uint16_t* x = reinterpret_cast<const uint16_t*>(&vr[r]);
#pragma unroll
      for (int e = 0; e < 8; ++e) vt[e * 8 + r] = x[e];
    }
  }
}

// One wavefront per (cache, 8-row tile); D = 128, bf16 input.
__global__ void __launch_bounds__(256) k_append_int4(Geom g, LayerView lv, const uint16_t* __restrict__ k,
                                                     const uint16_t* __restrict__ v, int T_, int64_t t0,
                                                     int which, int64_t ret_tile0, int ret_tiles,
                                                     int str_tiles) {
  const int lane = threadIdx.x & 63;
  const int tile = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nret = g.B * lv.n_ret;
  const int y = blockIdx.y;
  const bool streaming = y >= nret;
  if (streaming && !(which & 2)) return;
  if (!streaming && !(which & 1)) return;
  if (tile >= (streaming ? str_tiles : ret_tiles)) return;
  const int cache = streaming ? y - nret : y;
  const int b = streaming ? cache / lv.n_str : cache / lv.n_ret;
  const int idx = streaming ? cache % lv.n_str : cache % lv.n_ret;
  const int kvh = streaming ? lv.str_kv[idx] : lv.ret_kv[idx];
  const CacheRegion& c = streaming ? lv.str : lv.ret;
  const int64_t row0 = (streaming ? int64_t(tile) : ret_tile0 + tile) * 8;
  uint8_t* kc = reinterpret_cast<uint8_t*>(c.k);
  uint32_t* vw = reinterpret_cast<uint32_t*>(c.v) + (cache * c.rows + row0) / 8 * 128;
  uint32_t w0 = 0, w1 = 0, written = 0;
  for (int r = 0; r < 8; ++r) {
    const int64_t row = row0 + r;
    const int t = source_token(streaming, row, t0, T_, g.S, g.R);
    if (t < 0) continue;
    const int64_t src = ((int64_t(b) * T_ + t) * g.Hkv + kvh) * 128 + 2 * lane;
    const uint32_t kp = *reinterpret_cast<const uint32_t*>(k + src);
    const uint32_t vp = *reinterpret_cast<const uint32_t*>(v + src);
    const Q4 qk = quantize_pair(bf16_to_f32(kp & 0xffff), bf16_to_f32(kp >> 16));
    const Q4 qv = quantize_pair(bf16_to_f32(vp & 0xffff), bf16_to_f32(vp >> 16));
    kc[k_code_byte(cache * c.rows + row, lane)] = static_cast<uint8_t>(qk.q0 | (qk.q1 << 4));
    if (lane == 0) {
      uint16_t* km = c.k_meta + (cache * c.rows + row) * 2;
      uint16_t* vm = c.v_meta + (cache * c.rows + row) * 2;
      km[0] = qk.s_bits;
      km[1] = qk.z_bits;
      vm[0] = qv.s_bits;
      vm[1] = qv.z_bits;
    }
    w0 |= qv.q0 << (4 * r);
    w1 |= qv.q1 << (4 * r);
    written |= 15u << (4 * r);
  }
  if (!written) return;
  if (written != 0xffffffffu) {
    w0 |= vw[2 * lane] & ~written;
    w1 |= vw[2 * lane + 1] & ~written;
  }
  vw[2 * lane] = w0;
  vw[2 * lane + 1] = w1;
}

template <int IO, int KVF>
__global__ void k_read(Geom g, CacheRegion c, int64_t cache, int streaming, int64_t pos0, int n, int which,
                       float* __restrict__ out) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= int64_t(n) * g.D) return;
  const int64_t p = pos0 + i / g.D;
  const int d = static_cast<int>(i % g.D);
  const int64_t row = streaming ? stream_slot(p, g.S, g.R) : p;
  out[i] = which == 0 ? cache_k<IO, KVF>(c, cache, row, g.D, d) : cache_v<IO, KVF>(c, cache, row, g.D, d);
}

__global__ void k_read_int4(Geom g, CacheRegion c, int64_t cache, int streaming, int64_t pos0, int n, int which,
                            uint8_t* __restrict__ codes, uint16_t* __restrict__ meta) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;  // one byte of codes
  if (i >= int64_t(n) * 64) return;
  const int64_t p = pos0 + i / 64;
  const int kb = static_cast<int>(i % 64);
  const int64_t row = streaming ? stream_slot(p, g.S, g.R) : p;
  uint8_t byte;
  if (which == 0) {
    byte = reinterpret_cast<const uint8_t*>(c.k)[k_code_byte(cache * c.rows + row, kb)];
  } else {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(c.v) + (cache * c.rows + (row & ~int64_t(7))) / 8 * 128;
    const uint32_t lo = (w[2 * kb] >> (4 * (row & 7))) & 15u;
    const uint32_t hi = (w[2 * kb + 1] >> (4 * (row & 7))) & 15u;
    byte = static_cast<uint8_t>(lo | (hi << 4));
  }
  codes[i] = byte;
  if (kb < 2) {
    const uint16_t* m = (which == 0 ? c.k_meta : c.v_meta) + (cache * c.rows + row) * 2;
    meta[(i / 64) * 2 + kb] = m[kb];
  }
}

__global__ void k_zero_i32(int* p, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

__global__ void k_zero_16b(uint4* p, uint64_t n) {
  for (uint64_t i = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += uint64_t(gridDim.x) * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

// SplitMix64 finaliser (Steele, Lea and Flood, OOPSLA 2014).
__device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

template <int IO>
__global__ void k_synth(typename IoType<IO>::T* __restrict__ out, uint64_t key, uint64_t c0, uint64_t n) {
  const float kScale = 0x1.bb67ae0000000p-16f;  // float32 nearest to sqrt(3) / 65536
  for (uint64_t i = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += uint64_t(gridDim.x) * blockDim.x) {
    const uint64_t w = mix64(key + (c0 + i + 1) * 0x9E3779B97F4A7C15ull);
    const int s = static_cast<int>((w & 0xffff) + ((w >> 16) & 0xffff) + ((w >> 32) & 0xffff) + (w >> 48));
    const float x = static_cast<float>(s - 131070) * kScale;
    if constexpr (IO == DUO_DTYPE_F32) out[i] = x;
    else if constexpr (IO == DUO_SYNTH_INT8) out[i] = static_cast<int8_t>(rintf(x * 32.0f));
    else out[i] = f32_to_bf16(x);
  }
}

uint64_t host_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

}  // namespace

hipError_t launch_append(const Geom& g, const LayerView& lv, const void* k, const void* v, int T, int64_t t0,
                         int which, hipStream_t st) {
  const int64_t first = t0 / 8, last = (t0 + T - 1) / 8;
  const int ret_tiles = static_cast<int>(last - first + 1);
  const int str_tiles = (g.S + g.R + 7) / 8;
  const int ny = g.B * (lv.n_ret + lv.n_str);
  if (ny == 0) return hipSuccess;
  if (g.kvfmt == DUO_KV_INT4_G128) {
    const int tiles = ret_tiles > str_tiles ? ret_tiles : str_tiles;
    dim3 grid((tiles + 3) / 4, ny);
    launch(k_append_int4, grid, dim3(256), 0, st, g, lv, static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), T, t0, which, first, ret_tiles, str_tiles);
  } else {
    const int tiles = ret_tiles > str_tiles ? ret_tiles : str_tiles;
    if (g.io == DUO_DTYPE_BF16) {
      int64_t ring_lo = t0 > g.S ? t0 : g.S;
      if (ring_lo < t0 + T - g.R) ring_lo = t0 + T - g.R;
      const int ring_have = ring_lo >= g.S ? static_cast<int>((ring_lo - g.S) % g.R) : 0;
      const int64_t tasks = int64_t(tiles) * (g.D / 8);
      dim3 grid(static_cast<unsigned>((tasks + 255) / 256), ny);
      launch(k_append_bf16, grid, dim3(256), 0, st, g, lv, static_cast<const uint16_t*>(k),
                         static_cast<const uint16_t*>(v), T, t0, which, first, ret_tiles, str_tiles, ring_lo, ring_have);
      return hipGetLastError();
    }
    const int per_block = 256 / g.D;
    dim3 grid((tiles + per_block - 1) / per_block, ny);
    if (g.io == DUO_DTYPE_F32)
      launch(k_append<float>, grid, dim3(per_block * g.D), 0, st, g, lv, static_cast<const float*>(k),
                         static_cast<const float*>(v), T, t0, which, first, ret_tiles, str_tiles);
    else
      launch(k_append<uint16_t>, grid, dim3(per_block * g.D), 0, st, g, lv,
                         static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), T, t0, which, first,
                         ret_tiles, str_tiles);
  }
  return hipGetLastError();
}

hipError_t launch_read(const Geom& g, const CacheRegion& c, int64_t cache, bool streaming, int64_t pos0, int n,
                       int which, float* out, hipStream_t st) {
  const int64_t total = int64_t(n) * g.D;
  dim3 grid(static_cast<unsigned>((total + 255) / 256));
  if (g.kvfmt == DUO_KV_INT4_G128)
    launch(k_read<DUO_DTYPE_BF16, DUO_KV_INT4_G128>, grid, dim3(256), 0, st, g, c, cache,
                       int(streaming), pos0, n, which, out);
  else if (g.io == DUO_DTYPE_F32)
    launch(k_read<DUO_DTYPE_F32, DUO_KV_SAME_AS_IO>, grid, dim3(256), 0, st, g, c, cache,
                       int(streaming), pos0, n, which, out);
  else
    launch(k_read<DUO_DTYPE_BF16, DUO_KV_SAME_AS_IO>, grid, dim3(256), 0, st, g, c, cache,
                       int(streaming), pos0, n, which, out);
  return hipGetLastError();
}

hipError_t launch_read_int4(const Geom& g, const CacheRegion& c, int64_t cache, bool streaming, int64_t pos0,
                            int n, int which, uint8_t* codes, uint16_t* meta, hipStream_t st) {
  const int64_t total = int64_t(n) * 64;
  launch(k_read_int4, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, st, g, c, cache,
                     int(streaming), pos0, n, which, codes, meta);
  return hipGetLastError();
}

hipError_t launch_zero_i32(int* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  launch(k_zero_i32, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

// Guard bands of the workspace: up to 64 per launch, one workgroup per band, each of its
// DUO_GUARD_BYTES / 4 threads writing one 32-bit word.
struct GuardList {
  uint64_t off[64];
  int n;
};

__global__ void k_guard_fill(char* base, GuardList g, uint32_t word) {
  if (static_cast<int>(blockIdx.x) < g.n && threadIdx.x < DUO_GUARD_BYTES / 4)
    reinterpret_cast<uint32_t*>(base + g.off[blockIdx.x])[threadIdx.x] = word;
}

hipError_t launch_guard_fill(char* base, const uint64_t* offsets, int n, uint32_t word, hipStream_t st) {
  for (int i = 0; i < n; i += 64) {
    GuardList g = {};
    g.n = n - i < 64 ? n - i : 64;
    for (int j = 0; j < g.n; ++j) g.off[j] = offsets[i + j];
    launch(k_guard_fill, dim3(static_cast<unsigned>(g.n)), dim3(DUO_GUARD_BYTES / 4), 0, st, base, g, word);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_zero_bytes(void* p, uint64_t n_bytes, hipStream_t st) {
  const uint64_t n = n_bytes / 16;
  if (n == 0) return hipSuccess;
  uint64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  launch(k_zero_16b, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, static_cast<uint4*>(p), n);
  return hipGetLastError();
}

hipError_t launch_synth(void* out, int dtype, uint64_t seed, uint32_t stream, uint64_t c0, uint64_t n,
                        hipStream_t st) {
  if (n == 0) return hipSuccess;
  const uint64_t key = host_mix64((seed << 32) | stream);
  uint64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (dtype == DUO_DTYPE_F32)
    launch(k_synth<DUO_DTYPE_F32>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                       static_cast<float*>(out), key, c0, n);
  else if (dtype == DUO_SYNTH_INT8)
    launch(k_synth<DUO_SYNTH_INT8>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                       static_cast<int8_t*>(out), key, c0, n);
  else
    launch(k_synth<DUO_DTYPE_BF16>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                       static_cast<uint16_t*>(out), key, c0, n);
  return hipGetLastError();
}

}  // namespace duo
