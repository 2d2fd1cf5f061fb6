// Split-K flash decoding on bf16 MFMA for gfx950 (head_dim 128).
//
// One decoding step of one layer: every retrieval KV head attends over its full cache
// (t + 1 rows) and every streaming KV head over its sink + recent slots, one launch for
// both kinds (hotpaper.ai page "DuoAttention: Efficient Long-Context LLM Inference
// with Retrieval and Streaming Heads", abstract: full KV cache for retrieval heads, a
// constant-length cache for streaming heads, decoding speed-up).  Each workgroup takes
// one key range of one KV head for all G query heads of that KV head (GQA shares every
// K/V byte read), keeps an online softmax in the base-2 domain, and writes an fp32
// partial (m, l, o); the last workgroup of each KV head merges the partials.
//
// Per wavefront, 32 keys at a time, with v_mfma_f32_16x16x32_bf16:
//   S^T[16 keys x 16 queries] = K[16 keys x 128] * Q^T   (two tiles, 4 k-steps each)
//   O^T[16 d x 16 queries]  += V^T[16 d x 32 keys] * P^T  (8 d-blocks)
// Query columns beyond G are zero and ignored.  Tile rows are loaded in the key order
// that makes each lane's 8 scores the 8 consecutive keys that lane then needs as the
// B operand of P*V, so probabilities never leave registers; V is read from the cache's
// d-major 8-key tiles, which already are the A-operand order of V^T.
#include "decode_common.h"

namespace duo {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ inline f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Largest x over lanes l, l ^ 16, l ^ 32 and l ^ 48 (the four 16-lane rows holding one
// query's scores), by two register swaps (v_permlane16_swap: rows 0 <-> 1 and 2 <-> 3;
// v_permlane32_swap: the wavefront's halves) instead of two LDS permutes and their waits.
__device__ inline float max_over_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Two floats to a bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ inline uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

constexpr int kWaves = 8;                 // wavefronts per decode workgroup (two per SIMD)
constexpr int kThreads = 64 * kWaves;
constexpr int kStride = 32 * kWaves;      // keys per round of the workgroup

struct Tile {
  u32x4 k0[4], k1[4];  // K rows for the two 16-key MFMA tiles, 4 k-steps each
  u32x4 v[8];          // V^T operand for the 8 d-blocks
};

// Buffer descriptor word 3 for raw (untyped) dword access on gfx9, and the
// non-temporal (streaming) cache policy for the tile loads.
constexpr int kRawBuffer = 0x00020000;
constexpr int kStreaming = 2;  // nt

// The split's K and V as bounds-checked buffers: a load past the split's last 32-key
// tile returns zeros without touching memory, so the ring can prefetch unconditionally
// (the compiler then counts every load) at no traffic cost.
struct SplitBuffers {
  __amdgpu_buffer_rsrc_t k, v;
};

// Loads the 32-key tile starting at key `base` (offset `rel` = base - key0 inside the
// split).  Lane l (row r = l % 16, group g = l / 16) holds key base + 8*(r/4) + (r%4)
// (tile 0) and that + 4 (tile 1), dims 32g .. 32g+31, and the V^T rows d = 16j + r of
// the 8-key block base + 8g.  K tiles are stored in operand order: chunk
// (t*4 + s)*64 + lane is one contiguous KB per load instruction.
__device__ inline void load_tile(Tile& t, const SplitBuffers& sb, int rel, int r, int grp) {
  const int lane = grp * 16 + r;
  const int kofs = (rel >> 5) * 8192 + lane * 16;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    t.k0[s] = __builtin_amdgcn_raw_buffer_load_b128(sb.k, kofs + s * 1024, 0, kStreaming);
    t.k1[s] = __builtin_amdgcn_raw_buffer_load_b128(sb.k, kofs + (4 + s) * 1024, 0, kStreaming);
  }
  const int vofs = (rel + 8 * grp) * 256 + r * 16;
#pragma unroll
  for (int j = 0; j < 8; ++j) t.v[j] = __builtin_amdgcn_raw_buffer_load_b128(sb.v, vofs + j * 256, 0, kStreaming);
}

// Merge of the split partials of one KV head (run by the last workgroup to finish).
// Each output element is owned by up to four threads; a thread walks its splits in
// batches of 32 whose (m, l, o) loads are all issued together, merging online with a
// running maximum, so a batch costs one memory round trip.  The owners of an element
// combine through LDS (`scratch`, 3 floats per thread).
__device__ void merge_splits_wide(const Geom& g, const DecodePlan& p, int b, int kvh, int nsplit, float* scratch,
                                  uint16_t* __restrict__ out) {
  constexpr int kBatch = 32;
  const int nout = g.G * 128;
  const int tpo = nout >= kThreads ? 1 : (kThreads / nout >= 4 ? 4 : kThreads / nout);  // owners per element
  const int per_pass = kThreads / tpo;
  const int part = threadIdx.x / per_pass;
  for (int e0 = 0; e0 < nout; e0 += per_pass) {
    const int e = e0 + threadIdx.x % per_pass;
    float M = kNegInf, L = 0.0f, acc = 0.0f;
    if (e < nout) {
      const int i = e >> 7, d = e & 127;
      for (int s0 = part; s0 < nsplit; s0 += kBatch * tpo) {
        float mm[kBatch], ll[kBatch], oo[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int s = s0 + u * tpo;
          if (s < nsplit) {
            const float* pp = partial_ptr(g, p, b, kvh * g.G + i, s);
            mm[u] = load_coherent(pp);
            ll[u] = load_coherent(pp + 1);
            oo[u] = load_coherent(pp + 2 + d);
          } else {
            mm[u] = kNegInf;
            ll[u] = 0.0f;
            oo[u] = 0.0f;
          }
        }
        float cm = M;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) cm = fmaxf(cm, mm[u]);
        const float ref = cm == kNegInf ? 0.0f : cm;
        const float sc = __builtin_amdgcn_exp2f(M - ref);
        L *= sc;
        acc *= sc;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const float w = __builtin_amdgcn_exp2f(mm[u] - ref);
          L = fmaf(w, ll[u], L);
          acc = fmaf(w, oo[u], acc);
        }
        M = cm;
      }
    }
    if (tpo > 1) {
      __syncthreads();
      scratch[3 * threadIdx.x] = M;
      scratch[3 * threadIdx.x + 1] = L;
      scratch[3 * threadIdx.x + 2] = acc;
      __syncthreads();
      if (part == 0) {
        for (int q2 = 1; q2 < tpo; ++q2) {
          const int o = 3 * (threadIdx.x + q2 * per_pass);
          const float M2 = scratch[o], L2 = scratch[o + 1], A2 = scratch[o + 2];
          const float Mx = fmaxf(M, M2);
          const float ref = Mx == kNegInf ? 0.0f : Mx;
          const float w1 = __builtin_amdgcn_exp2f(M - ref), w2 = __builtin_amdgcn_exp2f(M2 - ref);
          L = L * w1 + L2 * w2;
          acc = acc * w1 + A2 * w2;
          M = Mx;
        }
      }
    }
    if (part == 0 && e < nout)
      out[(int64_t(b) * g.Hq + kvh * g.G + (e >> 7)) * 128 + (e & 127)] = f32_to_bf16(acc / L);
  }
}

__global__ void __launch_bounds__(512) k_decode_mfma(Geom g, LayerView lv, DecodePlan p,
                                                       const uint16_t* __restrict__ q, uint16_t* __restrict__ out) {
  __shared__ float s_m[kWaves][16], s_l[kWaves][16];
  __shared__ __attribute__((aligned(16))) float s_o[kWaves][16][132];  // (16-byte rows) also the merge scratch

  const DecodeItem it = decode_item(g, lv, p, blockIdx.x);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
  const int r = lane & 15, grp = lane >> 4;
  const int G = g.G;
  const CacheRegion& c = it.retrieval ? lv.ret : lv.str;
  const uint16_t* K = reinterpret_cast<const uint16_t*>(c.k);
  const uint16_t* V = reinterpret_cast<const uint16_t*>(c.v);
  const int64_t row0 = it.cache * c.rows;
  // fused append of this step's token: retrieval row t or its streaming slot
  const int64_t new_row =
      p.k_new ? (it.retrieval ? it.t : p.varlen ? stream_slot(it.t, g.S, g.R) : p.new_slot) : -1;
  const uint16_t* k_new = p.k_new ? p.k_new + (int64_t(it.b) * g.Hkv + it.kvh) * 128 : nullptr;
  const uint16_t* v_new = p.v_new ? p.v_new + (int64_t(it.b) * g.Hkv + it.kvh) * 128 : nullptr;
  constexpr int kRing = 2;  // tiles in flight per wavefront
  const bool has_new = new_row >= it.key0 && new_row < it.key1;  // uniform
  // The workgroup whose range holds the new row writes it to the cache and waits for the
  // stores to land in its XCD's L2 before any of its wavefronts loads that row's tile:
  // the loads then see the new token like any other row.  When the row lies beyond the
  // tiles of the first ring round (the usual case: it is the last key of the range), the
  // first round's loads are issued before the write, so the write's latency hides
  // under theirs instead of delaying this workgroup, which has no slack when the splits
  // are all full.
  const bool append_late = has_new && new_row - it.key0 >= int64_t(kStride) * kRing;
  auto append = [&]() {
    if (threadIdx.x < 128) {
      uint16_t* Kw = reinterpret_cast<uint16_t*>(c.k);
      uint16_t* Vw = reinterpret_cast<uint16_t*>(c.v);
      const int d = threadIdx.x;
      Kw[k_chunk_tiled(row0 + new_row, d >> 3) + (d & 7)] = k_new[d];
      Vw[v_index(it.cache, c.rows, new_row, 128, d)] = v_new[d];
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  if (has_new && !append_late) append();

  // Q^T operand: column r = query head kvh*G + r (zero beyond G), dims 32g + 8s .. +7.
  u32x4 qop[4];
  {
    const bool real = r < G;
    const u32x4* qp = reinterpret_cast<const u32x4*>(q + (int64_t(it.b) * g.Hq + it.kvh * G + (real ? r : 0)) * 128 +
                                                     32 * grp);
#pragma unroll
    for (int s = 0; s < 4; ++s) qop[s] = real ? qp[s] : u32x4{0, 0, 0, 0};
  }

  float m = kNegInf, l = 0.0f;
  f32x4 o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const float sl2 = g.scale_log2;
  // Each wavefront takes every kWaves-th 32-key tile of the range and keeps a ring of
  // kRing tiles in flight: the slot just consumed is refilled with the tile kRing
  // rounds ahead (past the range: a bounds-checked load of zeros, no memory traffic).
  const int ntile32 = static_cast<int>((it.key1 - it.key0 + 31) >> 5);
  SplitBuffers sb;
  sb.k = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(K + ((row0 + it.key0) >> 5) * 4096), 0,
                                           ntile32 * 8192, kRawBuffer);
  sb.v = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(V + (row0 + it.key0) * 128), 0, ntile32 * 8192,
                                           kRawBuffer);
  Tile ring[kRing];
  const int rel0 = 32 * wave;
  // this wavefront's tiles, processed kRing per iteration with no early exit (a tile
  // past the range is all zeros and fully masked: it adds nothing)
  const int64_t span = it.key1 - it.key0 - rel0;
  const int n_tiles = span > 0 ? static_cast<int>((span + kStride - 1) / kStride) : 0;
  const int n_iter = __builtin_amdgcn_readfirstlane((n_tiles + kRing - 1) / kRing);
#pragma unroll
  for (int u = 0; u < kRing; ++u) load_tile(ring[u], sb, rel0 + kStride * u, r, grp);
  if (append_late) append();
  for (int iter = 0; iter < n_iter; ++iter) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      const int rel = rel0 + kStride * (kRing * iter + u);
      const int64_t base = it.key0 + rel;
      Tile& cur = ring[u];
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        s0 = mfma16(cur.k0[s], qop[s], s0);
        s1 = mfma16(cur.k1[s], qop[s], s1);
      }
      // lane holds scores of keys base + 8*grp + 0..7 for query r; keys past the range
      // become -inf, the max is kept on raw scores and the scale folded into the FMA
      float sc[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
      const int64_t kfirst = base + 8 * grp;
      if (base + 32 > it.key1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) sc[i] = kfirst + i < it.key1 ? sc[i] : kNegInf;
      }
      float mx = sc[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sc[i]);
      mx = max_over_rows(mx) * sl2;
      const float mn = fmaxf(m, mx);
      const float mref = mn == kNegInf ? 0.0f : mn;
      if (__ballot(mn > m)) {  // some lane's max moved: rescale (alpha is exactly 1 elsewhere)
        const float alpha = __builtin_amdgcn_exp2f(m - mref);
        l *= alpha;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] *= alpha;
      }
      m = mn;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sc[i] = __builtin_amdgcn_exp2f(fmaf(sc[i], sl2, -mref));
        l += sc[i];
      }
      const u32x4 pb = {pack_bf16(sc[0], sc[1]), pack_bf16(sc[2], sc[3]), pack_bf16(sc[4], sc[5]),
                        pack_bf16(sc[6], sc[7])};
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = mfma16(cur.v[j], pb, o[j]);
      load_tile(cur, sb, rel + kStride * kRing, r, grp);
    }
  }

  // Combine the wavefronts: lane sums over its group, then across waves in LDS (only
  // the G real query columns are written).
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (r < G) {
    if (grp == 0) {
      s_m[wave][r] = m;
      s_l[wave][r] = l;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<f32x4*>(&s_o[wave][r][16 * j + 4 * grp]) = o[j];
  }
  __syncthreads();

  const int pairs = G * 128;
  for (int e = threadIdx.x; e < pairs; e += kThreads) {
    const int qi = e >> 7, d = e & 127;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][qi]);
    float L = 0.0f, acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = s_l[w][qi] > 0.0f ? __builtin_amdgcn_exp2f(s_m[w][qi] - M) : 0.0f;
      L = fmaf(wt, s_l[w][qi], L);
      acc = fmaf(wt, s_o[w][qi][d], acc);
    }
    const int h = it.kvh * G + qi;
    if (it.nsplit == 1) {
      out[(int64_t(it.b) * g.Hq + h) * 128 + d] = f32_to_bf16(acc / L);
    } else {
      float* pp = partial_ptr(g, p, it.b, h, it.split);
      store_coherent(pp + 2 + d, acc);
      if (d == 0) {
        store_coherent(pp, M);
        store_coherent(pp + 1, L);
      }
    }
  }
  if (it.nsplit > 1 && last_arrival(p.counters + it.b * g.Hkv + it.kvh, it.nsplit))
    merge_splits_wide(g, p, it.b, it.kvh, it.nsplit, &s_o[0][0][0], out);
}

// ---- int4 caches ------------------------------------------------------------------
//
// Codes enter the bf16 MFMA as the exact values 128 + c (bf16 bits 0x4300 | c), built
// with one byte permute per pair of codes, and the per-vector scale s and zero z are
// applied algebraically (hotpaper.ai page, abstract and main results: the method runs
// with a 4-bit KV cache; the format is one group per 128-value vector with fp16 s, z):
//   score_j = s_j * (sum_d q_d (128 + c_jd) - 128 * sum_d q_d) + z_j * sum_d q_d
//   o_d     = sum_j p'_j (128 + c_jd) - 128 * sum_j p'_j + sum_j p_j z_j,  p'_j = bf16(p_j s_j)
// which equals attention over the dequantised values s*c + z up to rounding.

// Eight 4-bit codes (byte b: codes 2b low, 2b+1 high) -> eight bf16 values 128 + c in
// the element order (0, 2, 4, 6, 1, 3, 5, 7).
__device__ inline u32x4 codes_to_bf16(uint32_t x) {
  const uint32_t lo = x & 0x0F0F0F0Fu;
  const uint32_t hi = (x >> 4) & 0x0F0F0F0Fu;
  const uint32_t k43 = 0x43434343u;
  return u32x4{__builtin_amdgcn_perm(k43, lo, 0x04010400u), __builtin_amdgcn_perm(k43, lo, 0x04030402u),
               __builtin_amdgcn_perm(k43, hi, 0x04010400u), __builtin_amdgcn_perm(k43, hi, 0x04030402u)};
}

// Reorder 8 bf16 (one u32x4, element order 0..7) to (0, 2, 4, 6, 1, 3, 5, 7).
__device__ inline u32x4 even_odd_bf16(u32x4 v) {
  return u32x4{__builtin_amdgcn_perm(v[1], v[0], 0x05040100u), __builtin_amdgcn_perm(v[3], v[2], 0x05040100u),
               __builtin_amdgcn_perm(v[1], v[0], 0x07060302u), __builtin_amdgcn_perm(v[3], v[2], 0x07060302u)};
}

__device__ inline float half_lo(uint32_t w) { return __half2float(__ushort_as_half(static_cast<unsigned short>(w & 0xffff))); }
__device__ inline float half_hi(uint32_t w) { return __half2float(__ushort_as_half(static_cast<unsigned short>(w >> 16))); }

struct Tile4 {
  uint32_t k0[4], k1[4];  // 32 codes (16 bytes) of the two K rows, one word per k-step
  uint32_t v[8];          // 8 codes (keys of the lane's block) for dims 16j + r
  u32x4 km0, km1;         // K (scale, zero) of keys base + 8g + 0..7 (4 per u32x4)
  u32x4 vm0, vm1;         // V (scale, zero) of the same keys
};

__device__ inline void load_tile4(Tile4& t, const CacheRegion& c, int64_t cache, int64_t base, int r, int grp) {
  const int64_t row0 = cache * c.rows;
  // K codes: 32-key tiles of 2 KB in operand order, one contiguous KB per instruction
  const u32x4* kt = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(c.k) + ((row0 + base) >> 5) * 2048) +
                    grp * 16 + r;
  const u32x4 a = __builtin_nontemporal_load(kt);
  const u32x4 b = __builtin_nontemporal_load(kt + 64);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    t.k0[s] = a[s];
    t.k1[s] = b[s];
  }
  const uint32_t* vw = reinterpret_cast<const uint32_t*>(c.v) + (row0 + base + 8 * grp) / 8 * 128 + r;
#pragma unroll
  for (int j = 0; j < 8; ++j) t.v[j] = __builtin_nontemporal_load(vw + 16 * j);
  const u32x4* km = reinterpret_cast<const u32x4*>(c.k_meta + (row0 + base + 8 * grp) * 2);
  const u32x4* vm = reinterpret_cast<const u32x4*>(c.v_meta + (row0 + base + 8 * grp) * 2);
  t.km0 = __builtin_nontemporal_load(km);
  t.km1 = __builtin_nontemporal_load(km + 1);
  t.vm0 = __builtin_nontemporal_load(vm);
  t.vm1 = __builtin_nontemporal_load(vm + 1);
}

__global__ void __launch_bounds__(512) k_decode_mfma_int4(Geom g, LayerView lv, DecodePlan p,
                                                            const uint16_t* __restrict__ q, uint16_t* __restrict__ out) {
  __shared__ float s_m[kWaves][16], s_l[kWaves][16];
  __shared__ __attribute__((aligned(16))) float s_o[kWaves][16][132];  // (16-byte rows) also the merge scratch

  const DecodeItem it = decode_item(g, lv, p, blockIdx.x);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
  const int r = lane & 15, grp = lane >> 4;
  const int G = g.G;
  const CacheRegion& c = it.retrieval ? lv.ret : lv.str;

  // Fused append of this step's token (retrieval row t or its streaming slot): the
  // workgroup whose range holds the row quantises K (wavefront 0) and V (wavefront 1)
  // exactly as the append kernel does and stores codes and (scale, zero) before any of
  // its wavefronts loads the row's tile (after the first ring round's loads when the row
  // lies beyond them, as in the bf16 kernel).  V codes share a word with the 7 other rows
  // of their 8-row block (never split between workgroups: splits are multiples of 64
  // rows); the token's nibbles go in with device-scope atomics, which bypass the CU's L1,
  // so the tile loads that follow cannot meet a stale line.
  constexpr int kRing = 3;  // tiles in flight per wavefront
  const int64_t new_row =
      p.k_new ? (it.retrieval ? it.t : p.varlen ? stream_slot(it.t, g.S, g.R) : p.new_slot) : -1;
  const bool has_new = new_row >= it.key0 && new_row < it.key1;  // uniform
  const bool append_late = has_new && new_row - it.key0 >= int64_t(kStride) * kRing;
  auto append = [&]() {
    if (wave < 2) {
      const uint16_t* src = (wave == 0 ? p.k_new : p.v_new) + (int64_t(it.b) * g.Hkv + it.kvh) * 128 + 2 * lane;
      const uint32_t x = *reinterpret_cast<const uint32_t*>(src);
      const Q4 qq = quantize_pair(bf16_to_f32(x & 0xffff), bf16_to_f32(x >> 16));
      const int64_t grow = it.cache * c.rows + new_row;
      uint16_t* meta = (wave == 0 ? c.k_meta : c.v_meta) + grow * 2;
      if (wave == 0) {
        reinterpret_cast<uint8_t*>(c.k)[k_code_byte(grow, lane)] = static_cast<uint8_t>(qq.q0 | (qq.q1 << 4));
      } else {
        uint32_t* vw = reinterpret_cast<uint32_t*>(c.v) + (grow & ~int64_t(7)) / 8 * 128 + 2 * lane;
        const int sh = 4 * static_cast<int>(new_row & 7);
        __hip_atomic_fetch_and(vw, ~(15u << sh), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_and(vw + 1, ~(15u << sh), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_or(vw, qq.q0 << sh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_or(vw + 1, qq.q1 << sh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (lane == 0) {
        meta[0] = qq.s_bits;
        meta[1] = qq.z_bits;
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  if (has_new && !append_late) append();

  // Q^T operand in the codes' element order; Qsum = sum of the query's 128 values.
  u32x4 qop[4];
  float qsum;
  {
    const bool real = r < G;
    const u32x4* qp = reinterpret_cast<const u32x4*>(q + (int64_t(it.b) * g.Hq + it.kvh * G + (real ? r : 0)) * 128 +
                                                     32 * grp);
    float part = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 v = real ? qp[s] : u32x4{0, 0, 0, 0};
      qop[s] = even_odd_bf16(v);
#pragma unroll
      for (int e = 0; e < 4; ++e) part += bf16_to_f32(v[e] & 0xffff) + bf16_to_f32(v[e] >> 16);
    }
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    qsum = part;
  }
  const float q128 = 128.0f * qsum;

  float m = kNegInf, l = 0.0f, zsum = 0.0f;
  f32x4 o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // sum_j p'_j over all 32 keys of a tile, on the matrix core: a row of bf16 ones
  // times P'^T (every row of the result holds the sum)
  f32x4 pacc = {0.f, 0.f, 0.f, 0.f};
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const float sl2 = g.scale_log2;
  Tile4 ring[kRing];
  const int64_t first = it.key0 + 32 * wave;
  const int64_t fallback = first < it.key1 ? first : it.key0;  // unconditional loads, as above
#pragma unroll
  for (int u = 0; u < kRing; ++u) {
    const int64_t b = first + kStride * u;
    load_tile4(ring[u], c, it.cache, b < it.key1 ? b : fallback, r, grp);
  }
  if (append_late) append();
  for (int64_t base0 = first; base0 < it.key1; base0 += kStride * kRing) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      const int64_t base = base0 + kStride * u;
      if (base >= it.key1) break;
      Tile4& cur = ring[u];
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        s0 = mfma16(codes_to_bf16(cur.k0[s]), qop[s], s0);
        s1 = mfma16(codes_to_bf16(cur.k1[s]), qop[s], s1);
      }
      // keys base + 8*grp + i: (scale, zero) pairs in km0 (i < 4) and km1 (i >= 4)
      float sc[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t mk = i < 4 ? cur.km0[i] : cur.km1[i - 4];
        sc[i] = fmaf(half_lo(mk), sc[i] - q128, half_hi(mk) * qsum);
      }
      const int64_t kfirst = base + 8 * grp;
      if (base + 32 > it.key1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) sc[i] = kfirst + i < it.key1 ? sc[i] : kNegInf;
      }
      float mx = sc[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sc[i]);
      mx = max_over_rows(mx) * sl2;
      const float mn = fmaxf(m, mx);
      const float mref = mn == kNegInf ? 0.0f : mn;
      if (__ballot(mn > m)) {
        const float alpha = __builtin_amdgcn_exp2f(m - mref);
        l *= alpha;
        zsum *= alpha;
        pacc *= alpha;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] *= alpha;
      }
      m = mn;
      float pw[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pi = __builtin_amdgcn_exp2f(fmaf(sc[i], sl2, -mref));
        const uint32_t mv = i < 4 ? cur.vm0[i] : cur.vm1[i - 4];
        l += pi;
        zsum = fmaf(pi, half_hi(mv), zsum);
        pw[i] = pi * half_lo(mv);
      }
      // P'^T operand in the V codes' key order (0, 2, 4, 6, 1, 3, 5, 7)
      const u32x4 pb = {pack_bf16(pw[0], pw[2]), pack_bf16(pw[4], pw[6]), pack_bf16(pw[1], pw[3]),
                        pack_bf16(pw[5], pw[7])};
      pacc = mfma16(ones, pb, pacc);
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = mfma16(codes_to_bf16(cur.v[j]), pb, o[j]);
      const int64_t nb = base + kStride * kRing;
      load_tile4(cur, c, it.cache, nb < it.key1 ? nb : fallback, r, grp);
    }
  }

  // Per-query corrections are summed over the lane's group, then applied to its O.
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  zsum += __shfl_xor(zsum, 16);
  zsum += __shfl_xor(zsum, 32);
  const float corr = zsum - 128.0f * pacc[0];  // pacc already sums all 32 keys of each tile
  if (r < G) {  // only the G real query columns
    if (grp == 0) {
      s_m[wave][r] = m;
      s_l[wave][r] = l;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<f32x4*>(&s_o[wave][r][16 * j + 4 * grp]) = o[j] + f32x4{corr, corr, corr, corr};
  }
  __syncthreads();

  const int pairs = G * 128;
  for (int e = threadIdx.x; e < pairs; e += kThreads) {
    const int qi = e >> 7, d = e & 127;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][qi]);
    float L = 0.0f, acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = s_l[w][qi] > 0.0f ? __builtin_amdgcn_exp2f(s_m[w][qi] - M) : 0.0f;
      L = fmaf(wt, s_l[w][qi], L);
      acc = fmaf(wt, s_o[w][qi][d], acc);
    }
    const int h = it.kvh * G + qi;
    if (it.nsplit == 1) {
      out[(int64_t(it.b) * g.Hq + h) * 128 + d] = f32_to_bf16(acc / L);
    } else {
      float* pp = partial_ptr(g, p, it.b, h, it.split);
      store_coherent(pp + 2 + d, acc);
      if (d == 0) {
        store_coherent(pp, M);
        store_coherent(pp + 1, L);
      }
    }
  }
  if (it.nsplit > 1 && last_arrival(p.counters + it.b * g.Hkv + it.kvh, it.nsplit))
    merge_splits_wide(g, p, it.b, it.kvh, it.nsplit, &s_o[0][0][0], out);
}

}  // namespace

hipError_t launch_decode_mfma(const Geom& g, const LayerView& lv, const DecodePlan& p, const void* q, void* out,
                              hipStream_t st) {
  const int items = g.B * (lv.n_ret * p.nsplit_r + lv.n_str * p.nsplit_s);
  if (items == 0) return hipSuccess;
  if (g.kvfmt == DUO_KV_INT4_G128)
    launch(k_decode_mfma_int4, dim3(items), dim3(kThreads), 0, st, g, lv, p, static_cast<const uint16_t*>(q),
                       static_cast<uint16_t*>(out));
  else
    launch(k_decode_mfma, dim3(items), dim3(kThreads), 0, st, g, lv, p, static_cast<const uint16_t*>(q),
                       static_cast<uint16_t*>(out));
  return hipGetLastError();
}

}  // namespace duo
