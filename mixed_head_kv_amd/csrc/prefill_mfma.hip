// Flash-style pre-filling on bf16 MFMA for gfx950 (head_dim 128), one kernel with two
// key sources:
//   retrieval heads: causal attention of the chunk's queries over every key [0, i],
//     read from the retrieval cache (the chunk is appended to it first);
//   streaming heads: the Lambda-shaped mask of sinks [0, S) plus the recent window
//     (i - R, i], over keys staged (k_chunk_tiles) into the same cache layout: the
//     sink rows, then the window rows of the launch's queries, taken from the chunk
//     inputs and from the constant-length cache as it stood before the chunk.
// Source: hotpaper.ai page "DuoAttention: Efficient Long-Context LLM Inference with
// Retrieval and Streaming Heads", abstract (full attention for retrieval heads, recent
// tokens and sinks for streaming heads, lower pre-filling latency) and its technical-
// approach section; cn.bg3.co article, 研究背景 section (pre-filling cost of full
// attention grows quadratically with the context).
//
// Workgroup: 4 or 8 wavefronts x 32 queries; under GQA its wavefronts take up to 4 query
// heads of one KV head (each head's query slices spread over the wavefronts), so each
// K/V tile in LDS serves every head of the group.  Keys move HBM -> LDS with
// direct loads in 64-key tiles, double-buffered (K rows with their 16-byte chunks
// XOR-swizzled by the row index so the permuted row reads hit distinct banks; V in
// d-major 8-key blocks).  Per 32-key half tile each wavefront runs, with
// v_mfma_f32_32x32x16_bf16,
//   S^T[32 keys x 32 queries] = K * Q^T    (8 k-steps over head_dim)
//   O^T[32 d x 32 queries]   += V^T * P^T  (4 d-blocks x 2 k-steps)
// Rows of the K operand are read in the permuted key order that leaves each lane
// holding, per k-step of P*V, the probabilities of 8 consecutive keys: exactly the
// B operand, so P stays in registers.  Every lane owns one query, so the online
// softmax rescale is lane-uniform; the row max needs one cross-half exchange.
#include <cstdlib>

#include "decode_common.h"

namespace duo {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTileKeys = 64;
constexpr int kKBytes = kTileKeys * 256;           // K rows, 16-byte chunks XOR-swizzled by row
constexpr int kVBytes = kTileKeys * 128 * 2;       // 16384
constexpr int kStageRows = 64;
// Workgroup shape, by wavefront count W (4 or 8): 32 (query, head) rows per wavefront,
// and each wavefront moves 16 / W of the tile's 16 K and 16 V kilobytes into LDS.
template <int W>
struct Shape {
  static constexpr int kRows = 32 * W;                      // (query, head) rows per workgroup
  static constexpr int kThreads = 64 * W;
  static constexpr int kDma = 16 / W;                       // 1 KB loads per wavefront, K and V each
  static constexpr int kSlotFloats = kRows * 128 + 2 * kRows;  // one split's partial (below)
};

__device__ inline f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats to a bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ inline uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// acc + lo + hi of a bf16 pair (one v_dot2 against (1, 1); the products are exact).
__device__ inline float sum_bf16_pair(uint32_t pair, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), __builtin_bit_cast(bf16x2, 0x3f803f80u), acc,
                                         false);
}

constexpr float kSlack = 8.0f;  // log2 units

// Wavefront issue priority (s_setprio) around the MFMA sections of the tile routine, in
// 4-wavefront workgroups (two per CU): of the two wavefronts sharing a SIMD, the one with
// matrix work ready issues it first and the other fills the cycles between with its
// softmax, so the matrix pipe idles less (measured 7-10% off the retrieval prefill).  The
// scheduling barriers keep the compiler from moving instructions across the change.  In
// 8-wavefront workgroups the two wavefronts of a SIMD meet at every tile's barrier and
// the raise, with the scheduling fences it needs, measured ~1% slower: none there.
template <int P, bool kOn>
__device__ inline void set_priority() {
  if constexpr (kOn) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(P);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// max(x of this lane, x of lane ^ 32): one v_permlane32_swap instead of an LDS permute.
__device__ inline float max_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Largest of 32 scores as a shallow tree of v_max3 (independent partial maxima).
__device__ inline float max32(const f32x16& a, const f32x16& b) {
  float t[11];
#pragma unroll
  for (int i = 0; i < 5; ++i) t[i] = fmaxf(fmaxf(a[3 * i], a[3 * i + 1]), a[3 * i + 2]);
  t[5] = fmaxf(fmaxf(a[15], b[0]), b[1]);
#pragma unroll
  for (int i = 0; i < 4; ++i) t[6 + i] = fmaxf(fmaxf(b[2 + 3 * i], b[3 + 3 * i]), b[4 + 3 * i]);
  t[10] = b[14];
  const float u0 = fmaxf(fmaxf(t[0], t[1]), t[2]), u1 = fmaxf(fmaxf(t[3], t[4]), t[5]);
  const float u2 = fmaxf(fmaxf(t[6], t[7]), t[8]), u3 = fmaxf(fmaxf(t[9], t[10]), b[15]);
  return fmaxf(fmaxf(u0, u1), fmaxf(u2, u3));
}

// Workgroups of one head kind in a prefill launch: (sequence, head group, query block,
// split), longest blocks first.  A head group is `pack` query heads of one KV head
// (GQA: they read the same K/V tiles, so one tile in LDS serves them all); a query
// block is 128 / pack queries, so a workgroup always holds 128 (query, head) rows, 32
// per wavefront: wavefront w takes head w % pack and queries 32 (w / pack) .. +31.
struct KindGrid {
  int n_heads;    // query heads of this kind per sequence
  int pack;       // query heads per workgroup: 4, 2 or 1, a divisor of G
  int qrows;      // queries per workgroup: 128 / pack
  int n_qblocks;  // ceil(nq / qrows)
  int nsplit;     // workgroups sharing one query block's key range (1 or 2; retrieval only)
  int q0, nq;     // queries: chunk rows [q0, q0 + nq)
  int blocks;     // B * (n_heads / pack) * n_qblocks * nsplit
};

// The per-launch scalars of a chunk-tile pass (k_chunk_tiles below).
struct ChunkScalars {
  const uint16_t* k;  // chunk inputs [B, T, Hkv, 128]
  const uint16_t* v;
  int T;
  int64_t t0;
  int ret_caches;     // blockIdx.y < ret_caches: retrieval append of cache y
  int64_t ret_tile0;  // first 64-row tile holding a chunk row
  int ret_tiles;
  int str_tiles;
  int64_t ring_lo;    // update: first chunk position kept in the cache (see source_token_fast)
  int ring_have;      // update: its ring index
  int64_t u_end;      // staging: end of the launch's query positions
  int sink_rows;      // staging: Sp
  int64_t p0;         // staging: position of window row Sp
};

template <bool UPDATE>
__device__ void chunk_tiles_body(const Geom& g, const LayerView& lv, const CacheRegion& stage, const ChunkScalars& a,
                                 int bx, int by, uint4 (*s_k)[16], uint16_t (*s_v)[128], int tid, bool active);

struct PrefillArgs {
  Geom g;
  LayerView lv;
  const uint16_t* q;    // [B, T, Hq, 128]
  uint16_t* out;        // [B, T, Hq, 128]
  int T;                // tokens of the chunk (row stride of q and out)
  int64_t t0;           // position of chunk row 0
  KindGrid ret;         // blocks [0, ret.blocks): retrieval heads
  KindGrid str;         // blocks [ret.blocks, ret.blocks + str.blocks): streaming heads
  float* scratch;       // split retrieval blocks: per (block, split) fp32 partial, Shape<W>::kSlotFloats each
  int* counters;        // split retrieval blocks: arrival counter per query block
  CacheRegion stage;    // streaming heads: the staged keys, one region per streaming cache
  int stage_sink_rows;  // streaming heads: staged sink rows (before the window rows)
  int64_t stage_p0;     // streaming heads: position held by the first window row
  // Both outputs of every head (head identification): when set, every KV head is a
  // retrieval head and the second grid computes every head's sink + window attention
  // over the retrieval caches, written here ([B, T, Hq, 128]).
  uint16_t* out_lambda;
  // Blocks [ret.blocks + str.blocks, + upd_blocks): the streaming caches' update with the
  // chunk (the k_chunk_tiles<true> pass), run in the same launch when every streaming
  // query of the chunk was staged before it (nothing later reads the cache as it stood).
  ChunkScalars upd;
  int upd_tiles;        // 64-row update tiles (str_tiles per streaming cache)
  int upd_blocks;       // workgroups running them, W / 4 tiles each
};

// Partial of one split of one workgroup's block: O [rows][128 dims], then m[rows],
// l[rows] (rows = 32 W); row 32 w + c is wavefront w's query c (of its head).

// Split partials move with buffer instructions carrying the sc1 cache-policy bit
// (device-coherent: written through / read past the XCD-local L2), so a partial written
// on one XCD is read correctly on another.  0x00020000 is the gfx9 buffer-descriptor
// word 3 for raw (untyped) dword access; num_records bounds every access to the slot.
constexpr int kCoherent = 16;  // sc1
template <int W>
__device__ inline __amdgpu_buffer_rsrc_t slot_rsrc(float* slot) {
  return __builtin_amdgcn_make_buffer_rsrc(slot, 0, Shape<W>::kSlotFloats * 4, 0x00020000);
}
// Byte offset of float4 chunk `c` (dims 4c .. 4c + 3) of row `ql` in a partial.
template <int W>
__device__ inline int o_chunk_offset(int c, int ql) { return (c * Shape<W>::kRows + ql) * 16; }

// Query head (of this kind) with index `idx`: the idx-th query head whose KV head has
// this kind, in KV-head-major order.
__device__ inline int kind_head(const PrefillArgs& a, bool streaming, int idx, int* kvh) {
  const int G = a.g.G;
  const int kv = streaming ? a.lv.str_kv[idx / G] : a.lv.ret_kv[idx / G];
  *kvh = kv;
  return kv * G + idx % G;
}

typedef __attribute__((address_space(3))) void* lds_void_ptr;
constexpr int kTileBytes = 64 * 128 * 2;   // one 64-key tile of K or of V
constexpr int kRsrcWord3 = 0x00020000;    // buffer descriptor word 3: 32-bit data format

// Retrieval tiles go HBM -> LDS directly (buffer_load_dwordx4 ... lds): each wavefront
// instruction fills one contiguous KB of LDS, lane L writing bytes 16L .. 16L + 15, so
// no registers hold the tile in flight.  The K KB `inst` holds rows 4 inst .. 4 inst + 3
// of the swizzled row-major tile, its lane L the chunk (row 4 inst + L/16, physical
// chunk L mod 16), gathered from the cache's MFMA-ordered 32-key tiles; V's d-major
// 8-key blocks are copied as they are.  `wave` is uniform; the caller waits (vmcnt)
// and synchronises before reading.  The buffer form (one descriptor per 16 KB tile)
// rather than the global one: the compiler counts a global load into LDS as an LDS
// access as well, and while one is in flight it waits for every outstanding LDS read
// before each product instead of for the one operand the product needs.
template <int W>
__device__ inline void tile_dma(const CacheRegion& c, int64_t cache, int64_t kb, char* ldsK, char* ldsV, int wave,
                                int lane, const int (&koff)[Shape<W>::kDma]) {
  constexpr int kDma = Shape<W>::kDma;
  // kb and the cache's first row are multiples of 32: the tile's 32-key cache tiles are
  // whole, and each lane's element offset inside them is loop-invariant (koff)
  const uint16_t* Kt = reinterpret_cast<const uint16_t*>(c.k) + ((cache * c.rows + kb) >> 5) * 4096;
  const char* Vt = c.v + ((cache * c.rows + kb) * 128) * 2;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Kt), 0, kTileBytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(Vt), 0, kTileBytes, kRsrcWord3);
#pragma unroll
  for (int u = 0; u < kDma; ++u) {
    const int inst = wave * kDma + u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_ptr)(ldsK + inst * 1024), 16, koff[u] * 2, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_ptr)(ldsV + inst * 1024), 16, inst * 1024 + lane * 16, 0, 0, 0);
  }
}

// Element offsets (inside a 64-key tile of the MFMA-ordered K cache) of the chunks lane
// `lane` of wavefront `wave` moves: LDS row 4 inst + L/16, physical chunk L mod 16 of the
// swizzled tile, inst = kDma wave + u.
template <int W>
__device__ inline void tile_dma_offsets(int wave, int lane, int (&koff)[Shape<W>::kDma]) {
#pragma unroll
  for (int u = 0; u < Shape<W>::kDma; ++u) {
    const int row = (wave * Shape<W>::kDma + u) * 4 + (lane >> 4);
    const int col16 = (lane & 15) ^ (row & 15);
    koff[u] = static_cast<int>(k_chunk_tiled(row, col16));
  }
}

// K operand of k-step st for the S^T product of a 32-key half tile starting at LDS row
// `row0`: lane (col, half) supplies key row0 + pi(col) and dims 64 half + 8 st .. +7, where
// pi(8j + 4h + i) = 16(j>>1) + 8h + 4(j&1) + i is the permuted key order that leaves each
// lane holding the probabilities of 8 consecutive keys.
__device__ inline int k_perm(int col) {
  return 16 * (col >> 4) + 8 * ((col >> 2) & 1) + 4 * ((col >> 3) & 1) + (col & 3);
}

// V^T operand (d-block jd, k-step u) of a 32-key half tile at LDS key `key0`: rows
// d = 32 jd + col, keys key0 + 16 u + 8 half .. +7, one 16-byte row of a d-major block.
__device__ inline u32x4 v_operand(const char* ldsV, int key0, int u, int jd, int col, int half) {
  return *reinterpret_cast<const u32x4*>(ldsV + ((key0 + 16 * u + 8 * half) >> 3) * 2048 + col * 16 + jd * 512);
}

// Scores of keys a query may not see become -inf, in place.  Register 4j + i of a
// 32-key block starting at position `base` holds key base + 8 half + c with
// c = 16(j>>1) + 4(j&1) + i; the query of the lane sits at position i_pos.  Visibility
// (the mask of the page's streaming heads splits into two disjoint key sets):
//   kMaskCausal : key <= i                      (retrieval heads)
//   kMaskSink   : key <= i and key < S          (streaming heads, sink rows)
//   kMaskWindow : key <= i, i - key < R, key >= S  (streaming heads, window rows)
// Each condition is a bound on c, computed once per block in 64-bit and clamped.
enum { kMaskCausal = 0, kMaskSink = 1, kMaskWindow = 2 };

__device__ inline int clamp_off(int64_t x) { return static_cast<int>(x < -1 ? -1 : (x > 64 ? 64 : x)); }

template <int KIND>
__device__ inline void mask_block(f32x16& s, int64_t base, int64_t i_pos, int half, int S, int R) {
  const int h8 = 8 * half;
  int c_hi = clamp_off(i_pos - base);  // key <= i
  int c_lo = -1;
  if (KIND == kMaskSink) c_hi = min(c_hi, clamp_off(S - base) - 1);                              // key < S
  if (KIND == kMaskWindow) c_lo = max(clamp_off(i_pos - R - base) + 1, clamp_off(S - base));  // i - key < R, key >= S
  c_hi -= h8;
  c_lo -= h8;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 16 * (j >> 1) + 4 * (j & 1) + i;
      s[4 * j + i] = (c <= c_hi && c >= c_lo) ? s[4 * j + i] : kNegInf;
    }
}

// Work a tile routine issues right after its first K reads (the next tile's loads into
// LDS in the unmasked loop, whose ~30 issue instructions then cover the reads' latency
// instead of delaying them).
struct NoIssue {
  __device__ void operator()() const {}
};

// One 64-key tile for the wavefront's 32 queries.  Both 32-key score blocks are formed
// first (16 MFMAs, the second block's K operands read while the first block's products
// run), the scores outside the mask are set to -inf in place when the tile needs it
// (`mask`, a uniform branch that touches only the score registers, so O stays in one
// register set), one running-max update serves the tile, and the probabilities are formed
// in four quarter steps of 8 keys per lane, each issued between the P*V MFMAs of the
// quarter before, so the vector ALU and the matrix cores work at the same time.  The running max m may lag the true one by up to kSlack
// (log2 units): weights are then at most 2^kSlack, harmless in fp32 and bf16, and the
// rescale (which touches all of O) runs only when some lane's max outgrows m + kSlack.
// `issue` runs once the K reads of the first score block are issued; kPrio selects the
// issue-priority raises around the MFMA sections.
template <bool kPrio, typename MaskFn, typename IssueFn = NoIssue>
__device__ __forceinline__ void tile_compute(const char* ldsK, const char* ldsV, const u32x4 (&qop)[8],
                                             f32x16 (&o)[4], float& m, float& l, float sl2, int col, int half,
                                             bool masked, const MaskFn& mask, const IssueFn& issue = IssueFn()) {
  const int pk = k_perm(col);
  const int sw = pk & 15;  // row swizzle (rows pk and 32 + pk share it)
  u32x4 kop[8];
#pragma unroll
  for (int st = 0; st < 8; ++st)
    kop[st] = *reinterpret_cast<const u32x4*>(ldsK + pk * 256 + (((8 * half + st) ^ sw) * 16));
  __builtin_amdgcn_sched_barrier(0);
  issue();
  __builtin_amdgcn_sched_barrier(0);
  set_priority<1, kPrio>();
  f32x16 s0 = {}, s1 = {};
#pragma unroll
  for (int st = 0; st < 8; ++st) s0 = mfma32(kop[st], qop[st], s0);
#pragma unroll
  for (int st = 0; st < 8; ++st)
    kop[st] = *reinterpret_cast<const u32x4*>(ldsK + (32 + pk) * 256 + (((8 * half + st) ^ sw) * 16));
  u32x4 v0[8];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int jd = 0; jd < 4; ++jd) v0[4 * u + jd] = v_operand(ldsV, 0, u, jd, col, half);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int st = 0; st < 8; ++st) s1 = mfma32(kop[st], qop[st], s1);
  set_priority<0, kPrio>();
  if (masked) {  // mask(s, off): scores of the 32-key block at tile offset off
    mask(s0, 0);
    mask(s1, 32);
  }
  const float mx = max_across_halves(max32(s0, s1)) * sl2;
  if (__ballot(mx > m + kSlack)) {
    const float mn = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f(m - (mn == kNegInf ? 0.0f : mn));
    l *= alpha;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] *= alpha;
    m = mn;
  }
  const float mref = m == kNegInf ? 0.0f : m;  // -inf only while every key so far is masked
  // Four quarter steps (8 keys of each lane per step): the exponentials and packing of a
  // step are issued while the MFMAs of the previous step run.
  u32x4 pb[4];
  auto probs = [&](const f32x16& sc, int h, u32x4& out) {
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(sc[8 * h + e], sl2, -mref));
    out = u32x4{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7])};
#pragma unroll
    for (int w = 0; w < 4; ++w) l = sum_bf16_pair(out[w], l);
  };
  probs(s0, 0, pb[0]);
  set_priority<1, kPrio>();
#pragma unroll
  for (int jd = 0; jd < 4; ++jd) o[jd] = mfma32(v0[jd], pb[0], o[jd]);
  probs(s0, 1, pb[1]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int jd = 0; jd < 4; ++jd) o[jd] = mfma32(v0[4 + jd], pb[1], o[jd]);
  probs(s1, 0, pb[2]);
#pragma unroll
  for (int jd = 0; jd < 4; ++jd) v0[jd] = v_operand(ldsV, 32, 0, jd, col, half);  // after its MFMA
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int jd = 0; jd < 4; ++jd) o[jd] = mfma32(v0[jd], pb[2], o[jd]);
  probs(s1, 1, pb[3]);
#pragma unroll
  for (int jd = 0; jd < 4; ++jd) v0[4 + jd] = v_operand(ldsV, 32, 1, jd, col, half);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int jd = 0; jd < 4; ++jd) o[jd] = mfma32(v0[4 + jd], pb[3], o[jd]);
  set_priority<0, kPrio>();
}

// Workgroups are dispatched to the 8 XCDs round-robin (id mod 8), each XCD with its own
// L2.  The G query heads of a KV head (times the key splits) read the same K/V tiles: a
// "unit" of U = G * nsplit logical ids.  This maps the dispatch id p so that the U ids of
// a unit share an XCD and are dispatched together (ids u mod 8 + 8 j of a run of 8 units),
// so the unit's tile reads after the first hit that XCD's L2; runs of 8 units keep the
// longest-first order.  Ids past the last whole run map to themselves.
__device__ inline int xcd_grouped(int p, int U, int n) {
  const int run = 8 * U;
  if (U <= 1 || p >= n / run * run) return p;
  const int r = p % run;
  return ((p / run) * 8 + r % 8) * U + r / 8;
}

// Retrieval workgroups (long) come first in the grid and streaming ones (short) after,
// so the streaming work fills the CUs that the retrieval blocks' uneven lengths leave
// idle towards the end of the launch.  W wavefronts per workgroup: 4 (two workgroups
// per CU) or 8 (one per CU, each tile shared by twice the rows: half the LDS fill per
// flop).
template <int W>
__global__ void __launch_bounds__(Shape<W>::kThreads, 8 / W) k_prefill_mfma(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];  // two tile buffers
  constexpr int kRows = Shape<W>::kRows;
  constexpr int kSlotFloats = Shape<W>::kSlotFloats;

  const Geom& g = a.g;
  const int upd0 = a.ret.blocks + a.str.blocks;
  if (static_cast<int>(blockIdx.x) >= upd0) {  // uniform: streaming cache update tiles
    // (256-thread tiles: a workgroup of W wavefronts runs W / 4 of them, each with its
    // own 32 KB of the LDS; a part past the last tile still takes the tile's barrier)
    const int part = static_cast<int>(threadIdx.x) >> 8;
    const int id = (static_cast<int>(blockIdx.x) - upd0) * (W / 4) + part;
    char* mine = lds + part * (kStageRows * 16 * 16 + kStageRows * 128 * 2);
    chunk_tiles_body<true>(g, a.lv, a.stage, a.upd, id % a.upd.str_tiles, id / a.upd.str_tiles,
                           reinterpret_cast<uint4(*)[16]>(mine),
                           reinterpret_cast<uint16_t(*)[128]>(mine + kStageRows * 16 * 16),
                           static_cast<int>(threadIdx.x) & 255, id < a.upd_tiles);
    return;
  }
  const bool streaming = static_cast<int>(blockIdx.x) >= a.ret.blocks;  // uniform
  const KindGrid& kg = streaming ? a.str : a.ret;
  const int n_groups = kg.n_heads / kg.pack;
  const int id = xcd_grouped(static_cast<int>(blockIdx.x) - (streaming ? a.ret.blocks : 0),
                             a.g.G / kg.pack * kg.nsplit, kg.blocks);
  // Longest query blocks first; head groups of one block adjacent.
  const int per_b = n_groups * kg.n_qblocks * kg.nsplit;
  const int b = id / per_b;
  const int rem = id % per_b;
  const int split = rem % kg.nsplit;
  const int hq = rem / kg.nsplit;
  const int qb = kg.n_qblocks - 1 - hq / n_groups;
  const int group = hq % n_groups;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
  const int col = lane & 31, half = lane >> 5;
  const int wq = wave / kg.pack;                          // the wavefront's 32-query slice
  // With both outputs requested the second grid reads the retrieval caches directly (row
  // = position) instead of staged streaming-cache keys.
  const bool dual = a.out_lambda != nullptr;
  const bool staged = streaming && !dual;
  int kvh;  // the same for every wavefront: pack divides G
  const int h = kind_head(a, staged, group * kg.pack + wave % kg.pack, &kvh);
  const int64_t cache = int64_t(b) * (staged ? a.lv.n_str : a.lv.n_ret) + a.lv.slot[kvh];

  const int q_first = kg.q0 + qb * kg.qrows;              // chunk-relative
  const int q_last = min(q_first + kg.qrows, kg.q0 + kg.nq) - 1;
  const int my_q = q_first + 32 * wq + col;               // this lane's query
  const bool q_valid = my_q <= q_last;
  const int64_t i_pos = a.t0 + (q_valid ? my_q : q_last); // absolute position
  const int64_t wave_q_hi = a.t0 + min(q_first + 32 * wq + 31, q_last);
  const int64_t wave_q_lo = a.t0 + q_first + 32 * wq;

  // Q^T operand: lane (col, half) holds dims 64*half + 8s .. +7 of its query, s = 0..7.
  u32x4 qop[8];
  {
    const int qrow = q_valid ? my_q : q_last;
    const u32x4* qp =
        reinterpret_cast<const u32x4*>(a.q + ((int64_t(b) * a.T + qrow) * g.Hq + h) * 128 + 64 * half);
#pragma unroll
    for (int s = 0; s < 8; ++s) qop[s] = qp[s];
  }

  float m = kNegInf, l = 0.0f;
  f32x16 o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[j][e] = 0.0f;

  const float sl2 = g.scale_log2;
  int koff[Shape<W>::kDma];
  tile_dma_offsets<W>(wave, lane, koff);

  if (!streaming) {
    // Retrieval: keys [0, t0 + q_last] of the cache, 64 per tile; a split takes a
    // contiguous share of the tiles (the diagonal ones go to the last split).  The leading
    // tiles hold only keys before the block's first query (visible to every query): they
    // run in a loop with the mask compiled out; the few tiles on the diagonal follow.
    const int64_t all_tiles = (a.t0 + q_last + kTileKeys) / kTileKeys;
    const int64_t t_begin = all_tiles * split / kg.nsplit;
    const int64_t ntiles = all_tiles * (split + 1) / kg.nsplit - t_begin;
    const int64_t kb_first = t_begin * kTileKeys;
    const int64_t first_q = a.t0 + q_first;
    int64_t n_inner = first_q >= kb_first + kTileKeys - 1 ? (first_q - (kb_first + kTileKeys - 1)) / kTileKeys + 1 : 0;
    if (n_inner > ntiles) n_inner = ntiles;
    if (ntiles > 0) tile_dma<W>(a.lv.ret, cache, kb_first, lds, lds + kKBytes, wave, lane, koff);
    __syncthreads();
    auto prefetch = [&](int64_t ti) {  // the next tile is in flight during the compute
      if (ti + 1 < ntiles) {
        char* nK = lds + ((ti + 1) & 1) * (kKBytes + kVBytes);
        tile_dma<W>(a.lv.ret, cache, kb_first + (ti + 1) * kTileKeys, nK, nK + kKBytes, wave, lane, koff);
      }
    };
    auto no_mask = [](f32x16&, int) {};
    // Tile ti sits in buffer ti & 1.  The unmasked loop takes two tiles per trip with the
    // buffer a compile-time constant, so each LDS read's buffer offset is an immediate of
    // the instruction and the per-lane read addresses stay in registers across tiles.
    auto inner = [&](int64_t t, auto buf) {
      const char* ldsK = lds + decltype(buf)::value * (kKBytes + kVBytes);
      tile_compute<W == 4>(ldsK, ldsK + kKBytes, qop, o, m, l, sl2, col, half, false, no_mask, [&] { prefetch(t); });
      __syncthreads();  // (waits for this wavefront's tile loads, LDS ones included)
    };
    int64_t ti = 0;
    for (; ti + 1 < n_inner; ti += 2) {
      inner(ti, std::integral_constant<int, 0>());
      inner(ti + 1, std::integral_constant<int, 1>());
    }
    if (ti < n_inner) inner(ti++, std::integral_constant<int, 0>());
    for (; ti < ntiles; ++ti) {
      const char* ldsK = lds + (ti & 1) * (kKBytes + kVBytes);
      const int64_t kb = kb_first + ti * kTileKeys;
      prefetch(ti);
      if (kb <= wave_q_hi) {  // (a tile wholly after the wavefront's queries is skipped)
        const bool inside = kb + kTileKeys - 1 <= wave_q_lo;  // every key visible to every query
        tile_compute<W == 4>(ldsK, ldsK + kKBytes, qop, o, m, l, sl2, col, half, !inside, [&](f32x16& sc, int off) {
          mask_block<kMaskCausal>(sc, kb + off, i_pos, half, 0, 0);
        });
      }
      __syncthreads();
    }
  } else {
    // Streaming: the staged sink tiles covering [0, min(S, last query + 1)), then the
    // staged window tiles covering [max(S, first query - R + 1), last query].  A
    // wavefront computes a tile when some key of it is visible to one of its queries,
    // masked unless every key is visible to all of them.
    const int S = g.S, R = g.R;
    const CacheRegion& src = dual ? a.lv.ret : a.stage;
    const int64_t sink_rows = dual ? 0 : a.stage_sink_rows;  // row of position p0 below
    const int64_t p0 = dual ? 0 : a.stage_p0;
    const int64_t qa = a.t0 + q_first, qz = a.t0 + q_last;
    const int n_sink = static_cast<int>(((S < qz + 1 ? S : qz + 1) + kTileKeys - 1) / kTileKeys);
    const int64_t lo = qa - R + 1 > S ? qa - R + 1 : S;
    const int64_t w_first = (sink_rows + lo - p0) / kTileKeys;
    const int n_win = lo <= qz ? static_cast<int>((sink_rows + qz - p0) / kTileKeys - w_first + 1) : 0;
    const int ntiles = n_sink + n_win;
    auto tile_row = [&](int ti) -> int64_t {
      return ti < n_sink ? int64_t(ti) * kTileKeys : (w_first + (ti - n_sink)) * kTileKeys;
    };
    const bool live = q_first + 32 * wq <= q_last;  // the wavefront has queries
    if (ntiles > 0) tile_dma<W>(src, cache, tile_row(0), lds, lds + kKBytes, wave, lane, koff);
    __syncthreads();
    for (int ti = 0; ti < ntiles; ++ti) {
      const char* ldsK = lds + (ti & 1) * (kKBytes + kVBytes);
      if (ti + 1 < ntiles) {  // the next tile is in flight during the compute
        char* nK = lds + ((ti + 1) & 1) * (kKBytes + kVBytes);
        tile_dma<W>(src, cache, tile_row(ti + 1), nK, nK + kKBytes, wave, lane, koff);
      }
      // (a window tile may cover sink rows too when S is not a multiple of 64: its mask
      // keeps keys >= S only, the sink tile's keys < S, so no key counts twice)
      const bool sink = ti < n_sink;
      const int64_t row = tile_row(ti);
      const int64_t p = sink ? row : p0 + (row - sink_rows);  // position of the first key
      const int64_t p_last = p + kTileKeys - 1;
      bool any, full;
      if (sink) {
        any = p < S && p <= wave_q_hi;
        full = p_last < S && p_last <= wave_q_lo;
      } else {
        any = p_last >= S && p <= wave_q_hi && p_last > wave_q_lo - R;
        full = p >= S && p_last <= wave_q_lo && p > wave_q_hi - R;
      }
      if (live && any)
        tile_compute<W == 4>(ldsK, ldsK + kKBytes, qop, o, m, l, sl2, col, half, !full, [&](f32x16& sc, int off) {
          if (sink)
            mask_block<kMaskSink>(sc, p + off, i_pos, half, S, R);
          else
            mask_block<kMaskWindow>(sc, p + off, i_pos, half, S, R);
        });
      __syncthreads();
    }
  }

  // normalise and store: lane holds query `col` of its wave, dims 32 jd + 8 j + 4 half + i
  l += __shfl_xor(l, 32);
  if (kg.nsplit > 1) {
    // Every split publishes its partial; the last one to arrive merges them all.  A
    // partial is O as float4 chunks [32 dim chunks][128 rows] (a wavefront's lanes
    // cover 512 contiguous bytes per store), then m[128] and l[128], all moved with
    // 16-byte device-coherent buffer accesses.
    const int pair = (b * n_groups + group) * kg.n_qblocks + qb;
    const int ql = 32 * wave + col;
    float* mine = a.scratch + (int64_t(pair) * kg.nsplit + split) * kSlotFloats;
    {
      const __amdgpu_buffer_rsrc_t rs = slot_rsrc<W>(mine);
#pragma unroll
      for (int jd = 0; jd < 4; ++jd)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 v = {__float_as_uint(o[jd][4 * j + 0]), __float_as_uint(o[jd][4 * j + 1]),
                           __float_as_uint(o[jd][4 * j + 2]), __float_as_uint(o[jd][4 * j + 3])};
          __builtin_amdgcn_raw_buffer_store_b128(v, rs, o_chunk_offset<W>(8 * jd + 2 * j + half, ql), 0, kCoherent);
        }
      if (half == 0) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m), rs, (kRows * 128 + ql) * 4, 0, kCoherent);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l), rs, (kRows * 128 + kRows + ql) * 4, 0, kCoherent);
      }
    }
    if (!last_arrival(a.counters + pair, kg.nsplit)) return;
    // Merge in split order whichever split arrived last, so the result is the same bits
    // on every run: L = sum_s w_s l_s, O = sum_s w_s O_s, w_s = 2^(m_s - M), the first
    // term a product and the rest fused multiply-adds.
    float M = m;
    for (int s2 = 0; s2 < kg.nsplit; ++s2) {
      if (s2 == split) continue;
      const __amdgpu_buffer_rsrc_t rs = slot_rsrc<W>(a.scratch + (int64_t(pair) * kg.nsplit + s2) * kSlotFloats);
      M = fmaxf(M, __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (kRows * 128 + ql) * 4, 0, kCoherent)));
    }
    float L = 0.0f;
    f32x16 acc[4];
    for (int s2 = 0; s2 < kg.nsplit; ++s2) {
      float ws, ls;  // an empty split has m = -inf: weight 0
      f32x16 os[4];
      if (s2 == split) {
        ws = __builtin_amdgcn_exp2f(m - M);
        ls = l;
#pragma unroll
        for (int jd = 0; jd < 4; ++jd) os[jd] = o[jd];
      } else {
        const __amdgpu_buffer_rsrc_t rs = slot_rsrc<W>(a.scratch + (int64_t(pair) * kg.nsplit + s2) * kSlotFloats);
        ws = __builtin_amdgcn_exp2f(
            __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (kRows * 128 + ql) * 4, 0, kCoherent)) - M);
        ls = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (kRows * 128 + kRows + ql) * 4, 0, kCoherent));
#pragma unroll
        for (int jd = 0; jd < 4; ++jd)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, o_chunk_offset<W>(8 * jd + 2 * j + half, ql), 0, kCoherent);
#pragma unroll
            for (int i = 0; i < 4; ++i) os[jd][4 * j + i] = __uint_as_float(v[i]);
          }
      }
      if (s2 == 0) {
        L = ws * ls;
#pragma unroll
        for (int jd = 0; jd < 4; ++jd) acc[jd] = os[jd] * ws;
      } else {
        L = fmaf(ws, ls, L);
#pragma unroll
        for (int jd = 0; jd < 4; ++jd)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[jd][e] = fmaf(ws, os[jd][e], acc[jd][e]);
      }
    }
    l = L;
#pragma unroll
    for (int jd = 0; jd < 4; ++jd) o[jd] = acc[jd];
  }
  if (q_valid) {
    const float inv = 1.0f / l;
    uint16_t* orow = (streaming && dual ? a.out_lambda : a.out) + ((int64_t(b) * a.T + my_q) * g.Hq + h) * 128;
#pragma unroll
    for (int jd = 0; jd < 4; ++jd)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * jd + 8 * j + 4 * half;
        const uint32_t w0 = pack_bf16(o[jd][4 * j + 0] * inv, o[jd][4 * j + 1] * inv);
        const uint32_t w1 = pack_bf16(o[jd][4 * j + 2] * inv, o[jd][4 * j + 3] * inv);
        *reinterpret_cast<uint2*>(orow + d) = make_uint2(w0, w1);
      }
  }
}

// Chunk keys into the layouts the attention kernel loads directly (MFMA-ordered K
// tiles, d-major V), one launch before the attention, two kinds of workgroup:
//
// Retrieval append: rows [t0, t0 + T) of every retrieval cache take the chunk's K/V
// (hotpaper.ai page, technical approach: retrieval heads keep every token).  Rows of
// the first and last 64-row tile outside that range are rewritten unchanged: earlier
// tokens are read back from the cache, rows past the chunk are zero (never written).
//
// Streaming cache update (after the chunk's attention): every slot of the constant-length
// cache that the chunk's tokens reach (a sink, or one of the last R positions) takes its
// token; the other slots are read back and rewritten unchanged.
//
// Streaming staging: the keys one launch of queries (chunk rows [q0, q0 + nq), positions
// [u0, u_end)) may see, per streaming cache, in a workspace region:
//   rows [0, Sp)            sink position = row, for row < S,
//   rows [Sp, Sp + W + n)   window position p0 + (row - Sp), p0 = u0 - W (W >= R - 1),
// each from the chunk input (position >= t0) or from the constant-length cache as it
// stood before the chunk (a sink, or one of the last R positions before t0).  Rows no
// query of the launch may see hold zeros (finite values, weighted by zero).
//
// One workgroup per 64 destination rows of one cache: row-major 16-byte loads (16 lanes
// per 256-byte row) into LDS, then every store instruction of a wavefront writes one
// contiguous KB of the cache layout (a 1 KB block of a K tile, or 64 dims x 8 keys of a V
// block).  Storing straight from registers (16 bytes per lane to 64 different lines per
// instruction) ran at under half the bandwidth.

struct ChunkTileArgs {
  Geom g;
  LayerView lv;
  CacheRegion stage;
  ChunkScalars s;
};

// UPDATE: the streaming cache update after the attention (its own instantiation, so
// profiles tell the two uses apart); otherwise the append + staging launch.
template <bool UPDATE>
__global__ void __launch_bounds__(256) k_chunk_tiles(ChunkTileArgs a) {
  __shared__ __attribute__((aligned(16))) uint4 s_k[kStageRows][16];  // chunk c of row r at [r][c ^ (r & 15)]
  __shared__ __attribute__((aligned(16))) uint16_t s_v[kStageRows][128];
  chunk_tiles_body<UPDATE>(a.g, a.lv, a.stage, a.s, static_cast<int>(blockIdx.x), static_cast<int>(blockIdx.y), s_k,
                           s_v, static_cast<int>(threadIdx.x), true);
}

// One 64-row tile (bx) of one cache (by) of a chunk-tile pass, run by 256 threads (tid
// 0..255); s_k, s_v: their LDS (s_k: chunk c of row r at [r][c ^ (r & 15)]).  Inactive
// (or past the last tile), the threads only take the one barrier the tile's threads
// take, so 256-thread parts of a larger workgroup stay in step.
template <bool UPDATE>
__device__ void chunk_tiles_body(const Geom& g, const LayerView& lv, const CacheRegion& stage, const ChunkScalars& a,
                                 int bx, int by, uint4 (*s_k)[16], uint16_t (*s_v)[128], int tid, bool active) {
  const bool ret = active && by < a.ret_caches;
  if (!active || bx >= (ret ? a.ret_tiles : a.str_tiles)) {  // uniform over the 256 threads
    __syncthreads();
    return;
  }
  const bool update = UPDATE && !ret;
  const int lane = tid & 63, wave = tid >> 6;
  const int cache = ret ? by : by - a.ret_caches;  // b * n_kind + index
  const int n_kind = ret ? lv.n_ret : lv.n_str;
  const int b = cache / n_kind;
  const int kvh = ret ? lv.ret_kv[cache % n_kind] : lv.str_kv[cache % n_kind];
  const int64_t row0 = (ret ? a.ret_tile0 + bx : int64_t(bx)) * kStageRows;
  const CacheRegion& held = ret ? lv.ret : lv.str;  // rows read back from a cache
  const CacheRegion& dst = ret ? lv.ret : (update ? lv.str : stage);
  const uint16_t* hk = reinterpret_cast<const uint16_t*>(held.k);
  const uint16_t* hv = reinterpret_cast<const uint16_t*>(held.v);
  const int ch = tid & 15;
  const int64_t in0 = int64_t(b) * a.T * g.Hkv + kvh;  // input row of chunk token t: in0 + t * Hkv
  const uint16_t* kin = a.k + in0 * 128 + 8 * ch;      // input token 0 of this head, chunk ch
  const uint16_t* vin = a.v + in0 * 128 + 8 * ch;

  // Source of each of the thread's 4 rows: 1 = chunk input, 2 = a cache row (`slot`),
  // 0 = none.  The loads are issued unconditionally from select-chosen addresses (a row
  // without an input reads input token 0 and discards it), all in flight together.
  int src[4], rr[4];
  int64_t slot[4];
  uint4 kr[4], vr[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    rr[u] = (tid >> 4) + 16 * u;
    const int64_t row = row0 + rr[u];
    int64_t tin = 0;
    if (ret) {
      tin = row - a.t0;
      src[u] = tin >= 0 ? (tin < a.T ? 1 : 0) : 2;
      slot[u] = row;
    } else if (update) {
      tin = source_token_fast(true, row, a.t0, a.T, g.S, g.R, a.ring_lo, a.ring_have);
      src[u] = tin >= 0 ? 1 : (row < g.S + g.R ? 2 : 0);
      slot[u] = row;
    } else {
      const bool sink = row < a.sink_rows;
      const int64_t pos = sink ? row : a.p0 + (row - a.sink_rows);
      const bool wanted = pos < a.u_end && (sink ? pos < g.S : pos >= g.S);
      src[u] = !wanted ? 0 : (pos >= a.t0 ? 1 : ((sink || pos >= a.t0 - g.R) ? 2 : 0));  // sinks, last R before t0
      slot[u] = src[u] == 2 ? stream_slot(pos, g.S, g.R) : 0;
      tin = pos - a.t0;
    }
    if (src[u] != 1) tin = 0;
    const uint16_t* kp = src[u] == 2 ? hk + k_chunk_tiled(int64_t(cache) * held.rows + slot[u], ch)
                                     : kin + tin * g.Hkv * 128;
    kr[u] = *reinterpret_cast<const uint4*>(kp);
    vr[u] = *reinterpret_cast<const uint4*>(vin + tin * g.Hkv * 128);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (src[u] == 0) kr[u] = make_uint4(0, 0, 0, 0);
    if (src[u] != 1) vr[u] = make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (src[u] == 2) {  // V of a cache row: eight 2-byte elements of the cache's d-major blocks
      uint16_t x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = hv[v_index(cache, held.rows, slot[u], 128, 8 * ch + e)];
      vr[u] = make_uint4(uint32_t(x[0]) | (uint32_t(x[1]) << 16), uint32_t(x[2]) | (uint32_t(x[3]) << 16),
                         uint32_t(x[4]) | (uint32_t(x[5]) << 16), uint32_t(x[6]) | (uint32_t(x[7]) << 16));
    }
    s_k[rr[u]][ch ^ (rr[u] & 15)] = kr[u];
    *reinterpret_cast<uint4*>(&s_v[rr[u]][8 * ch]) = vr[u];
  }
  __syncthreads();

  // K: 16 blocks of 1 KB (two 32-key tiles); block 8 q + 4 t + s, lane (grp, r) holds
  // dims 8 (4 grp + s) .. +7 of key 32 q + 8 (r >> 2) + (r & 3) + 4 t.
  uint16_t* sk = reinterpret_cast<uint16_t*>(dst.k) + ((int64_t(cache) * dst.rows + row0) >> 5) * 4096;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int blk = 4 * u + wave;
    const int r = lane & 15, c = 4 * (lane >> 4) + (blk & 3);
    const int key = 32 * (blk >> 3) + 8 * (r >> 2) + (r & 3) + 4 * ((blk >> 2) & 1);
    *reinterpret_cast<uint4*>(sk + (blk * 64 + lane) * 8) = s_k[key][c ^ (key & 15)];
  }
  // V: 8 blocks of 8 keys x 128 dims; unit (block b8, dim d) = keys 8 b8 .. +7 of dim d.
  uint16_t* sv = reinterpret_cast<uint16_t*>(dst.v) + (int64_t(cache) * dst.rows + row0) * 128;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int idx = tid + 256 * u;
    const int b8 = idx >> 7, d = idx & 127;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = uint32_t(s_v[8 * b8 + 2 * j][d]) | (uint32_t(s_v[8 * b8 + 2 * j + 1][d]) << 16);
    *reinterpret_cast<uint4*>(sv + (8 * b8) * 128 + d * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace

// Wavefronts per prefill workgroup for a chunk's attention: 8 when G is a multiple of 4
// (four heads of a KV head in every workgroup, two 32-query slices each), else 4 (MHA:
// 256-query blocks measured slower than 128).  The streaming-only launches use 4.
int prefill_waves(const Geom& g) { return g.G % 4 == 0 ? 8 : 4; }

// Grid of n_heads query heads (KV-head-major) over chunk rows [q0, q0 + nq) for
// workgroups of W wavefronts: head groups of the largest of 4, 2, 1 heads that divides
// G, query blocks of 32 W / pack rows.
static KindGrid kind_grid(const Geom& g, int W, int n_heads, int q0, int nq, int nsplit) {
  KindGrid k = {};
  k.n_heads = n_heads;
  k.pack = g.G % 4 == 0 ? 4 : (g.G % 2 == 0 ? 2 : 1);
  k.qrows = 32 * W / k.pack;
  k.n_qblocks = (nq + k.qrows - 1) / k.qrows;
  k.nsplit = nsplit;
  k.q0 = q0;
  k.nq = nq;
  k.blocks = nq > 0 ? g.B * (n_heads / k.pack) * k.n_qblocks * nsplit : 0;
  return k;
}

// Streaming-head grid of the queries in chunk rows [q0, q0 + nq).
static KindGrid streaming_grid(const Geom& g, int W, const LayerView& lv, int q0, int nq) {
  return kind_grid(g, W, lv.n_str * g.G, q0, nq, 1);
}

static PrefillArgs prefill_args(const Geom& g, const LayerView& lv, const CacheRegion& stage, const void* q,
                                void* out, int T, int64_t t0) {
  PrefillArgs a = {};
  a.g = g;
  a.lv = lv;
  a.q = static_cast<const uint16_t*>(q);
  a.out = static_cast<uint16_t*>(out);
  a.T = T;
  a.t0 = t0;
  a.stage = stage;
  a.stage_sink_rows = stage_sink_rows(g.S);
  a.ret = a.str = kind_grid(g, 4, 0, 0, 0, 1);
  return a;
}

// Scalars of the streaming caches' update with chunk rows [t0, t0 + T) (every cache:
// str_tiles tiles each).
static ChunkScalars update_scalars(const Geom& g, const LayerView& lv, const void* k, const void* v, int T,
                                   int64_t t0) {
  ChunkScalars u = {};
  u.k = static_cast<const uint16_t*>(k);
  u.v = static_cast<const uint16_t*>(v);
  u.T = T;
  u.t0 = t0;
  u.str_tiles = static_cast<int>(lv.str.rows / kStageRows);
  int64_t ring_lo = t0 > g.S ? t0 : g.S;
  if (ring_lo < t0 + T - g.R) ring_lo = t0 + T - g.R;
  u.ring_lo = ring_lo;
  u.ring_have = static_cast<int>((ring_lo - g.S) % g.R);
  return u;
}

hipError_t launch_prefill_mfma(const Geom& g, const LayerView& lv, const CacheRegion& stage, const void* q, void* out,
                               int T, int64_t t0, int nq_streaming, float* scratch, int64_t scratch_floats,
                               int* counters, int num_cu, hipStream_t st, void* out_lambda, const void* upd_k,
                               const void* upd_v, PrefillLaunchInfo* info) {
  PrefillArgs a = prefill_args(g, lv, stage, q, out, T, t0);
  a.out_lambda = static_cast<uint16_t*>(out_lambda);
  const int W = prefill_waves(g);
  const int64_t slot_floats = W == 8 ? Shape<8>::kSlotFloats : Shape<4>::kSlotFloats;
  if (upd_k && g.B * lv.n_str > 0) {  // the streaming caches' update joins the launch
    a.upd = update_scalars(g, lv, upd_k, upd_v, T, t0);
    a.upd_tiles = a.upd.str_tiles * g.B * lv.n_str;
    a.upd_blocks = (a.upd_tiles + W / 4 - 1) / (W / 4);
  }
  KindGrid& r = a.ret;
  r = kind_grid(g, W, lv.n_ret * g.G, 0, T, 1);
  // Split a query block's keys over two workgroups when the retrieval blocks alone would
  // leave fewer than eight wavefronts per CU (one wavefront per SIMD cannot hide its own
  // MFMA, LDS and barrier latencies) and the keys and scratch allow it.
  const int64_t pairs = int64_t(g.B) * (r.n_heads / r.pack) * r.n_qblocks;
  int nsplit = 1;
  if (pairs < 8 / W * int64_t(num_cu) && t0 + T >= 2048 && pairs <= kPrefillCounters &&
      pairs * 2 * slot_floats <= scratch_floats)
    nsplit = 2;
  if (const char* e = std::getenv("DUO_PREFILL_SPLIT")) {
    const int f = std::atoi(e);
    if (f == 1 || (f == 2 && pairs <= kPrefillCounters && pairs * 2 * slot_floats <= scratch_floats)) nsplit = f;
  }
  r.nsplit = nsplit;
  r.blocks = static_cast<int>(pairs * nsplit);
  a.scratch = scratch;
  a.counters = counters;
  if (out_lambda) {  // every head, every query of the chunk, over the retrieval caches
    a.str = kind_grid(g, W, r.n_heads, 0, T, 1);
  } else {
    a.str = streaming_grid(g, W, lv, 0, nq_streaming);
  }
  a.stage_p0 = t0 - stage_window_rows(g.R);
  const int64_t blocks = int64_t(r.blocks) + a.str.blocks + a.upd_blocks;
  if (info) *info = PrefillLaunchInfo{W, r.pack, r.qrows, r.nsplit, r.blocks, a.str.blocks, a.upd_blocks};
  if (blocks == 0) return hipSuccess;
  if (W == 8)
    launch(k_prefill_mfma<8>, dim3(static_cast<unsigned>(blocks)), dim3(Shape<8>::kThreads), 2 * (kKBytes + kVBytes),
           st, a);
  else
    launch(k_prefill_mfma<4>, dim3(static_cast<unsigned>(blocks)), dim3(Shape<4>::kThreads), 2 * (kKBytes + kVBytes),
           st, a);
  return hipGetLastError();
}

hipError_t launch_chunk_tiles(const Geom& g, const LayerView& lv, const CacheRegion& stage, const void* k,
                              const void* v, int T, int64_t t0, bool retrieval, int q0, int nq, hipStream_t st) {
  ChunkTileArgs a = {};
  a.g = g;
  a.lv = lv;
  a.stage = stage;
  a.s.k = static_cast<const uint16_t*>(k);
  a.s.v = static_cast<const uint16_t*>(v);
  a.s.T = T;
  a.s.t0 = t0;
  a.s.ret_caches = retrieval && T > 0 ? g.B * lv.n_ret : 0;
  a.s.ret_tile0 = t0 / kStageRows;
  a.s.ret_tiles = static_cast<int>((t0 + T + kStageRows - 1) / kStageRows - a.s.ret_tile0);
  const int str_caches = nq > 0 ? g.B * lv.n_str : 0;
  a.s.sink_rows = stage_sink_rows(g.S);
  const int window_rows = stage_window_rows(g.R);
  a.s.str_tiles = str_caches ? (a.s.sink_rows + window_rows) / kStageRows + (nq + kStageRows - 1) / kStageRows : 0;
  a.s.u_end = t0 + q0 + nq;
  a.s.p0 = t0 + q0 - window_rows;
  const int tiles = a.s.ret_caches && a.s.ret_tiles > a.s.str_tiles ? a.s.ret_tiles : a.s.str_tiles;
  if (a.s.ret_caches + str_caches == 0 || tiles == 0) return hipSuccess;
  launch(k_chunk_tiles<false>, dim3(static_cast<unsigned>(tiles), static_cast<unsigned>(a.s.ret_caches + str_caches)),
         dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_stream_cache_update(const Geom& g, const LayerView& lv, const void* k, const void* v, int T,
                                      int64_t t0, hipStream_t st) {
  const int caches = g.B * lv.n_str;
  if (caches == 0 || T <= 0) return hipSuccess;
  ChunkTileArgs a = {};
  a.g = g;
  a.lv = lv;
  a.s = update_scalars(g, lv, k, v, T, t0);
  launch(k_chunk_tiles<true>, dim3(static_cast<unsigned>(a.s.str_tiles), static_cast<unsigned>(caches)), dim3(256), 0,
         st, a);
  return hipGetLastError();
}

hipError_t launch_prefill_stream_mfma(const Geom& g, const LayerView& lv, const CacheRegion& stage, const void* q,
                                      void* out, int T, int64_t t0, int q0, int nq, hipStream_t st) {
  // (streaming heads only: short blocks, for which 4-wavefront workgroups, two per CU,
  // measured faster than the shared tiles of 8)
  PrefillArgs a = prefill_args(g, lv, stage, q, out, T, t0);
  a.str = streaming_grid(g, 4, lv, q0, nq);
  a.stage_p0 = t0 + q0 - stage_window_rows(g.R);
  if (a.str.blocks == 0) return hipSuccess;
  launch(k_prefill_mfma<4>, dim3(static_cast<unsigned>(a.str.blocks)), dim3(Shape<4>::kThreads),
         2 * (kKBytes + kVBytes), st, a);
  return hipGetLastError();
}

}  // namespace duo
