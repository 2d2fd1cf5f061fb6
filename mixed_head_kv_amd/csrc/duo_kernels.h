// Launchers of the HIP kernels (internal to libduo_attn.so).  Each returns the
// hipError_t of its launch; arguments are validated by the caller (duo_attn.cpp).
#pragma once

#include <hip/hip_ext.h>

#include <utility>

#include "duo_common.h"

namespace duo {

// Kernel timing.  When a caller of the library's API profiles, it parks a start/stop
// event pair here just before the launcher runs; the launcher hands them to
// hipExtLaunchKernelGGL, which stamps them when the dispatch itself begins and ends
// (no marker packets of their own, so the timed interval is the kernel's execution and
// the stream gets no extra commands).  One pair serves one launch.
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
LaunchEvents& launch_events();  // per host thread

// Launch errors are left for the caller's hipGetLastError().
template <typename... KArgs, typename... Args>
void launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t lds, hipStream_t st, Args&&... args) {
  LaunchEvents& ev = launch_events();
  const LaunchEvents use = ev;  // null events: a plain launch
  ev = LaunchEvents{};
  hipExtLaunchKernelGGL(kernel, grid, block, lds, st, use.start, use.stop, 0u, std::forward<Args>(args)...);
}

// Fused append/evict of T tokens at positions [t0, t0 + T) into every cache of the
// layer: retrieval heads store every row, streaming heads keep sinks and the last
// `recent` positions.  `which`: 1 = retrieval caches only, 2 = streaming only, 3 = both.
hipError_t launch_append(const Geom& g, const LayerView& lv, const void* k, const void* v, int T,
                         int64_t t0, int which, hipStream_t st);

// Straightforward causal prefill attention on the vector ALUs (any dtype, D 64/128).
// Keys before t0 come from the caches, keys from t0 on from the chunk inputs.
hipError_t launch_prefill_valu(const Geom& g, const LayerView& lv, const void* q, const void* k,
                               const void* v, void* out, int T, int64_t t0, hipStream_t st);

// Prefill attention on bf16 MFMA (D = 128), one launch: the retrieval heads (causal,
// keys [0, t0 + T) read from the retrieval caches, so the chunk must have been appended
// there first) and the streaming-head queries of chunk rows [0, nq_streaming) over the
// keys staged by launch_chunk_tiles.  When the retrieval blocks alone are few (under
// eight wavefronts per CU) each block's key range is split over two workgroups that
// merge through `scratch` (fp32 partials, coherent) and `counters` (kPrefillCounters
// ints, zero between calls).
// upd_k / upd_v != null: the streaming caches' update with the chunk (K/V inputs) runs
// in the same launch (valid when no later staging reads the caches as they stood).
// out_lambda != null (every KV head a retrieval head): the second grid computes every
// head's sink + window attention over the retrieval caches for all T queries and writes
// it there, beside the full causal output in `out`.
// What a prefill launch was (filled when `info` is given): workgroup shape and grid.
struct PrefillLaunchInfo {
  int waves, pack, qrows, nsplit;
  int ret_blocks, str_blocks, upd_blocks;
};
hipError_t launch_prefill_mfma(const Geom& g, const LayerView& lv, const CacheRegion& stage, const void* q, void* out,
                               int T, int64_t t0, int nq_streaming, float* scratch, int64_t scratch_floats,
                               int* counters, int num_cu, hipStream_t st, void* out_lambda = nullptr,
                               const void* upd_k = nullptr, const void* upd_v = nullptr,
                               PrefillLaunchInfo* info = nullptr);

// Chunk keys into the layouts the MFMA prefill loads directly (bf16, D = 128), one
// launch: with `retrieval`, rows [t0, t0 + T) of every retrieval cache (the append);
// with nq > 0, the keys that the streaming-head queries of chunk rows [q0, q0 + nq) may
// see (sinks, and the window from R - 1 positions before q0 on), from the chunk inputs
// and from the streaming caches as they stood before the chunk, into `stage`.  `stage`
// holds at least stage_sink_rows(S) + stage_window_rows(R) + nq rounded up to a multiple
// of 64 rows per streaming cache, in the cache layout.
hipError_t launch_chunk_tiles(const Geom& g, const LayerView& lv, const CacheRegion& stage, const void* k,
                              const void* v, int T, int64_t t0, bool retrieval, int q0, int nq, hipStream_t st);

// The chunk's tokens into the streaming (constant-length) caches, bf16 with D = 128:
// sinks and the last R positions, the rest kept; the same result as launch_append with
// which = 2, through the coalesced tile writer.
hipError_t launch_stream_cache_update(const Geom& g, const LayerView& lv, const void* k, const void* v, int T,
                                      int64_t t0, hipStream_t st);

// Streaming-head (sink + window) prefill on bf16 MFMA (D = 128) of the queries in chunk
// rows [q0, q0 + nq) (at most kStageTokens), over the keys staged by launch_chunk_tiles;
// for the queries after the first kStageTokens of a chunk.
// Wavefronts per MFMA prefill workgroup for a layer shape (4 or 8).
int prefill_waves(const Geom& g);

hipError_t launch_prefill_stream_mfma(const Geom& g, const LayerView& lv, const CacheRegion& stage, const void* q,
                                      void* out, int T, int64_t t0, int q0, int nq, hipStream_t st);

// Most sequences one decode launch takes when their lengths differ.
constexpr int kMaxVarlen = 32;

struct DecodePlan {
  int64_t t;          // query position (the largest one when varlen is set)
  // varlen != 0: the sequences' query positions differ and sequence b's is t_seq[b]
  // (batch <= kMaxVarlen); the split sizes are planned for t.
  int varlen;
  int64_t t_seq[kMaxVarlen];
  int chunk_r;        // keys per split, retrieval heads
  int nsplit_r;
  int chunk_s;        // keys per split, streaming heads
  int nsplit_s;
  float* partials;    // [B * Hq * max_splits * (D + 2)]
  int max_splits;     // partial slots per query head (at least nsplit_r and nsplit_s)
  int* counters;      // [B * Hkv] arrival counters, zero between calls
  // Fused append (MFMA decode): K/V of the token at position t ([B, Hkv, D]), or null
  // when the token is already in the caches.  It lands in retrieval row t and in
  // streaming slot `new_slot` (with varlen: row t_seq[b] and that position's slot).
  const uint16_t* k_new;
  const uint16_t* v_new;
  int64_t new_slot;
};

// Split-K decode attention (all heads of the layer, one launch, merge by the last
// arriving workgroup of each KV head).  VALU version, any dtype / format.
hipError_t launch_decode_valu(const Geom& g, const LayerView& lv, const DecodePlan& p, const void* q,
                              void* out, hipStream_t st);

// Same on MFMA for bf16 and int4 caches with D = 128.
hipError_t launch_decode_mfma(const Geom& g, const LayerView& lv, const DecodePlan& p, const void* q,
                              void* out, hipStream_t st);

// 8-bit-weight linear layer y = x * (c * s)^T (bf16 x [M, K], int8 c [N, K], fp32 s [N]),
// output channels [0, n1) to y0, [n1, n2) to y1, [n2, N) to y2 (each row-major with its
// own row length); channels [0, rope_end) are rotated per 128-channel head with the
// position pos[m] of row m.  K % 128 == 0, N % 256 == 0, M >= 1.
struct W8Args {
  const uint16_t* x;
  const int8_t* w;
  const float* scale;
  const int64_t* pos;  // [M] device, when rope_end > 0
  uint16_t* y0;
  uint16_t* y1;
  uint16_t* y2;
  int64_t M;
  int K, N, n1, n2, rope_end;
  double theta_pow[6];  // base^(-2^j / 64), j = 0..5: theta_d is the product over d's bits
};
hipError_t launch_w8(const W8Args& a, hipStream_t st);

// Inspection: stored vectors of positions [pos0, pos0 + n) of one cache, as fp32
// (dequantised for int4) or as raw int4 codes + (scale, zero).
hipError_t launch_read(const Geom& g, const CacheRegion& c, int64_t cache, bool streaming, int64_t pos0,
                       int n, int which, float* out, hipStream_t st);
hipError_t launch_read_int4(const Geom& g, const CacheRegion& c, int64_t cache, bool streaming, int64_t pos0,
                            int n, int which, uint8_t* codes, uint16_t* meta, hipStream_t st);
hipError_t launch_zero_i32(int* p, int64_t n, hipStream_t st);
// Clears n_bytes (a multiple of 16, 16-byte aligned) with a fill kernel.
hipError_t launch_zero_bytes(void* p, uint64_t n_bytes, hipStream_t st);
// Fills the n guard bands (DUO_GUARD_BYTES each) at byte offsets `offsets` (host array)
// from `base` with the 32-bit `word`.
hipError_t launch_guard_fill(char* base, const uint64_t* offsets, int n, uint32_t word, hipStream_t st);
hipError_t launch_synth(void* out, int dtype, uint64_t seed, uint32_t stream, uint64_t c0, uint64_t n,
                        hipStream_t st);

}  // namespace duo
