// Split-K decode pieces shared by the VALU and MFMA decode kernels: the mapping of
// workgroups to (sequence, KV head, key range), the fp32 partial buffer, and the
// log-sum-exp merge run by the last workgroup to finish for each KV head.
#pragma once

#include "duo_kernels.h"

namespace duo {

constexpr float kNegInf = -__builtin_huge_valf();

struct DecodeItem {
  int b, kvh, split, nsplit;
  bool retrieval;
  int64_t t;                  // the sequence's query position
  int64_t cache, key0, key1;  // cache rows [key0, key1) of this split (empty: 0, 0)
};

// Workgroups are laid out retrieval splits first, then streaming splits, per sequence.
__device__ inline DecodeItem decode_item(const Geom& g, const LayerView& lv, const DecodePlan& p, int item) {
  DecodeItem it;
  const int per_b = lv.n_ret * p.nsplit_r + lv.n_str * p.nsplit_s;
  it.b = item / per_b;
  it.t = p.t;
  if (p.varlen) {
    // constant indices: the plan stays in the kernel-argument segment (an indexed read
    // of the by-value argument would copy it to scratch memory)
#pragma unroll
    for (int s = 0; s < kMaxVarlen; ++s)
      if (s == it.b) it.t = p.t_seq[s];
  }
  int r = item % per_b;
  int64_t nkeys;
  int chunk, idx;
  if (r < lv.n_ret * p.nsplit_r) {
    it.retrieval = true;
    idx = r / p.nsplit_r;
    it.split = r % p.nsplit_r;
    it.nsplit = p.nsplit_r;
    chunk = p.chunk_r;
    nkeys = it.t + 1;
    it.kvh = lv.ret_kv[idx];
    it.cache = int64_t(it.b) * lv.n_ret + idx;
  } else {
    r -= lv.n_ret * p.nsplit_r;
    it.retrieval = false;
    idx = r / p.nsplit_s;
    it.split = r % p.nsplit_s;
    it.nsplit = p.nsplit_s;
    chunk = p.chunk_s;
    nkeys = it.t + 1 < g.S + g.R ? it.t + 1 : g.S + g.R;  // valid slots are [0, nkeys)
    it.kvh = lv.str_kv[idx];
    it.cache = int64_t(it.b) * lv.n_str + idx;
  }
  it.key0 = int64_t(it.split) * chunk;
  it.key1 = it.key0 + chunk < nkeys ? it.key0 + chunk : nkeys;
  // a shorter sequence of a varlen batch leaves its last splits without keys: they
  // produce the empty partial (m = -inf, l = 0), which the merge weighs with zero
  if (it.key0 >= nkeys) it.key0 = it.key1 = 0;
  return it;
}

__device__ inline float* partial_ptr(const Geom& g, const DecodePlan& p, int b, int h, int split) {
  return p.partials + ((int64_t(b) * g.Hq + h) * p.max_splits + split) * (g.D + 2);
}

// Split partials cross workgroups (and XCDs, each with its own L2) inside one launch.
// They are written and read with device-coherent (agent-scope) accesses, which bypass
// the non-coherent L2 lines, so the handoff needs no L2 write-back or invalidate:
// writers wait for their coherent stores to complete before the counter increment, and
// the last workgroup to arrive reads every partial coherently.
__device__ inline void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge of the split partials of one KV head's G query heads: (m_s, l_s, o_s) in the
// base-2 domain; o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
template <int IO>
__device__ void merge_splits(const Geom& g, const DecodePlan& p, int b, int kvh, int nsplit, void* out) {
  const int pairs = g.G * g.D;
  for (int e = threadIdx.x; e < pairs; e += blockDim.x) {
    const int i = e / g.D, d = e % g.D;
    const int h = kvh * g.G + i;
    float M = kNegInf;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, load_coherent(partial_ptr(g, p, b, h, s)));
    float L = 0.0f, acc = 0.0f;
    for (int s = 0; s < nsplit; ++s) {
      const float* ps = partial_ptr(g, p, b, h, s);
      const float w = exp2f(load_coherent(ps) - M);
      L = fmaf(w, load_coherent(ps + 1), L);
      acc = fmaf(w, load_coherent(ps + 2 + d), acc);
    }
    io_store<IO>(out, (int64_t(b) * g.Hq + h) * g.D + d, acc / L);
  }
}

// Returns true in every thread of the workgroup that arrived last for (b, kvh), after
// which the coherent partials of all splits are visible to it.  Resets the counter for
// the next call.  Every thread's coherent partial stores must precede the call.
__device__ inline bool last_arrival(int* counter, int nsplit) {
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0);  // this wavefront's coherent stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == nsplit - 1;
    if (s_last) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return s_last;
}

}  // namespace duo
