// Mixed-head attention on the vector ALUs: any I/O dtype (fp32 / bf16), head_dim 64 or
// 128, and any cache format.  This is the fp32 path (the MFMA kernels are bf16) and
// the path for shapes the MFMA kernels do not cover.
//
// Visibility (hotpaper.ai page "DuoAttention: Efficient Long-Context LLM Inference
// with Retrieval and Streaming Heads", abstract; nav.superapi.store "What is
// DuoAttention", Technical principles): a retrieval head's query at position i sees
// every key j <= i; a streaming head's query sees the sinks j < S and the recent
// window i - j < R.  Softmax runs in the base-2 domain (scores pre-multiplied by
// scale * log2 e) with an online running max and sum.
#include "decode_common.h"

namespace duo {
namespace {

// One thread per query row (64 rows per workgroup), online softmax over the row's
// visible keys.  Keys before t0 come from the caches as they stood before the chunk;
// keys from t0 on come from the chunk's own K/V inputs.
template <int IO, int D>
__global__ void __launch_bounds__(64) k_prefill_valu(Geom g, LayerView lv, const void* __restrict__ q,
                                                     const void* __restrict__ kin, const void* __restrict__ vin,
                                                     void* __restrict__ out, int T, int64_t t0) {
  const int t = blockIdx.x * 64 + threadIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  if (t >= T) return;
  const int kvh = h / g.G;
  const bool retrieval = lv.kind[kvh] == kKindRetrieval;
  const int64_t cache = int64_t(b) * (retrieval ? lv.n_ret : lv.n_str) + lv.slot[kvh];
  const CacheRegion& c = retrieval ? lv.ret : lv.str;
  const int64_t i = t0 + t;

  float qv[D], o[D];
  const int64_t qrow = ((int64_t(b) * T + t) * g.Hq + h) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qv[d] = io_load<IO>(q, qrow + d) * g.scale_log2;
    o[d] = 0.0f;
  }
  float m = kNegInf, l = 0.0f;

  auto visit = [&](int64_t j) {
    float s = 0.0f;
    if (j >= t0) {
      const int64_t krow = ((int64_t(b) * T + (j - t0)) * g.Hkv + kvh) * D;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(qv[d], io_load<IO>(kin, krow + d), s);
    } else {
      const int64_t row = retrieval ? j : stream_slot(j, g.S, g.R);
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(qv[d], cache_k<IO, DUO_KV_SAME_AS_IO>(c, cache, row, D, d), s);
    }
    const float mn = fmaxf(m, s);
    const float alpha = exp2f(m - mn);
    const float p = exp2f(s - mn);
    l = l * alpha + p;
    m = mn;
    if (j >= t0) {
      const int64_t vrow = ((int64_t(b) * T + (j - t0)) * g.Hkv + kvh) * D;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(p, io_load<IO>(vin, vrow + d), o[d] * alpha);
    } else {
      const int64_t row = retrieval ? j : stream_slot(j, g.S, g.R);
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(p, cache_v<IO, DUO_KV_SAME_AS_IO>(c, cache, row, D, d), o[d] * alpha);
    }
  };

  if (retrieval) {
    for (int64_t j = 0; j <= i; ++j) visit(j);
  } else {
    const int64_t sink_end = i + 1 < g.S ? i + 1 : g.S;
    for (int64_t j = 0; j < sink_end; ++j) visit(j);
    int64_t w0 = i - g.R + 1;
    if (w0 < g.S) w0 = g.S;
    for (int64_t j = w0; j <= i; ++j) visit(j);
  }
  const float inv = 1.0f / l;
  const int64_t orow = ((int64_t(b) * T + t) * g.Hq + h) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) io_store<IO>(out, orow + d, o[d] * inv);
}

// One workgroup (256 threads) per (sequence, KV head, split).  Scores of 256 keys at a
// time for all G query heads; PV accumulation with thread (head, d) pairs.
template <int IO, int KVF, int D>
__global__ void __launch_bounds__(256) k_decode_valu(Geom g, LayerView lv, DecodePlan p, const void* __restrict__ q,
                                                     void* __restrict__ out) {
  constexpr int kKeys = 256;
  constexpr int kMaxPairs = DUO_MAX_GROUP * D / 256;
  __shared__ float qs[DUO_MAX_GROUP][D];
  __shared__ float sc[DUO_MAX_GROUP][kKeys];
  __shared__ float m_run[DUO_MAX_GROUP], l_run[DUO_MAX_GROUP], alpha[DUO_MAX_GROUP];

  const DecodeItem it = decode_item(g, lv, p, blockIdx.x);
  const int G = g.G;
  const CacheRegion& c = it.retrieval ? lv.ret : lv.str;
  for (int e = threadIdx.x; e < G * D; e += 256) {
    const int i = e / D, d = e % D;
    qs[i][d] = io_load<IO>(q, (int64_t(it.b) * g.Hq + it.kvh * G + i) * D + d) * g.scale_log2;
  }
  if (threadIdx.x < G) {
    m_run[threadIdx.x] = kNegInf;
    l_run[threadIdx.x] = 0.0f;
  }
  float acc[kMaxPairs];
#pragma unroll
  for (int a = 0; a < kMaxPairs; ++a) acc[a] = 0.0f;
  __syncthreads();

  for (int64_t base = it.key0; base < it.key1; base += kKeys) {
    const int64_t j = base + threadIdx.x;
    const bool valid = j < it.key1;
    for (int i = 0; i < G; ++i) sc[i][threadIdx.x] = kNegInf;
    if (valid) {
      for (int i = 0; i < G; ++i) {
        float s = 0.0f;
#pragma unroll 8
        for (int d = 0; d < D; ++d) s = fmaf(qs[i][d], cache_k<IO, KVF>(c, it.cache, j, D, d), s);
        sc[i][threadIdx.x] = s;
      }
    }
    __syncthreads();
    // per query head: block max, new running max, probabilities, running sum
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int i = wave; i < G; i += 4) {
      float mx = kNegInf;
      for (int k = lane; k < kKeys; k += 64) mx = fmaxf(mx, sc[i][k]);
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      const float mn = fmaxf(m_run[i], mx);
      float sum = 0.0f;
      for (int k = lane; k < kKeys; k += 64) {
        const float pk = exp2f(sc[i][k] - mn);
        sc[i][k] = pk;
        sum += pk;
      }
      for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
      if (lane == 0) {
        const float a = exp2f(m_run[i] - mn);
        alpha[i] = a;
        l_run[i] = l_run[i] * a + sum;
        m_run[i] = mn;
      }
    }
    __syncthreads();
    const int nk = static_cast<int>(it.key1 - base < kKeys ? it.key1 - base : kKeys);
#pragma unroll
    for (int a = 0; a < kMaxPairs; ++a) {
      const int e = threadIdx.x + a * 256;
      if (e < G * D) {
        const int i = e / D, d = e % D;
        float s = acc[a] * alpha[i];
        for (int k = 0; k < nk; ++k) s = fmaf(sc[i][k], cache_v<IO, KVF>(c, it.cache, base + k, D, d), s);
        acc[a] = s;
      }
    }
    __syncthreads();
  }

  if (it.nsplit == 1) {
#pragma unroll
    for (int a = 0; a < kMaxPairs; ++a) {
      const int e = threadIdx.x + a * 256;
      if (e < G * D) {
        const int i = e / D, d = e % D;
        io_store<IO>(out, (int64_t(it.b) * g.Hq + it.kvh * G + i) * D + d, acc[a] / l_run[i]);
      }
    }
    return;
  }
#pragma unroll
  for (int a = 0; a < kMaxPairs; ++a) {
    const int e = threadIdx.x + a * 256;
    if (e < G * D) {
      const int i = e / D, d = e % D;
      float* ps = partial_ptr(g, p, it.b, it.kvh * G + i, it.split);
      store_coherent(ps + 2 + d, acc[a]);
      if (d == 0) {
        store_coherent(ps, m_run[i]);
        store_coherent(ps + 1, l_run[i]);
      }
    }
  }
  if (last_arrival(p.counters + it.b * g.Hkv + it.kvh, it.nsplit)) merge_splits<IO>(g, p, it.b, it.kvh, it.nsplit, out);
}

}  // namespace

hipError_t launch_prefill_valu(const Geom& g, const LayerView& lv, const void* q, const void* k, const void* v,
                               void* out, int T, int64_t t0, hipStream_t st) {
  dim3 grid((T + 63) / 64, g.Hq, g.B);
  // (bf16 with head_dim 128 runs on the MFMA kernels only)
  if (g.io == DUO_DTYPE_F32) {
    if (g.D == 64)
      launch(k_prefill_valu<DUO_DTYPE_F32, 64>, grid, dim3(64), 0, st, g, lv, q, k, v, out, T, t0);
    else
      launch(k_prefill_valu<DUO_DTYPE_F32, 128>, grid, dim3(64), 0, st, g, lv, q, k, v, out, T, t0);
  } else if (g.D == 64) {
    launch(k_prefill_valu<DUO_DTYPE_BF16, 64>, grid, dim3(64), 0, st, g, lv, q, k, v, out, T, t0);
  } else {
    return hipErrorNotSupported;
  }
  return hipGetLastError();
}

hipError_t launch_decode_valu(const Geom& g, const LayerView& lv, const DecodePlan& p, const void* q, void* out,
                              hipStream_t st) {
  const int items = g.B * (lv.n_ret * p.nsplit_r + lv.n_str * p.nsplit_s);
  if (items == 0) return hipSuccess;
  dim3 grid(items);
#define DUO_DECODE_VALU(IO, KVF, D) \
  launch(k_decode_valu<IO, KVF, D>, grid, dim3(256), 0, st, g, lv, p, q, out)
  // (int4 caches and bf16 with head_dim 128 run on the MFMA kernels only)
  if (g.kvfmt == DUO_KV_INT4_G128) return hipErrorNotSupported;
  if (g.io == DUO_DTYPE_F32) {
    if (g.D == 64) DUO_DECODE_VALU(DUO_DTYPE_F32, DUO_KV_SAME_AS_IO, 64);
    else DUO_DECODE_VALU(DUO_DTYPE_F32, DUO_KV_SAME_AS_IO, 128);
  } else if (g.D == 64) {
    DUO_DECODE_VALU(DUO_DTYPE_BF16, DUO_KV_SAME_AS_IO, 64);
  } else {
    return hipErrorNotSupported;
  }
#undef DUO_DECODE_VALU
  return hipGetLastError();
}

}  // namespace duo
