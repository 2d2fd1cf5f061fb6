// The linear layers on either side of the attention, with 8-bit weights, on gfx950:
//   y[m, n] = s[n] * sum_k x[m, k] * c[n, k]
// with bf16 activations x [M, K], int8 weight codes c [N, K] (output channel n, input k,
// row-major) and one fp32 scale s[n] per output channel, fp32 accumulation, bf16 output.
// The fused QKV projection also applies the rotary position encoding to its query and
// key heads in the epilogue (dims d and d + 64 of a 128-dim head rotated by
// pos * theta_d, theta_d = base^(-d / 64)) and writes Q, K and V to their own arrays.
//
// The source pages (hotpaper.ai page "DuoAttention: Efficient Long-Context LLM Inference
// with Retrieval and Streaming Heads", abstract and main results) combine the method
// with 8-bit weights and a 4-bit KV cache; they give no weight format and no position
// encoding, so the format here is weight-only int8 with per-channel scales and the
// encoding is the RoFormer rotation in the pairing the Llama models use.
//
// Two kernels:
//   k_w8_gemm  (M > 64, pre-filling): 256 x 256 output tiles, 8 wavefronts of 128 x 64,
//     v_mfma_f32_32x32x16_bf16.  x and code tiles of 64 inputs go HBM -> LDS with direct
//     loads, three stages deep; each wavefront converts the codes it needs to bf16 in
//     registers (one sign-extending byte convert per code, exact).  Its waits are L2
//     misses: each XCD's first touch of a 64-input slice of the x and code tiles.
//   k_w8_gemv  (M <= 64, decoding): HBM-bound on the codes.  A workgroup owns 16 output
//     channels; its 8 wavefronts split the inputs, each streaming 128-input slices of
//     the 16 rows with v_mfma_f32_16x16x32_bf16 (channels x tokens), then the partial
//     sums meet in LDS.
#include <cmath>

#include "duo_kernels.h"

namespace duo {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;

__device__ inline f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}
__device__ inline f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// Four int8 codes (one dword) to four bf16 values, exactly: each byte is sign-extended and
// converted to fp32 (one SDWA convert per byte), and the pairs keep their fp32 high
// halves (|c| <= 128 needs 8 significant bits, so the truncation is exact).
__device__ inline void codes_to_bf16(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const float f0 = static_cast<float>(static_cast<int8_t>(w & 0xff));
  const float f1 = static_cast<float>(static_cast<int8_t>((w >> 8) & 0xff));
  const float f2 = static_cast<float>(static_cast<int8_t>((w >> 16) & 0xff));
  const float f3 = static_cast<float>(static_cast<int8_t>(w >> 24));
  lo = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  hi = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
}

// The MFMA operand (8 bf16) of 8 codes held in two dwords.
__device__ inline u32x4 code_operand(uint32_t a, uint32_t b) {
  uint32_t r0, r1, r2, r3;
  codes_to_bf16(a, r0, r1);
  codes_to_bf16(b, r2, r3);
  return u32x4{r0, r1, r2, r3};
}

// cos and sin of the rotation of first-half dim d (theta_d = base^(-d / 64)) at
// position pos.  The angle is reduced in fp64 (pos up to millions of radians) to a
// fraction of a turn in [-1/2, 1/2], whose sine and cosine the hardware evaluates.
__device__ inline void rope_cs(int64_t pos, double turns_per_pos, float& c, float& s) {
  double t = static_cast<double>(pos) * turns_per_pos;
  t -= rint(t);
  const float f = static_cast<float>(t);
  c = __builtin_amdgcn_cosf(f);
  s = __builtin_amdgcn_sinf(f);
}

// theta_d / (2 pi) in turns per position, theta_d = base^(-d / 64) for d < 64: the
// product of the precomputed powers base^(-2^j / 64) over the set bits j of d (at most
// six fp64 products, relative error below 1e-15).
__device__ inline double rope_turns(int d, const double (&theta_pow)[6]) {
  double t = 0.15915494309189533577;
#pragma unroll
  for (int j = 0; j < 6; ++j)
    if ((d >> j) & 1) t *= theta_pow[j];
  return t;
}

// Output element (m, channel n) to its array: channels [0, n1) go to y0 (row length n1),
// [n1, n2) to y1 and [n2, N) to y2.
__device__ inline uint16_t* out_ptr(const W8Args& a, int64_t m, int n) {
  if (n < a.n1) return a.y0 + m * a.n1 + n;
  if (n < a.n2) return a.y1 + m * (a.n2 - a.n1) + (n - a.n1);
  return a.y2 + m * (a.N - a.n2) + (n - a.n2);
}

// ---- pre-filling: tiled GEMM ----------------------------------------------------------

// Output tile: (128 WM) rows x 256 channels, 4 WM wavefronts of 128 x 64, inputs in
// stages of 64.  x tile rows are 128 B and code tile rows 64 B; their 16-byte chunks are
// XOR-swizzled so that the 16 lanes one LDS read serves (16 consecutive rows, one
// logical chunk) hit 16 distinct 16-byte bank groups of the 256-byte bank window.
constexpr int kBN = 256, kBK = 64;
constexpr int kBBytes = kBN * kBK;

template <int WM>
struct GemmShape {
  static constexpr int kBM = 128 * WM;
  static constexpr int kThreads = 256 * WM;
  static constexpr int kABytes = kBM * kBK * 2;
  static constexpr int kStageBytes = kABytes + kBBytes;
  static constexpr int kADma = kABytes / 1024 / (4 * WM);  // direct loads per wavefront and stage
  static constexpr int kBDma = kBBytes / 1024 / (4 * WM);
};

__device__ inline int a_chunk(int row, int c) { return c ^ ((row >> 1) & 7); }  // x tile: 2 rows per window
__device__ inline int b_chunk(int row, int q) { return q ^ ((row >> 2) & 3); }  // code tile: 4 rows per window

// s_waitcnt with only the vector-memory count bounded (gfx9 encoding: vmcnt in bits 3:0
// and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Every wavefront's direct loads but its newest N have landed in LDS, and every
// wavefront has finished reading the stage before: the wait, then the barrier, with
// compiler fences so no memory access moves across.
template <int N>
__device__ inline void stage_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  wait_vmcnt<N>();
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Output tile of workgroup `id`.  Workgroups go to the 8 XCDs in turn, so XCD id % 8 runs
// ids congruent to it; when the column tiles split evenly, each XCD takes a band of
// column tiles and walks its rows band by band, so the workgroups resident on one XCD at
// a time share their x and code tiles in that XCD's L2.
__device__ inline void gemm_tile(int id, int tiles_m, int tiles_n, int& tm, int& tn) {
  if ((tiles_n & 7) == 0) {
    const int per = tiles_n >> 3;
    const int slot = id >> 3;
    tm = slot / per;
    tn = (id & 7) * per + slot % per;
  } else {
    tm = id / tiles_n;
    tn = id % tiles_n;
  }
}

// Stage S_ of the x and code tiles into LDS buffer BUF_: each wavefront's direct loads.
// (The kernel template is also instantiated for its host stub, where the load builtin
// takes a non-const pointer: a const source there silently drops the stub.)
#define W8_GEMM_DMA(S_, BUF_)                                                                                  \
  do {                                                                                                         \
    char* dA = lds + (BUF_) * Sh::kStageBytes;                                                                 \
    char* dB = dA + Sh::kABytes;                                                                               \
    _Pragma("unroll") for (int u = 0; u < Sh::kADma; ++u) __builtin_amdgcn_global_load_lds(                    \
        const_cast<uint16_t*>(asrc[u] + (S_) * kBK), (lds_void_ptr)(dA + (Sh::kADma * wave + u) * 1024), 16, 0, 0);                   \
    _Pragma("unroll") for (int u = 0; u < Sh::kBDma; ++u) __builtin_amdgcn_global_load_lds(                    \
        const_cast<int8_t*>(bsrc[u] + (S_) * kBK), (lds_void_ptr)(dB + (Sh::kBDma * wave + u) * 1024), 16, 0, 0);                   \
  } while (0)

// STAGES LDS buffers, loads STAGES - 1 stages ahead of the compute.
template <int WM, int STAGES>
__global__ void __launch_bounds__(512, 2) k_w8_gemm(W8Args a, int tiles_m, int tiles_n) {
  using Sh = GemmShape<WM>;
  constexpr int kAhead = STAGES - 1;
  constexpr int kDma = Sh::kADma + Sh::kBDma;
  extern __shared__ __attribute__((aligned(16))) char lds[];  // STAGES x (x tile, code tile)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int tm, tn;
  gemm_tile(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = int64_t(tm) * Sh::kBM;
  const int n0 = tn * kBN;
  const int K = a.K;

  // Direct-load sources.  x tile KB `inst` holds rows 8 inst + L/8, lane L writing
  // physical chunk L % 8; rows past M read row M - 1 (their outputs are not stored).  Code
  // tile KB `inst` holds rows 16 inst + L/4, physical chunk L % 4.
  const uint16_t* asrc[Sh::kADma];
  const int8_t* bsrc[Sh::kBDma];
#pragma unroll
  for (int u = 0; u < Sh::kADma; ++u) {
    const int row = 8 * (Sh::kADma * wave + u) + (lane >> 3);
    const int c = a_chunk(row, lane & 7);
    const int64_t grow = m0 + row < a.M ? m0 + row : a.M - 1;
    asrc[u] = a.x + grow * K + 8 * c;
  }
#pragma unroll
  for (int u = 0; u < Sh::kBDma; ++u) {
    const int row = 16 * (Sh::kBDma * wave + u) + (lane >> 2);
    bsrc[u] = a.w + int64_t(n0 + row) * K + 16 * b_chunk(row, lane & 3);
  }

  // Wavefront tile: rows 128 wm .. +127, channels of head wn / 2 (128 each): blocks
  // nb = 0, 1 at dims 32 (wn % 2) + 64 nb .. +31, so the two dims of every rotation pair
  // (d and d + 64) sit in the same lane and register.
  const int wm = wave >> 2, wn = wave & 3;
  const int col = lane & 31, kg = lane >> 5;
  int nrow[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) nrow[nb] = 128 * (wn >> 1) + 32 * (wn & 1) + 64 * nb + col;

  f32x16 acc[4][2];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x16{};

  // MFMA k-slot (kg, j) of k-step s is input 32 kg + 8 s + j of the 64-input stage, so a
  // lane's codes for the four steps are 32 contiguous bytes and its x values for step s
  // are logical chunk 4 kg + s of its row.
  const int ns = K / kBK;
#pragma unroll
  for (int s = 0; s < kAhead; ++s)
    if (s < ns) W8_GEMM_DMA(s, s);
  // stage 0 landed: every later stage issued so far may still be in flight
  if (ns >= kAhead)
    stage_barrier<kDma * (kAhead - 1)>();
  else
    stage_barrier<0>();
  for (int s = 0; s < ns; ++s) {
    const int buf = s % STAGES;
    if (s + kAhead < ns) W8_GEMM_DMA(s + kAhead, (s + kAhead) % STAGES);
    const char* A = lds + buf * Sh::kStageBytes;
    const char* B = A + Sh::kABytes;
    // every LDS read of the stage is issued up front, so their latency overlaps the
    // conversions and the first products
    u32x4 aop[4][4];
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int r = 128 * wm + 32 * mb + col;
        aop[st][mb] = *reinterpret_cast<const u32x4*>(A + r * 128 + a_chunk(r, 4 * kg + st) * 16);
      }
    u32x4 craw[2][2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int r = nrow[nb];
      craw[nb][0] = *reinterpret_cast<const u32x4*>(B + r * 64 + b_chunk(r, 2 * kg) * 16);
      craw[nb][1] = *reinterpret_cast<const u32x4*>(B + r * 64 + b_chunk(r, 2 * kg + 1) * 16);
    }
    __builtin_amdgcn_sched_barrier(0);  // (keeps the reads ahead of their uses)
    u32x4 bop[2][4];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      bop[nb][0] = code_operand(craw[nb][0][0], craw[nb][0][1]);
      bop[nb][1] = code_operand(craw[nb][0][2], craw[nb][0][3]);
      bop[nb][2] = code_operand(craw[nb][1][0], craw[nb][1][1]);
      bop[nb][3] = code_operand(craw[nb][1][2], craw[nb][1][3]);
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        acc[mb][0] = mfma32(aop[st][mb], bop[0][st], acc[mb][0]);
        acc[mb][1] = mfma32(aop[st][mb], bop[1][st], acc[mb][1]);
      }
    }
    // stage s + 1 landed (later stages may still be in flight) and stage s is free
    if (s + kAhead < ns)
      stage_barrier<kDma * (kAhead - 1)>();
    else
      stage_barrier<0>();
  }

  // Epilogue: lane holds channels n0 + nrow[0], n0 + nrow[1] and, in register e of row
  // block mb, row 128 wm + 32 mb + 8 (e / 4) + 4 kg + e % 4.
  const int ch0 = n0 + nrow[0], ch1 = n0 + nrow[1];
  const float s0 = a.scale[ch0], s1 = a.scale[ch1];
  const bool rotate = ch0 < a.rope_end;  // uniform: a wavefront's channels are one head
  const double tpp = rotate ? rope_turns(ch0 & 63, a.theta_pow) : 0.0;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t m = m0 + 128 * wm + 32 * mb + 8 * (e >> 2) + 4 * kg + (e & 3);
      if (m >= a.M) continue;
      float y0 = acc[mb][0][e] * s0, y1 = acc[mb][1][e] * s1;
      if (rotate) {
        float c, s;
        rope_cs(a.pos[m], tpp, c, s);
        const float r0 = y0 * c - y1 * s;
        y1 = y1 * c + y0 * s;
        y0 = r0;
      }
      *out_ptr(a, m, ch0) = f32_to_bf16(y0);
      *out_ptr(a, m, ch1) = f32_to_bf16(y1);
    }
  }
}

// ---- decoding: split-input GEMV on MFMA ---------------------------------------------

// Channel of MFMA row r (0..15) of workgroup wg.  With the rotation, the 8 workgroups of
// a head take dims 8 j .. 8 j + 7 (rows 0-7) and their partners 64 + 8 j .. (rows 8-15);
// a lane then holds the partner of its rows in lane ^ 32.
__device__ inline int gemv_channel(int wg, int r, bool rope_layout) {
  if (!rope_layout) return wg * 16 + r;
  const int j = wg & 7;
  return (wg >> 3) * 128 + (r < 8 ? 8 * j + r : 64 + 8 * j + (r - 8));
}

template <int TB>
__global__ void __launch_bounds__(512) k_w8_gemv(W8Args a) {
  constexpr int kSteps = TB == 1 ? 4 : 2;  // 128-input slices in flight per wavefront
  __shared__ f32x4 s_part[8][TB][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const bool rope_layout = a.rope_end > 0;
  const int ch = gemv_channel(blockIdx.x, r, rope_layout);
  // A operand: codes of channel ch; B operand: x of token 16 tb + r (zero past M).  MFMA
  // k-slot (g, j) of step s is input 32 g + 8 s + j of the 128-input slice.  (Reading
  // each row's 64-byte halves whole, or the codes with non-temporal loads, measured the
  // same.)
  const int8_t* wrow = a.w + int64_t(ch) * a.K + 32 * g;
  const uint16_t* xrow[TB];
  bool real[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int64_t t = 16 * tb + r;
    real[tb] = t < a.M;
    xrow[tb] = a.x + (real[tb] ? t : 0) * a.K + 32 * g;
  }
  const int nslices = a.K >> 7;
  f32x4 acc[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int s0 = wave; s0 < nslices; s0 += 8 * kSteps) {
    u32x4 wv[kSteps][2];
    u32x4 xv[kSteps][TB][4];
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      // slices past the end re-read slice s0 (valid memory) and are dropped below
      const int sl = s0 + 8 * u < nslices ? s0 + 8 * u : s0;
      const u32x4* wp = reinterpret_cast<const u32x4*>(wrow + sl * 128);
      wv[u][0] = wp[0];
      wv[u][1] = wp[1];
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const u32x4* xp = reinterpret_cast<const u32x4*>(xrow[tb] + sl * 128);
        xv[u][tb][0] = xp[0];
        xv[u][tb][1] = xp[1];
        xv[u][tb][2] = xp[2];
        xv[u][tb][3] = xp[3];
      }
    }
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      if (s0 + 8 * u >= nslices) break;  // uniform
      u32x4 aop[4];
      aop[0] = code_operand(wv[u][0][0], wv[u][0][1]);
      aop[1] = code_operand(wv[u][0][2], wv[u][0][3]);
      aop[2] = code_operand(wv[u][1][0], wv[u][1][1]);
      aop[3] = code_operand(wv[u][1][2], wv[u][1][3]);
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4 b = real[tb] ? xv[u][tb][q] : u32x4{0, 0, 0, 0};
          acc[tb] = mfma16(aop[q], b, acc[tb]);
        }
    }
  }

#pragma unroll
  for (int tb = 0; tb < TB; ++tb) s_part[wave][tb][lane] = acc[tb];
  __syncthreads();
  if (wave >= TB) return;
  f32x4 sum = s_part[0][wave][lane];
#pragma unroll
  for (int w = 1; w < 8; ++w) sum += s_part[w][wave][lane];

  // lane holds rows 4 g .. 4 g + 3 (channels) of token 16 wave + r
  const int c0 = gemv_channel(blockIdx.x, 4 * g, rope_layout);
  const f32x4 sc = *reinterpret_cast<const f32x4*>(a.scale + c0);
  float y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = sum[i] * sc[i];
  const int64_t m = 16 * wave + r;
  const bool rotate = c0 < a.rope_end;  // the head's 8 workgroups agree: uniform
  if (rotate) {
    float partner[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) partner[i] = __shfl_xor(y[i], 32);
    const int64_t pos = a.pos[m < a.M ? m : 0];
    const int d0 = (c0 & 127) & 63;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float c, s;
      rope_cs(pos, rope_turns(d0 + i, a.theta_pow), c, s);
      y[i] = g < 2 ? y[i] * c - partner[i] * s : y[i] * c + partner[i] * s;
    }
  }
  if (m < a.M) {
    uint16_t* o = out_ptr(a, m, c0);
    const uint32_t lo = uint32_t(f32_to_bf16(y[0])) | (uint32_t(f32_to_bf16(y[1])) << 16);
    const uint32_t hi = uint32_t(f32_to_bf16(y[2])) | (uint32_t(f32_to_bf16(y[3])) << 16);
    *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
  }
}

// (the kernel is named by the non-template caller: that is where its host stub is emitted)
template <int WM, int STAGES>
hipError_t launch_gemm(void (*kernel)(W8Args, int, int), const W8Args& a, hipStream_t st) {
  using Sh = GemmShape<WM>;
  constexpr int lds = STAGES * Sh::kStageBytes;
  const int tiles_m = static_cast<int>((a.M + Sh::kBM - 1) / Sh::kBM);
  const int tiles_n = a.N / kBN;
  // More than 64 KB of dynamic LDS needs the attribute; set once per process (a
  // thread-safe static), on the device current at the first call.
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  launch(kernel, dim3(static_cast<unsigned>(tiles_m * tiles_n)), dim3(Sh::kThreads), lds, st, a, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_w8(const W8Args& a, hipStream_t st) {
  if (a.M <= 64) {
    const dim3 grid(static_cast<unsigned>(a.N / 16));
    if (a.M <= 16)
      launch(k_w8_gemv<1>, grid, dim3(512), 0, st, a);
    else if (a.M <= 32)
      launch(k_w8_gemv<2>, grid, dim3(512), 0, st, a);
    else
      launch(k_w8_gemv<4>, grid, dim3(512), 0, st, a);
    return hipGetLastError();
  }
  // (measured on the 4096 x 4096 x 12288 projection: two or three stages, one or two
  // workgroups per CU and issue priorities all land within 5% of each other)
  return launch_gemm<2, 3>(k_w8_gemm<2, 3>, a, st);
}

}  // namespace duo
