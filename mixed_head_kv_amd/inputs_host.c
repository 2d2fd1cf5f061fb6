/* Host twin of the seeded input generator in inputs.py (same definition, bit for bit),
 * for producing multi-gigabyte K/V histories quickly on the host (tests, the bench's
 * CPU baseline).  SplitMix64 (Steele, Lea and Flood, "Fast Splittable Pseudorandom
 * Number Generators", OOPSLA 2014) as a counter generator: key = mix64((seed << 32) |
 * stream), word n = mix64(key + (n + 1) * GAMMA); a value is the sum S of the word's four
 * 16-bit fields, x = fp32(S - 131070) * fp32(sqrt(3) / 65536), then bf16 (nearest even)
 * when asked.  Holds no attention arithmetic.  Built by mixed_head_kv_amd/build.py with
 * gcc (OpenMP); inputs.py falls back to NumPy when the library is absent. */
#include <stdint.h>
#include <string.h>

static const uint64_t GAMMA = 0x9E3779B97F4A7C15ull;

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline float value_f32(uint64_t key, uint64_t counter, float scale) {
  const uint64_t w = mix64(key + (counter + 1) * GAMMA);
  const int64_t s = (int64_t)((w & 0xFFFF) + ((w >> 16) & 0xFFFF) + ((w >> 32) & 0xFFFF) + (w >> 48));
  return (float)(s - 131070) * scale;
}

static inline uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

/* Rows of one head at the given positions: out[i * D + d] is the value of counter
 * (pos[i] * H + head) * D + d (fp32 into out_f32, or bf16 bits into out_bf16, whichever
 * is non-null).  `scale` is fp32(sqrt(3) / 65536) as inputs.py computes it. */
void duo_inputs_head_rows(uint64_t seed, uint32_t stream, const int64_t* pos, int64_t n, int64_t head, int64_t H,
                          int64_t D, float scale, float* out_f32, uint16_t* out_bf16) {
  const uint64_t key = mix64((seed << 32) | stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const uint64_t c0 = ((uint64_t)pos[i] * (uint64_t)H + (uint64_t)head) * (uint64_t)D;
    for (int64_t d = 0; d < D; ++d) {
      const float x = value_f32(key, c0 + (uint64_t)d, scale);
      if (out_f32) out_f32[i * D + d] = x;
      if (out_bf16) out_bf16[i * D + d] = f32_to_bf16(x);
    }
  }
}

/* A contiguous counter range [c0, c0 + n). */
void duo_inputs_range(uint64_t seed, uint32_t stream, uint64_t c0, int64_t n, float scale, float* out_f32,
                      uint16_t* out_bf16) {
  const uint64_t key = mix64((seed << 32) | stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const float x = value_f32(key, c0 + (uint64_t)i, scale);
    if (out_f32) out_f32[i] = x;
    if (out_bf16) out_bf16[i] = f32_to_bf16(x);
  }
}
