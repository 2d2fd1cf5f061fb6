/*
 * duo_linear.h -- the linear layers on either side of the attention, with 8-bit
 * weights.  Exported by libduo_attn.so.
 *
 * The method runs with 8-bit weights and a 4-bit KV cache (hotpaper.ai page
 * "DuoAttention: Efficient Long-Context LLM Inference with Retrieval and Streaming
 * Heads", abstract and main results: Llama-3-8B decodes 3.3M tokens on one A100 that
 * way).  The pages give no weight format and no position encoding; these calls take
 * weight-only int8 quantization with one fp32 scale per output channel, and the rotary
 * position encoding (RoFormer, Su et al. 2021) in the "rotate half" pairing of the
 * Llama models, applied to query and key heads after the projection.
 *
 * Layouts (all row-major, device pointers, 16-byte aligned unless stated):
 *   x      [M, K]  bfloat16 activations (M tokens)
 *   w      [N, K]  int8 codes in [-127, 127], output channel n's K codes contiguous
 *   scale  [N]     float32, the weight of (n, k) is w[n, k] * scale[n]
 * The product is accumulated in fp32 and rounded once to bfloat16 (nearest even).
 * Constraints: K a positive multiple of 128 (<= 2^20), N a positive multiple of 256
 * (<= 2^20), 1 <= M <= 2^24; otherwise DUO_E_UNSUPPORTED.  M <= 64 (decoding) runs an
 * HBM-bound kernel that streams each code once; larger M (pre-filling) a tiled MFMA
 * kernel.  Calls run on `hip_stream`, allocate nothing and do not synchronise.
 * Errors: DUO_E_INVALID (NULL or misaligned pointer, bad argument), DUO_E_UNSUPPORTED
 * (shape outside the constraints), DUO_E_HIP (launch failure).
 */
#ifndef DUO_LINEAR_H
#define DUO_LINEAR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* y [M, N] bfloat16 = x * (w * scale)^T: the output projection after the attention
 * (x = the attention output [M, Hq * head_dim]), or any other such layer. */
int duo_linear_w8(const void* x, int64_t M, int32_t K, const int8_t* w, const float* scale, int32_t N,
                  void* y, void* hip_stream);

/* Fused QKV projection with the rotary encoding, for tokens x [M, hidden] (bfloat16)
 * at absolute positions positions[m] (device int64 [M], 8-byte aligned, >= 0).  The
 * weight's N = (n_q_heads + 2 n_kv_heads) * head_dim output channels are the query
 * heads, then the key heads, then the value heads, head_dim consecutive channels each.
 * Writes q [M, n_q_heads, head_dim], k and v [M, n_kv_heads, head_dim] (bfloat16, the
 * layouts duo_prefill and duo_decode take for a batch of sequences laid out token by
 * token).  In every query and key head, dims d and d + head_dim/2 (d < head_dim/2) are
 * rotated by the angle positions[m] * rope_base^(-2 d / head_dim):
 *   out[d] = y[d] cos a - y[d + h] sin a,  out[d + h] = y[d + h] cos a + y[d] sin a,
 * with the angle reduced in fp64.  head_dim must be 128; rope_base > 1 (Llama-2 uses
 * 10000, Llama-3 500000). */
int duo_qkv_rope_w8(const void* x, int64_t M, int32_t hidden, const int64_t* positions, const int8_t* w_qkv,
                    const float* scale, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                    float rope_base, void* q, void* k, void* v, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* DUO_LINEAR_H */
