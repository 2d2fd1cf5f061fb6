/*
 * duo_synth.h -- seeded synthetic input generation on the device (benchmark and test
 * harness; not part of the attention method).  Exported by libduo_attn.so.
 *
 * Fills d_out[i], i in [0, n), with the value of counter counter0 + i of stream
 * `stream` under `seed`, using the SplitMix64 counter generator (Steele, Lea and
 * Flood, OOPSLA 2014): key = mix64((seed << 32) | stream), word(c) = mix64(key +
 * (c + 1) * 0x9E3779B97F4A7C15); the value is (sum of the four 16-bit fields of the
 * word - 131070) converted to float32 and multiplied by float32(sqrt(3)/65536), then
 * rounded to nearest even into `dtype` (DUO_DTYPE_F32 or DUO_DTYPE_BF16), or, for
 * DUO_SYNTH_INT8, multiplied by 32 (exact) and rounded to the nearest even integer, an
 * int8 weight code in [-111, 111] (synthetic 8-bit weights).  The
 * host-side NumPy generator in mixed_head_kv_amd/inputs.py implements the same
 * definition, so any slice can be regenerated on the host bit for bit.
 *
 * d_out: device pointer, 16-byte aligned, n elements of `dtype` (1 byte each for
 * DUO_SYNTH_INT8).  Runs on the
 * caller's stream, does not synchronise.  Errors: DUO_E_INVALID (null/misaligned
 * pointer, unknown dtype), DUO_E_HIP (launch failure).
 */
#ifndef DUO_SYNTH_H
#define DUO_SYNTH_H

#include <stdint.h>

#define DUO_SYNTH_INT8 2  /* dtype value of duo_synth_fill: int8 weight codes */

#ifdef __cplusplus
extern "C" {
#endif

int duo_synth_fill(void* d_out, int32_t dtype, uint64_t seed, uint32_t stream, uint64_t counter0,
                   uint64_t n, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* DUO_SYNTH_H */
