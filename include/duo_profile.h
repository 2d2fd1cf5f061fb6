/*
 * duo_profile.h -- per-kernel timing of a duo_handle (tracing).  Exported by
 * libduo_attn.so.
 *
 * While profiling is enabled on a handle, every kernel launch the handle makes is
 * bracketed by two hipEvents recorded on the stream of that launch, so the measured
 * interval is the kernel's own execution on that stream.  duo_profile_collect waits
 * for the recorded events, adds up elapsed milliseconds and launch counts per kernel
 * class, and clears the record.  Event objects are pooled by the handle (host-side
 * HIP resources; no device memory is allocated).  Recording adds one event pair per
 * launch on the stream.
 *
 * Errors: DUO_E_INVALID (NULL handle or output array), DUO_E_HIP (event failure).
 */
#ifndef DUO_PROFILE_H
#define DUO_PROFILE_H

#include <stdint.h>

#include "duo_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

#define DUO_KERNEL_APPEND             0  /* fused append / evict (and int4 quantise) */
#define DUO_KERNEL_PREFILL_RETRIEVAL  1  /* prefill attention: retrieval heads, and (MFMA path) the
                                                first 4096 streaming-head queries of a chunk */
#define DUO_KERNEL_PREFILL_STREAMING  2  /* sink + window prefill attention of further streaming-head
                                                queries (MFMA path, chunks over 4096 tokens) */
#define DUO_KERNEL_DECODE             3  /* split-K decode attention with merge, all heads */
#define DUO_KERNEL_PREFILL_STAGE      4  /* prefill chunk into retrieval caches + streaming staging */
#define DUO_KERNEL_QKV_ROPE           5  /* duo_qkv_rope_w8 (thread profiler) */
#define DUO_KERNEL_LINEAR             6  /* duo_linear_w8 (thread profiler) */
#define DUO_KERNEL_CLASSES            7

/* on != 0 starts recording, on == 0 stops (recorded events stay until collected). */
int duo_profile_enable(duo_handle* h, int32_t on);

/* total_ms[DUO_KERNEL_CLASSES], launches[DUO_KERNEL_CLASSES]: filled with the sums
 * since the last collect.  Synchronises on the recorded events. */
int duo_profile_collect(duo_handle* h, double* total_ms, int64_t* launches);

/* The same for the calls that take no handle (duo_linear.h), per host thread: while on,
 * their launches from the calling thread are stamped; collect as above (only the
 * classes of those calls are non-zero).  Errors: DUO_E_INVALID (NULL output array),
 * DUO_E_HIP. */
int duo_profile_thread_enable(int32_t on);
int duo_profile_thread_collect(double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* DUO_PROFILE_H */
