/*
 * duo_attn.h -- C ABI of the mixed-head (retrieval / streaming) KV attention library
 * for AMD Instinct MI355X (gfx950).  Library: libduo_attn.so.
 *
 * What the library computes
 * -------------------------
 * Each transformer layer's KV heads are split into two kinds.  A retrieval head keeps
 * a full KV cache and its queries attend causally to every token; a streaming head
 * keeps a constant-length cache holding only the attention sinks and the most recent
 * tokens, and its queries attend to exactly those.  Sources: hotpaper.ai page
 * "DuoAttention: Efficient Long-Context LLM Inference with Retrieval and Streaming
 * Heads", abstract (full KV cache for retrieval heads, light constant-length cache of
 * recent tokens and sinks for streaming heads; applies to both decoding and
 * pre-filling; MHA and GQA models) and its technical-approach section (two caches per
 * layer); "What is DuoAttention" (nav.superapi.store), Technical principles.
 *
 * For a query at absolute position i (0-based) the visible keys are
 *   retrieval head: { j : j <= i }
 *   streaming head: { j : j <= i and (j < sink or i - j < recent) }
 * scores are scale * <q_i, k_j> (scale = 1/sqrt(head_dim) unless set), softmax over
 * the visible set, output sum_j p_ij v_j; accumulation in fp32, output in the I/O
 * dtype rounded to nearest even.  Sinks are positions 0..sink-1; the recent window
 * includes the current token, so a streaming cache holds exactly sink + recent tokens.
 * Query head h uses KV head h / (n_q_heads / n_kv_heads) (MHA when equal, GQA
 * otherwise) and takes that KV head's label.
 *
 * Conventions (all entry points)
 * ------------------------------
 * - Pointers named d_* or documented as device pointers are HIP device memory owned
 *   by the caller.  The library never allocates device memory: the caller provides
 *   one workspace (size from duo_kv_bytes) that holds every cache, table and scratch
 *   buffer.  The library owns only the small host-side handle.
 * - Work is enqueued on the caller's stream (hipStream_t passed as void*, NULL = the
 *   default stream) and no call synchronises.  Buffers must stay valid until the
 *   stream has run the work.  Calls on one handle must be ordered (same stream, or
 *   the caller orders the streams): they share the workspace's scratch region.
 * - Every call validates all arguments before enqueuing anything; a call that
 *   returns an error has changed no state.  Device pointers must be 16-byte aligned.
 * - Return codes: DUO_OK, or a negative DUO_E_* code with a message available from
 *   duo_last_error() (thread-local).
 * - A handle is not thread-safe.
 * - Fault injection, for tests of error handling: when the environment variable
 *   DUO_FAULT_INJECT holds "all" or a comma-separated list of entry-point names
 *   (e.g. "duo_decode,duo_kv_append"), each named call of duo_kv_init, duo_kv_attach,
 *   duo_prefill, duo_prefill_seq, duo_prefill_dual, duo_kv_append, duo_kv_append_seq,
 *   duo_decode, duo_decode_static, duo_kv_read and duo_kv_read_int4 returns DUO_E_HIP after its
 *   argument checks, before any HIP call and without changing any state.  The
 *   variable is read at every call; unset or empty, nothing changes.
 * - Launch log, for debugging: with the environment variable DUO_LOG set (non-empty, not
 *   "0"), duo_kv_init, duo_kv_append, duo_prefill (bf16 head_dim 128 caches) and the
 *   decode calls write one line each to stderr with their launch parameters (workspace
 *   size; workgroup shape, splits and grid sizes).  Nothing else changes.
 *
 * Tensor layouts (row-major, contiguous, batch B = cfg.batch):
 *   Q, O for prefill : [B, T, n_q_heads, head_dim]      (token-major, as a fused QKV
 *   K, V for prefill : [B, T, n_kv_heads, head_dim]      projection produces them)
 *   Q, O for decode  : [B, n_q_heads, head_dim]
 *   K, V for decode  : [B, n_kv_heads, head_dim]
 * Element type: float32 (DUO_DTYPE_F32) or bfloat16 (DUO_DTYPE_BF16), cfg.io_dtype.
 */
#ifndef DUO_ATTN_H
#define DUO_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define DUO_OK             0
#define DUO_E_INVALID     -1  /* null / misaligned pointer, value out of range        */
#define DUO_E_UNSUPPORTED -2  /* valid request the library does not implement         */
#define DUO_E_CAPACITY    -3  /* length + tokens > max_context, or workspace too small */
#define DUO_E_STATE       -4  /* call not allowed in the handle's current state        */
#define DUO_E_HIP         -5  /* a HIP runtime call or kernel launch failed            */

/* I/O element types. */
#define DUO_DTYPE_F32  0
#define DUO_DTYPE_BF16 1

/* KV cache formats. */
#define DUO_KV_SAME_AS_IO 0  /* caches hold K/V in the I/O type, bit-exact copies   */
#define DUO_KV_INT4_G128  1  /* 4-bit codes, one group per 128-value vector, fp16
                                scale and zero (bf16 I/O, head_dim 128 only).  Format
                                of one vector x: s = fp16(fp32(fp32(max-min)/15)),
                                z = fp16(min), q = clamp(rint_even(fp32(fp32(x-z)/s)),
                                0, 15) (q = 0 when s == 0); dequantised value
                                fp32(q*s + z).  The pages only name a 4-bit KV cache
                                (hotpaper.ai page, abstract and main results). */

/* Limits of the library. */
#define DUO_MAX_KV_HEADS 64
#define DUO_MAX_GROUP    16   /* n_q_heads / n_kv_heads */
#define DUO_MAX_WINDOW   (1 << 28)  /* largest sink, and largest recent */

typedef struct duo_config {
  int32_t n_layers;     /* >= 1 */
  int32_t batch;        /* >= 1; sequences of a batch share one length and one mask */
  int32_t n_q_heads;    /* multiple of n_kv_heads */
  int32_t n_kv_heads;   /* 1..DUO_MAX_KV_HEADS */
  int32_t head_dim;     /* 64 or 128 */
  int32_t sink;         /* attention-sink tokens, 0..DUO_MAX_WINDOW */
  int32_t recent;       /* recent-window tokens including the current one,
                           1..DUO_MAX_WINDOW (larger: DUO_E_UNSUPPORTED) */
  int32_t io_dtype;     /* DUO_DTYPE_* */
  int32_t kv_format;    /* DUO_KV_* */
  int32_t reserved;     /* must be 0 */
  int64_t max_context;  /* tokens per sequence the retrieval caches can hold, >= 1 */
  float scale;          /* softmax scale; 0 means 1/sqrt(head_dim) */
  /* Host pointer, [n_layers * n_kv_heads] bytes, 1 = retrieval head, 0 = streaming
   * head (the per-head label that the method fixes before inference: hotpaper.ai
   * page, abstract; cn.bg3.co article, DuoAttention 的创新设计).  Copied at init. */
  const uint8_t* retrieval_mask;
} duo_config;

typedef struct duo_handle duo_handle;

/* Size in bytes of the device workspace duo_kv_init needs for cfg.  Returns
 * DUO_E_INVALID / DUO_E_UNSUPPORTED for a config init would reject. */
int duo_kv_bytes(const duo_config* cfg, uint64_t* out_bytes);

/* Create a handle over a caller-allocated device workspace of `bytes` bytes
 * (>= duo_kv_bytes, 256-byte aligned).  Regroups each layer's KV heads by their label
 * into a dense list of retrieval heads and a dense list of streaming heads, and lays
 * out one full cache per retrieval KV head and one constant-length (sink + recent
 * slots) cache per streaming KV head, per layer and sequence: the two kinds of KV cache
 * each layer keeps (hotpaper.ai page "DuoAttention: Efficient Long-Context LLM
 * Inference with Retrieval and Streaming Heads", abstract and technical-approach
 * section; cn.bg3.co article, DuoAttention 的创新设计).  Clears the workspace and fills
 * its guard bands (fill kernels on `stream`).  Every layer starts with length 0.  The workspace must not be
 * used by anything else while the handle lives.  Errors: DUO_E_INVALID (bad config,
 * null or misaligned workspace), DUO_E_UNSUPPORTED, DUO_E_CAPACITY (bytes too small),
 * DUO_E_HIP (the fill kernel failed to launch; no handle is returned). */
int duo_kv_init(const duo_config* cfg, void* d_workspace, uint64_t bytes, void* hip_stream,
                duo_handle** out);

/* Resume from a saved state: a handle over a workspace that holds what an earlier handle
 * with the same config left in it between calls (its bytes saved and copied back, or
 * the same memory), with the tokens held per layer and sequence given in the host array
 * lengths[n_layers * batch] (layer-major; duo_kv_length_seq of the earlier handle).
 * Nothing in the workspace is cleared or written (the first handle on a device still
 * sets up that device's static scratch once).  Resuming this way and re-creating the
 * state with duo_kv_init plus duo_kv_append of the same tokens give the same caches, so
 * the same outputs.  Errors: as duo_kv_init, and DUO_E_INVALID for a null lengths array
 * or a length outside 0..max_context. */
int duo_kv_attach(const duo_config* cfg, void* d_workspace, uint64_t bytes, const int64_t* lengths,
                  duo_handle** out);

/* Workspace guard bands, for checks that no kernel writes outside its region: every
 * region of the workspace (each cache, the split scratch, the counters, the staging
 * buffers) is followed by DUO_GUARD_BYTES bytes that duo_kv_init fills with the 32-bit
 * word DUO_GUARD_WORD (little-endian, repeated) and that nothing else writes.
 * Writes the byte offsets (from the workspace start) of the first `max` bands into the
 * host array `offsets` and the number of bands into *n (the full count, also when max
 * is smaller).  A caller compares the bands with the pattern after its work has run.
 * Errors: DUO_E_INVALID (null handle or n, max < 0, null offsets with max > 0). */
#define DUO_GUARD_BYTES 256u
#define DUO_GUARD_WORD 0xD0A5C3E1u
int duo_kv_guard_bands(const duo_handle* h, uint64_t* offsets, int32_t max, int32_t* n);

/* Causal attention of n_tokens new tokens of `layer` (positions len .. len+T-1) and
 * append of their K/V (pre-filling; a prompt may be split into chunks, one call each,
 * and the result equals one unchunked call).  The method pre-fills retrieval heads
 * with full attention and streaming heads over the sinks and recent tokens only
 * (hotpaper.ai page "DuoAttention: Efficient Long-Context LLM Inference with Retrieval
 * and Streaming Heads", abstract: lower pre-filling latency; cn.bg3.co article,
 * 研究背景: full-attention pre-filling cost grows quadratically with the context).  q, k, v, out: device pointers in the
 * prefill layouts above.  Retrieval heads attend to every earlier token of the
 * sequence; streaming heads to the sinks and the recent window, read from their
 * constant-length cache as it stood before the call plus the chunk itself.  After the
 * call the layer's length is len + T.  int4 caches: DUO_E_UNSUPPORTED (decode-only
 * format of the library).  Every sequence of the batch must hold the same length len
 * (else DUO_E_STATE; duo_prefill_seq fills one sequence).  Errors: DUO_E_INVALID
 * (T <= 0, bad layer, null or misaligned pointer), DUO_E_CAPACITY
 * (len + T > max_context). */
int duo_prefill(duo_handle* h, int32_t layer, const void* q, const void* k, const void* v,
                int32_t n_tokens, void* out, void* hip_stream);

/* Pre-filling for head identification: for every query head, both its full causal
 * attention (out_full) and its streaming attention, the sinks plus the recent window
 * (out_streaming), over the same keys.  The method labels heads by an optimization
 * that compares a head's full-attention and streaming-attention behaviour
 * (hotpaper.ai page "DuoAttention: Efficient Long-Context LLM Inference with Retrieval
 * and Streaming Heads", abstract: optimization-based identification of the retrieval
 * heads with synthetic data); the pages give neither its objective nor how the two
 * outputs are mixed, so this call returns the two outputs and nothing more.  The layer
 * must hold full caches for every head (its retrieval_mask entries all 1; else
 * DUO_E_STATE) and use bf16 I/O, head_dim 128 and bf16 caches (else
 * DUO_E_UNSUPPORTED).  Layouts and chunking as duo_prefill; the chunk's K/V are
 * appended; out_full and out_streaming are [B, T, Hq, D]. */
int duo_prefill_dual(duo_handle* h, int32_t layer, const void* q, const void* k, const void* v,
                     int32_t n_tokens, void* out_full, void* out_streaming, void* hip_stream);

/* Append n_tokens K/V rows (prefill layout, no attention) at positions len .. len+T-1:
 * retrieval heads store every row, streaming heads keep the sinks and the last
 * `recent` tokens (evicting older ones); int4 caches quantise on the way in.  The two
 * caches are the method's full cache for retrieval heads and its constant-length cache
 * of sinks and recent tokens for streaming heads (hotpaper.ai page, abstract and
 * technical-approach section); the 4-bit format is the one DUO_KV_INT4_G128 states
 * (same page, abstract and main results: combined with a 4-bit KV cache).  Used to
 * fill long contexts.  Errors as duo_prefill. */
int duo_kv_append(duo_handle* h, int32_t layer, const void* k, const void* v, int32_t n_tokens,
                  void* hip_stream);

/* One decoding step of `layer`: for every sequence b, appends its k_new / v_new row
 * (decode layout) at position t_b = len_b, the sequence's own length, then its query
 * (decode layout) at position t_b attends to the visible keys (so the new token sees
 * itself), writing out.  Retrieval heads attend over the full cache and streaming
 * heads over their constant-length cache of sinks and recent tokens (hotpaper.ai page
 * "DuoAttention: Efficient Long-Context LLM Inference with Retrieval and Streaming
 * Heads", abstract: decoding speed-up; cn.bg3.co article, 研究背景: decoding cost of
 * full attention grows linearly with the context).  If k_new and v_new are both NULL nothing is appended and the
 * queries attend at t_b = len_b - 1 (their K/V were appended earlier, e.g. by
 * duo_kv_append).  The lengths may differ between sequences (filled with the
 * per-sequence calls below) when batch <= 32.  Retrieval heads use split-K flash
 * decoding over the full cache with a log-sum-exp merge; streaming heads read their
 * sink + recent slots.  Errors: DUO_E_INVALID, DUO_E_CAPACITY (append past
 * max_context), DUO_E_STATE (NULL k_new/v_new with an empty sequence, or only one of
 * them NULL), DUO_E_UNSUPPORTED (lengths that differ with batch > 32). */
int duo_decode(duo_handle* h, int32_t layer, const void* q, const void* k_new, const void* v_new,
               void* out, void* hip_stream);

/* ---- Decoding without any allocation -------------------------------------------- */
/* For callers that cannot allocate device memory at all (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): duo_decode with its split-K
 * partials and arrival counters in a static device array that the library holds,
 * DUO_STATIC_SCRATCH_BYTES per GPU (each GPU the library runs on keeps its copy until
 * the process ends), instead of the handle's workspace.  Same arguments, semantics and
 * results as duo_decode; it calls no hipMalloc, hipFree or allocating routine.  The
 * array's address is set up at the first duo_kv_init on each device (with that device
 * current); the handle uses its init device's array.  Every call on one GPU, from any
 * handle, shares that array: calls that overlap on one GPU (different streams not
 * ordered by the caller) race and give wrong results.  The kernels leave the arrival
 * counters at zero after every call.  Errors: those of duo_decode; DUO_E_CAPACITY when
 * the batch's arrival counters (batch * n_kv_heads above 16384) or one split of every
 * query head (batch * n_q_heads * (head_dim + 2) * 4 bytes) do not fit; DUO_E_UNSUPPORTED
 * when the context needs more splits than fit (the split count shrinks as
 * batch * n_q_heads grows); DUO_E_HIP when the array's set-up failed. */
#define DUO_STATIC_SCRATCH_BYTES (16u << 20)
int duo_decode_static(duo_handle* h, int32_t layer, const void* q, const void* k_new,
                      const void* v_new, void* out, void* hip_stream);

/* Tokens currently held for `layer` (the position of the next appended token) when
 * every sequence holds the same number; DUO_E_STATE when they differ. */
int duo_kv_length(const duo_handle* h, int32_t layer, int64_t* out_len);

/* ---- Per-sequence calls ------------------------------------------------------- */
/* The sequences of a batch are independent requests, each with its own caches and
 * length; decoding with the dual caches is what lets a GPU hold many long contexts
 * at once (hotpaper.ai page "DuoAttention: Efficient Long-Context LLM Inference with
 * Retrieval and Streaming Heads", abstract and main results: decoding memory and the
 * context one GPU serves).  These calls act on sequence `seq` (0 <= seq < batch)
 * alone, so that the sequences of a batch can hold different lengths; duo_decode then
 * serves them all in one step.  The pointers are one sequence's tensors: the layouts
 * above with B = 1.  Errors as the batch calls, and DUO_E_INVALID for seq out of
 * range.  Calls on one handle are ordered by the caller's stream. */

/* duo_prefill of sequence `seq` alone, at positions len_seq .. len_seq + T - 1. */
int duo_prefill_seq(duo_handle* h, int32_t layer, int32_t seq, const void* q, const void* k,
                    const void* v, int32_t n_tokens, void* out, void* hip_stream);

/* duo_kv_append of sequence `seq` alone (int4 caches quantise on the way in). */
int duo_kv_append_seq(duo_handle* h, int32_t layer, int32_t seq, const void* k, const void* v,
                      int32_t n_tokens, void* hip_stream);

/* Tokens currently held by sequence `seq` of `layer`. */
int duo_kv_length_seq(const duo_handle* h, int32_t layer, int32_t seq, int64_t* out_len);

/* Free the host handle (the workspace stays the caller's).  NULL is allowed. */
void duo_kv_free(duo_handle* h);

/* Message of the last error on this thread ("" if none). */
const char* duo_last_error(void);

/* ---- Inspection (used by tests to check the caches) --------------------------- */

/* Copy the stored K (which = 0) or V (which = 1) vectors of one sequence `b`, KV head
 * `kv_head` of `layer`, for absolute positions pos0 .. pos0+n-1, into d_out
 * ([n, head_dim] float32, device).  int4 caches are dequantised to fp32(q*s + z), the
 * format's value (bit-exact).  The int4 decode kernel does not form these values: it
 * feeds the codes to the matrix cores and applies s and z algebraically (per key, the
 * score is s * (sum over d of q_d * code_d) + z * sum over d of q_d, and likewise for
 * the value side), which equals attention over the dequantised values up to rounding
 * (held to the bf16 tolerance against the oracle over fp32(q*s + z)).  Positions must be held by sequence b: < len_b for
 * retrieval heads, visible from position len_b - 1 for streaming heads; otherwise
 * DUO_E_INVALID. */
int duo_kv_read(const duo_handle* h, int32_t layer, int32_t b, int32_t kv_head, int32_t which,
                int64_t pos0, int32_t n, float* d_out, void* hip_stream);

/* int4 caches only: copy the packed codes (n * 64 bytes, byte k = code 2k in the low
 * nibble and code 2k+1 in the high nibble, element order) and the fp16 scale and zero
 * bit patterns (n * 2 uint16: scale, zero) of the same vectors as duo_kv_read. */
int duo_kv_read_int4(const duo_handle* h, int32_t layer, int32_t b, int32_t kv_head, int32_t which,
                     int64_t pos0, int32_t n, uint8_t* d_codes, uint16_t* d_meta, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* DUO_ATTN_H */
