// Host side of libduo_attn.so: argument validation, workspace layout, head regrouping,
// per-layer lengths and kernel launches.  The C ABI is declared in include/duo_attn.h.
//
// Head regrouping: the per-KV-head retrieval / streaming label (fixed before inference,
// hotpaper.ai page "DuoAttention: Efficient Long-Context LLM Inference with Retrieval
// and Streaming Heads", abstract; cn.bg3.co article, DuoAttention 的创新设计) splits
// each layer's KV heads into a dense list of retrieval heads and a dense list of
// streaming heads, so each kind launches as one batch of workgroups and owns one
// contiguous cache region.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/duo_attn.h"
#include "../../include/duo_profile.h"
#include "../../include/duo_synth.h"
#include "../../include/duo_linear.h"
#include "duo_kernels.h"

using duo::CacheRegion;
using duo::Geom;
using duo::LayerView;

// The static scratch of duo_decode_static (one copy per GPU; see setup_static_scratch).
static __device__ __align__(256) char scratch[DUO_STATIC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int ok() {
  g_last_error.clear();
  return DUO_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(DUO_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// DUO_LOG set (non-empty, not "0"): every compute call writes one line of its launch
// parameters to stderr.  Read at every call; changes nothing else.
bool log_enabled() {
  const char* e = std::getenv("DUO_LOG");
  return e && *e && std::strcmp(e, "0") != 0;
}

// DUO_FAULT_INJECT ("all" or a comma-separated list of entry-point names): the named
// call fails with DUO_E_HIP here, after its argument checks and before any HIP call or
// state change.
int injected_fault(const char* call) {
  const char* e = std::getenv("DUO_FAULT_INJECT");
  if (!e || !*e) return DUO_OK;
  if (std::strcmp(e, "all") != 0 &&
      (std::string(",") + e + ",").find(std::string(",") + call + ",") == std::string::npos)
    return DUO_OK;
  return fail(DUO_E_HIP, std::string(call) + ": fault injected (DUO_FAULT_INJECT)");
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr uint64_t kAlign = 256;
uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

struct LayerLayout {
  int n_ret = 0, n_str = 0;
  uint64_t ret_k = 0, ret_v = 0, ret_km = 0, ret_vm = 0;
  uint64_t str_k = 0, str_v = 0, str_km = 0, str_vm = 0;
};

struct Layout {
  int64_t cap = 0;   // retrieval rows per cache
  int64_t nslot = 0; // streaming slots per cache
  std::vector<LayerLayout> layers;
  uint64_t partials = 0, counters = 0, prefill_counters = 0, total = 0;
  // streaming-head prefill staging (bf16, head_dim 128, bf16 caches only)
  int stage_tokens = 0;       // queries per staged launch
  int64_t stage_rows = 0;     // rows per streaming cache
  int stage_caches = 0;       // batch * most streaming heads of any layer
  uint64_t stage_k = 0, stage_v = 0;
  std::vector<uint64_t> guards;  // offsets of the guard bands (one after every region)
};

int validate_config(const duo_config* c) {
  if (!c) return fail(DUO_E_INVALID, "config is NULL");
  if (c->n_layers < 1) return fail(DUO_E_INVALID, "n_layers must be >= 1");
  if (c->batch < 1) return fail(DUO_E_INVALID, "batch must be >= 1");
  if (c->n_kv_heads < 1 || c->n_kv_heads > DUO_MAX_KV_HEADS)
    return fail(DUO_E_INVALID, "n_kv_heads must be in 1..64");
  if (c->n_q_heads < 1 || c->n_q_heads % c->n_kv_heads)
    return fail(DUO_E_INVALID, "n_q_heads must be a positive multiple of n_kv_heads");
  if (c->n_q_heads / c->n_kv_heads > DUO_MAX_GROUP)
    return fail(DUO_E_UNSUPPORTED, "n_q_heads / n_kv_heads above 16 is not supported");
  if (c->head_dim != 64 && c->head_dim != 128) return fail(DUO_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (c->sink < 0) return fail(DUO_E_INVALID, "sink must be >= 0");
  if (c->recent < 1) return fail(DUO_E_INVALID, "recent must be >= 1");
  // Bounded so that every sum of sink, recent and a tile's rows stays within int32
  // (kernels index the constant-length caches with 32-bit slot counts).
  if (c->sink > DUO_MAX_WINDOW || c->recent > DUO_MAX_WINDOW)
    return fail(DUO_E_UNSUPPORTED, "sink and recent above 2^28 tokens each are not supported");
  if (c->max_context < 1 || c->max_context > (int64_t(1) << 40)) return fail(DUO_E_INVALID, "max_context out of range");
  if (c->io_dtype != DUO_DTYPE_F32 && c->io_dtype != DUO_DTYPE_BF16) return fail(DUO_E_INVALID, "unknown io_dtype");
  if (c->kv_format != DUO_KV_SAME_AS_IO && c->kv_format != DUO_KV_INT4_G128)
    return fail(DUO_E_INVALID, "unknown kv_format");
  if (c->kv_format == DUO_KV_INT4_G128 && (c->io_dtype != DUO_DTYPE_BF16 || c->head_dim != 128))
    return fail(DUO_E_UNSUPPORTED, "int4 KV needs bf16 I/O and head_dim 128");
  if (c->reserved != 0) return fail(DUO_E_INVALID, "reserved must be 0");
  if (!(c->scale >= 0.0f) || !std::isfinite(c->scale)) return fail(DUO_E_INVALID, "scale must be finite and >= 0");
  if (!c->retrieval_mask) return fail(DUO_E_INVALID, "retrieval_mask is NULL");
  const int64_t n = int64_t(c->n_layers) * c->n_kv_heads;
  for (int64_t i = 0; i < n; ++i)
    if (c->retrieval_mask[i] > 1) return fail(DUO_E_INVALID, "retrieval_mask entries must be 0 or 1");
  return DUO_OK;
}

// Byte layout of the workspace.  Returns false on arithmetic overflow.
bool make_layout(const duo_config* c, Layout* L) {
  const uint64_t B = c->batch, D = c->head_dim;
  L->cap = int64_t(align_up(uint64_t(c->max_context), duo::kRowAlign));
  L->nslot = int64_t(align_up(uint64_t(c->sink) + uint64_t(c->recent), duo::kRowAlign));
  const bool int4 = c->kv_format == DUO_KV_INT4_G128;
  const uint64_t esize = c->io_dtype == DUO_DTYPE_F32 ? 4 : 2;
  // bytes per stored vector (codes or values) and per meta entry
  const uint64_t vec = int4 ? D / 2 : D * esize;
  const uint64_t meta = int4 ? 4 : 0;
  uint64_t off = 0;
  const long double limit = 1.0e18L;
  L->guards.clear();
  // A region of `bytes` bytes at the current offset, then its guard band.
  auto region = [&](uint64_t bytes) {
    const uint64_t at = off;
    off = align_up(off + bytes, kAlign);
    L->guards.push_back(off);
    off += DUO_GUARD_BYTES;
    return at;
  };
  L->layers.assign(c->n_layers, LayerLayout());
  for (int l = 0; l < c->n_layers; ++l) {
    LayerLayout& y = L->layers[l];
    for (int h = 0; h < c->n_kv_heads; ++h)
      (c->retrieval_mask[l * c->n_kv_heads + h] ? y.n_ret : y.n_str)++;
    const long double ret_rows = (long double)B * y.n_ret * L->cap;
    const long double str_rows = (long double)B * y.n_str * L->nslot;
    if (ret_rows * vec * 2 + str_rows * vec * 2 + (ret_rows + str_rows) * meta * 2 + (long double)off > limit)
      return false;
    const uint64_t rr = B * y.n_ret * uint64_t(L->cap), sr = B * y.n_str * uint64_t(L->nslot);
    y.ret_k = region(rr * vec);
    y.ret_v = region(rr * vec);
    y.str_k = region(sr * vec);
    y.str_v = region(sr * vec);
    if (int4) {
      y.ret_km = region(rr * meta);
      y.ret_vm = region(rr * meta);
      y.str_km = region(sr * meta);
      y.str_vm = region(sr * meta);
    }
  }
  L->partials = region(B * c->n_q_heads * uint64_t(duo::kMaxSplits) * (D + 2) * 4);
  L->counters = region(B * c->n_kv_heads * 4);
  L->prefill_counters = region(uint64_t(duo::kPrefillCounters) * 4);
  if (c->io_dtype == DUO_DTYPE_BF16 && D == 128 && !int4) {
    int n_str = 0;
    for (const LayerLayout& y : L->layers) n_str = y.n_str > n_str ? y.n_str : n_str;
    L->stage_tokens = int(L->cap < duo::kStageTokens ? L->cap : duo::kStageTokens);
    L->stage_rows = duo::stage_sink_rows(c->sink) + duo::stage_window_rows(c->recent) + L->stage_tokens;
    L->stage_caches = int(B) * n_str;
    const uint64_t bytes = uint64_t(L->stage_caches) * uint64_t(L->stage_rows) * D * 2;
    L->stage_k = region(bytes);
    L->stage_v = region(bytes);
  }
  L->total = off;
  return true;
}

}  // namespace

// Kernel timing (duo_profile.h): event pairs stamped at the dispatch of each launch.
struct Profiler {
  bool profiling = false;
  struct Mark { int cls; hipEvent_t start, stop; };
  std::vector<Mark> marks;
  std::vector<hipEvent_t> event_pool;
  ~Profiler() {
    for (Mark& m : marks) { event_pool.push_back(m.start); event_pool.push_back(m.stop); }
    for (hipEvent_t e : event_pool) (void)hipEventDestroy(e);
  }
};

struct duo_handle : Profiler {
  duo_config cfg;
  std::vector<uint8_t> mask;
  char* ws = nullptr;
  uint64_t ws_bytes = 0;
  Layout layout;
  Geom geom;
  std::vector<LayerView> views;
  std::vector<int64_t> len;  // [layer * batch + sequence]: tokens held
  CacheRegion stage{};   // streaming-head prefill staging (MFMA path)
  int stage_tokens = 0;
  float* partials = nullptr;
  int64_t partial_floats = 0;
  int* counters = nullptr;
  int* prefill_counters = nullptr;
  int num_cu = 256;
  int device = 0;                // the device current at init (its static scratch serves duo_decode_static)
  bool use_mfma = false;         // bf16 caches: MFMA prefill + decode (append fused into decode)
  bool use_mfma_decode = false;  // MFMA decode (bf16 or int4 caches)
};

namespace duo {
LaunchEvents& launch_events() {
  thread_local LaunchEvents ev;
  return ev;
}
}  // namespace duo

namespace {

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

hipEvent_t take_event(Profiler* h) {
  if (!h->event_pool.empty()) {
    hipEvent_t e = h->event_pool.back();
    h->event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Times the one kernel launch made inside its scope when the handle is profiling: the
// launcher stamps the event pair at the dispatch's own begin and end.
struct KernelMark {
  Profiler* h;
  int cls;
  hipEvent_t start = nullptr, stop = nullptr;
  KernelMark(Profiler* h_, int cls_, hipStream_t) : h(h_), cls(cls_) {
    if (!h->profiling) return;
    start = take_event(h);
    stop = start ? take_event(h) : nullptr;
    if (start && stop) {
      duo::launch_events() = duo::LaunchEvents{start, stop};
    } else {
      if (start) h->event_pool.push_back(start);
      start = nullptr;
    }
  }
  ~KernelMark() {
    if (!start) return;
    if (duo::launch_events().start == nullptr) {  // the launch took the pair
      h->marks.push_back(Profiler::Mark{cls, start, stop});
    } else {                                       // nothing was launched
      duo::launch_events() = duo::LaunchEvents{};
      h->event_pool.push_back(start);
      h->event_pool.push_back(stop);
    }
  }
};

int check_layer(const duo_handle* h, int32_t layer) {
  if (!h) return fail(DUO_E_INVALID, "handle is NULL");
  if (layer < 0 || layer >= h->cfg.n_layers) return fail(DUO_E_INVALID, "layer out of range");
  return DUO_OK;
}

int check_ptr(const void* p, const char* name) {
  if (!p) return fail(DUO_E_INVALID, std::string(name) + " is NULL");
  if (!aligned16(p)) return fail(DUO_E_INVALID, std::string(name) + " is not 16-byte aligned");
  return DUO_OK;
}

// Decode plan of `layer` at query position t with split partials in `partials`
// (max_splits slots per query head) and arrival counters in `counters`.  Returns false
// (with the error set) when the key range cannot be split within max_splits.
bool make_plan(const duo_handle* h, int32_t layer, int64_t t, float* partials, int* counters, int max_splits,
               duo::DecodePlan* out) {
  duo::DecodePlan& p = *out;
  p.t = t;
  p.varlen = 0;
  for (int b = 0; b < duo::kMaxVarlen; ++b) p.t_seq[b] = t;
  p.partials = partials;
  p.max_splits = max_splits;
  p.counters = counters;
  p.k_new = nullptr;
  p.v_new = nullptr;
  p.new_slot = duo::stream_slot(t, h->cfg.sink, h->cfg.recent);
  const int64_t nkeys = t + 1;
  const int64_t batch = h->cfg.batch;
  // Streaming heads: one split each (no merge) up to 2048 slots; a longer window is
  // split in pieces of at least 2048 slots, and of at least 1/max_splits of the window
  // so that the split count stays within the partial buffer.
  const int64_t window = int64_t(h->cfg.sink) + int64_t(h->cfg.recent);
  const int64_t nslots = nkeys < window ? nkeys : window;
  int64_t chunk_s = nslots < 2048 ? nslots : 2048;
  const int64_t min_chunk_s = (nslots + max_splits - 1) / max_splits;
  if (chunk_s < min_chunk_s) chunk_s = min_chunk_s;
  chunk_s = int64_t(align_up(uint64_t(chunk_s), 64));
  // Retrieval heads: the decode workgroup fills a CU, so the splits share what the
  // streaming workgroups leave of one workgroup per CU (at least 512 keys per split, a
  // multiple of 64, within the partial buffer).
  const int64_t heads = batch * h->views[layer].n_ret;
  const int64_t nsplit_s = (nslots + chunk_s - 1) / chunk_s;
  const int64_t str_wgs = batch * h->views[layer].n_str * nsplit_s;
  int64_t chunk = 512;
  if (heads > 0) {
    int64_t slots = h->num_cu - str_wgs;
    if (slots < heads) slots = heads;
    const int64_t per_head = slots / heads;
    const int64_t want = (nkeys + per_head - 1) / per_head;
    if (want > chunk) chunk = want;
  }
  const int64_t min_chunk = (nkeys + max_splits - 1) / max_splits;
  if (chunk < min_chunk) chunk = min_chunk;
  // a split's K and V are addressed with 32-bit byte offsets (256 bytes per key)
  constexpr int64_t kMaxChunk = int64_t(1) << 22;
  if (chunk > kMaxChunk) chunk = kMaxChunk;
  chunk = int64_t(align_up(uint64_t(chunk), 64));
  if (chunk_s > kMaxChunk) chunk_s = kMaxChunk;
  p.chunk_r = int(chunk);
  p.nsplit_r = int((nkeys + chunk - 1) / chunk);
  p.chunk_s = int(chunk_s);
  p.nsplit_s = int((nslots + chunk_s - 1) / chunk_s);
  if (p.nsplit_r > max_splits || p.nsplit_s > max_splits) {
    fail(DUO_E_UNSUPPORTED, "decode key range needs more splits than the partial buffer holds");
    return false;
  }
  return true;
}

// ---- Static scratch of duo_decode_static ------------------------------------------
// Device memory that the library holds for callers that cannot allocate: one array per
// GPU (each device holds its own copy of a __device__ array until the process ends).
// Its device address is taken once per device with hipGetSymbolAddress, with that
// device current, at the first duo_kv_init on it; host code uses that address only (the
// array's name is a host-side stand-in, not a device address).  Layout: arrival
// counters first (kStaticCounterBytes), then split partials.
constexpr uint64_t kStaticCounterBytes = 64 << 10;
static_assert(DUO_STATIC_SCRATCH_BYTES > kStaticCounterBytes, "static scratch too small");

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, once set up
int g_scratch_state[kMaxDevices];   // 0: not set up, 1: ready, -1: set-up failed
std::string g_scratch_err[kMaxDevices];

// Set-up on the current device `dev` (once): the array's device address, and its
// counters cleared by a fill kernel (the kernels leave every counter at zero after
// each call, so one clear serves every later call).  The clear is waited for here, so
// calls on any stream afterwards see zeroed counters.
void setup_static_scratch(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_state[dev] != 0) return;
  void* ptr = nullptr;
  hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e == hipSuccess && ptr == nullptr) e = hipErrorInvalidSymbol;
  if (e == hipSuccess) e = duo::launch_zero_bytes(ptr, kStaticCounterBytes, nullptr);
  if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
  if (e != hipSuccess) {
    g_scratch_state[dev] = -1;
    g_scratch_err[dev] = std::string("static scratch set-up: ") + hipGetErrorString(e);
    return;
  }
  g_scratch_ptr[dev] = static_cast<char*>(ptr);
  g_scratch_state[dev] = 1;
}

struct StaticScratch {
  float* partials;
  int* counters;
  int max_splits;
};

// The static scratch of the handle's device, sized for its decode.
int static_scratch(const duo_handle* h, StaticScratch* out) {
  const int dev = h->device;
  if (dev < 0 || dev >= kMaxDevices) return fail(DUO_E_UNSUPPORTED, "static scratch: device index above 63");
  char* base = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_state[dev] != 1)
      return fail(DUO_E_HIP, g_scratch_state[dev] == 0 ? std::string("static scratch was not set up")
                                                        : g_scratch_err[dev]);
    base = g_scratch_ptr[dev];
  }
  const uint64_t counters = uint64_t(h->cfg.batch) * h->cfg.n_kv_heads * 4;
  if (counters > kStaticCounterBytes)
    return fail(DUO_E_CAPACITY, "static scratch: batch * n_kv_heads above 16384 arrival counters");
  const uint64_t per_split = uint64_t(h->cfg.batch) * h->cfg.n_q_heads * (h->cfg.head_dim + 2) * 4;
  uint64_t splits = (DUO_STATIC_SCRATCH_BYTES - kStaticCounterBytes) / per_split;
  if (splits > uint64_t(duo::kMaxSplits)) splits = duo::kMaxSplits;
  if (splits < 1)
    return fail(DUO_E_CAPACITY, "static scratch: one split of every query head needs " + std::to_string(per_split) +
                                    " bytes, above the library's " + std::to_string(DUO_STATIC_SCRATCH_BYTES - kStaticCounterBytes));
  out->counters = reinterpret_cast<int*>(base);
  out->partials = reinterpret_cast<float*>(base + kStaticCounterBytes);
  out->max_splits = int(splits);
  return DUO_OK;
}

}  // namespace

extern "C" {

const char* duo_last_error(void) { return g_last_error.c_str(); }

int duo_kv_bytes(const duo_config* cfg, uint64_t* out_bytes) {
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (!out_bytes) return fail(DUO_E_INVALID, "out_bytes is NULL");
  Layout L;
  if (!make_layout(cfg, &L)) return fail(DUO_E_INVALID, "workspace size overflows");
  *out_bytes = L.total;
  return ok();
}

// Checks shared by duo_kv_init and duo_kv_attach (config, workspace pointer and size);
// fills the layout.
static int check_workspace(const duo_config* cfg, void* d_workspace, uint64_t bytes, duo_handle** out, Layout* L) {
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (!out) return fail(DUO_E_INVALID, "out is NULL");
  if (!d_workspace) return fail(DUO_E_INVALID, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(d_workspace) % kAlign) return fail(DUO_E_INVALID, "workspace is not 256-byte aligned");
  if (!make_layout(cfg, L)) return fail(DUO_E_INVALID, "workspace size overflows");
  if (bytes < L->total) return fail(DUO_E_CAPACITY, "workspace smaller than duo_kv_bytes()");
  return DUO_OK;
}

// A handle over the workspace with every length 0 (host state only, apart from the
// once-per-device set-up of the static scratch).
static duo_handle* new_handle(const duo_config* cfg, void* d_workspace, uint64_t bytes, const Layout& L) {
  duo_handle* h = new duo_handle();
  h->cfg = *cfg;
  h->mask.assign(cfg->retrieval_mask, cfg->retrieval_mask + size_t(cfg->n_layers) * cfg->n_kv_heads);
  h->cfg.retrieval_mask = h->mask.data();
  h->ws = static_cast<char*>(d_workspace);
  h->ws_bytes = bytes;
  h->layout = L;
  Geom& g = h->geom;
  g.B = cfg->batch;
  g.Hq = cfg->n_q_heads;
  g.Hkv = cfg->n_kv_heads;
  g.G = cfg->n_q_heads / cfg->n_kv_heads;
  g.D = cfg->head_dim;
  g.S = cfg->sink;
  g.R = cfg->recent;
  g.io = cfg->io_dtype;
  g.kvfmt = cfg->kv_format;
  g.scale = cfg->scale > 0.0f ? cfg->scale : 1.0f / std::sqrt(float(cfg->head_dim));
  g.scale_log2 = g.scale * 1.4426950408889634f;
  const bool int4 = cfg->kv_format == DUO_KV_INT4_G128;
  h->views.resize(cfg->n_layers);
  for (int l = 0; l < cfg->n_layers; ++l) {
    const LayerLayout& y = L.layers[l];
    LayerView& v = h->views[l];
    std::memset(&v, 0, sizeof(v));
    v.n_ret = y.n_ret;
    v.n_str = y.n_str;
    // bf16 K with head_dim 128 lives in MFMA-ordered 32-key tiles (int4 K codes always do)
    const int tiled = cfg->io_dtype == DUO_DTYPE_BF16 && cfg->head_dim == 128 && !int4;
    v.ret = CacheRegion{h->ws + y.ret_k, h->ws + y.ret_v,
                        int4 ? reinterpret_cast<uint16_t*>(h->ws + y.ret_km) : nullptr,
                        int4 ? reinterpret_cast<uint16_t*>(h->ws + y.ret_vm) : nullptr, L.cap, tiled};
    v.str = CacheRegion{h->ws + y.str_k, h->ws + y.str_v,
                        int4 ? reinterpret_cast<uint16_t*>(h->ws + y.str_km) : nullptr,
                        int4 ? reinterpret_cast<uint16_t*>(h->ws + y.str_vm) : nullptr, L.nslot, tiled};
    int nr = 0, ns = 0;
    for (int kv = 0; kv < cfg->n_kv_heads; ++kv) {
      if (h->mask[size_t(l) * cfg->n_kv_heads + kv]) {
        v.kind[kv] = duo::kKindRetrieval;
        v.slot[kv] = nr;
        v.ret_kv[nr++] = kv;
      } else {
        v.kind[kv] = duo::kKindStreaming;
        v.slot[kv] = ns;
        v.str_kv[ns++] = kv;
      }
    }
  }
  h->len.assign(size_t(cfg->n_layers) * cfg->batch, 0);
  h->stage = CacheRegion{h->ws + L.stage_k, h->ws + L.stage_v, nullptr, nullptr, L.stage_rows, 1};
  h->stage_tokens = L.stage_tokens;
  h->partials = reinterpret_cast<float*>(h->ws + L.partials);
  h->counters = reinterpret_cast<int*>(h->ws + L.counters);
  h->prefill_counters = reinterpret_cast<int*>(h->ws + L.prefill_counters);
  h->partial_floats = int64_t(cfg->batch) * cfg->n_q_heads * duo::kMaxSplits * (cfg->head_dim + 2);
  int dev = 0;
  if (hipGetDevice(&dev) == hipSuccess) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) h->num_cu = n;
    h->device = dev;
    setup_static_scratch(dev);
  }
  // bf16 with head_dim 128 runs on the MFMA kernels (int4 caches: decode only); fp32
  // I/O and head_dim 64 on the vector-ALU kernels.
  h->use_mfma = cfg->io_dtype == DUO_DTYPE_BF16 && cfg->head_dim == 128 && cfg->kv_format == DUO_KV_SAME_AS_IO;
  h->use_mfma_decode = cfg->io_dtype == DUO_DTYPE_BF16 && cfg->head_dim == 128;
  return h;
}

int duo_kv_init(const duo_config* cfg, void* d_workspace, uint64_t bytes, void* hip_stream, duo_handle** out) {
  Layout L;
  int rc = check_workspace(cfg, d_workspace, bytes, out, &L);
  if (rc) return rc;
  if ((rc = injected_fault("duo_kv_init"))) return rc;
  duo_handle* h = new_handle(cfg, d_workspace, bytes, L);
  if (log_enabled())
    std::fprintf(stderr, "duo: init layers=%d batch=%d heads=%d/%d head_dim=%d workspace=%llu bytes (%zu guard bands) "
                 "kernels=%s\n", cfg->n_layers, cfg->batch, cfg->n_q_heads, cfg->n_kv_heads, cfg->head_dim,
                 static_cast<unsigned long long>(L.total), L.guards.size(),
                 h->use_mfma ? "mfma" : (h->use_mfma_decode ? "mfma decode, valu prefill" : "valu"));
  // Clear every cache and the counters.  The MFMA kernels read whole 32/64-row tiles
  // and weight rows past the valid length by exactly zero, which needs those rows
  // finite; cleared memory guarantees it.
  hipError_t e = duo::launch_zero_bytes(h->ws, L.partials, as_stream(hip_stream));
  if (e == hipSuccess)
    e = duo::launch_zero_bytes(h->ws + L.counters, L.total - L.counters, as_stream(hip_stream));
  if (e == hipSuccess)
    e = duo::launch_guard_fill(h->ws, L.guards.data(), static_cast<int>(L.guards.size()), DUO_GUARD_WORD,
                               as_stream(hip_stream));
  if (e != hipSuccess) {
    delete h;
    return hip_fail(e, "clearing the workspace");
  }
  *out = h;
  return ok();
}

int duo_kv_attach(const duo_config* cfg, void* d_workspace, uint64_t bytes, const int64_t* lengths,
                  duo_handle** out) {
  Layout L;
  int rc = check_workspace(cfg, d_workspace, bytes, out, &L);
  if (rc) return rc;
  if (!lengths) return fail(DUO_E_INVALID, "lengths is NULL");
  const size_t n = size_t(cfg->n_layers) * cfg->batch;
  for (size_t i = 0; i < n; ++i)
    if (lengths[i] < 0 || lengths[i] > cfg->max_context)
      return fail(DUO_E_INVALID, "lengths must be in 0..max_context");
  if ((rc = injected_fault("duo_kv_attach"))) return rc;
  duo_handle* h = new_handle(cfg, d_workspace, bytes, L);
  h->len.assign(lengths, lengths + n);
  *out = h;
  return ok();
}

void duo_kv_free(duo_handle* h) { delete h; }

int duo_kv_guard_bands(const duo_handle* h, uint64_t* offsets, int32_t max, int32_t* n) {
  if (!h) return fail(DUO_E_INVALID, "handle is NULL");
  if (!n) return fail(DUO_E_INVALID, "n is NULL");
  if (max < 0) return fail(DUO_E_INVALID, "max must be >= 0");
  if (max > 0 && !offsets) return fail(DUO_E_INVALID, "offsets is NULL");
  const std::vector<uint64_t>& g = h->layout.guards;
  for (size_t i = 0; i < g.size() && i < size_t(max); ++i) offsets[i] = g[i];
  *n = static_cast<int32_t>(g.size());
  return ok();
}

static int64_t& seq_len(duo_handle* h, int32_t layer, int32_t seq) { return h->len[size_t(layer) * h->cfg.batch + seq]; }
static int64_t seq_len(const duo_handle* h, int32_t layer, int32_t seq) {
  return h->len[size_t(layer) * h->cfg.batch + seq];
}

// The layer's length when every sequence of the batch holds the same number of tokens.
static int batch_len(const duo_handle* h, int32_t layer, int64_t* out) {
  const int64_t l0 = seq_len(h, layer, 0);
  for (int32_t b = 1; b < h->cfg.batch; ++b)
    if (seq_len(h, layer, b) != l0)
      return fail(DUO_E_STATE, "the sequences of the batch hold different lengths (use the per-sequence calls)");
  *out = l0;
  return DUO_OK;
}

int duo_kv_length(const duo_handle* h, int32_t layer, int64_t* out_len) {
  int rc = check_layer(h, layer);
  if (rc) return rc;
  if (!out_len) return fail(DUO_E_INVALID, "out_len is NULL");
  int64_t l = 0;
  if ((rc = batch_len(h, layer, &l))) return rc;
  *out_len = l;
  return ok();
}

int duo_kv_length_seq(const duo_handle* h, int32_t layer, int32_t seq, int64_t* out_len) {
  int rc = check_layer(h, layer);
  if (rc) return rc;
  if (seq < 0 || seq >= h->cfg.batch) return fail(DUO_E_INVALID, "sequence index out of range");
  if (!out_len) return fail(DUO_E_INVALID, "out_len is NULL");
  *out_len = seq_len(h, layer, seq);
  return ok();
}

static int check_tokens(int64_t len, int64_t max_context, int32_t n_tokens) {
  if (n_tokens <= 0) return fail(DUO_E_INVALID, "n_tokens must be > 0");
  if (len + n_tokens > max_context) return fail(DUO_E_CAPACITY, "length + n_tokens exceeds max_context");
  return DUO_OK;
}

// The caches of one sequence as a batch of one: every region starts at the sequence's
// first cache (caches are whole multiples of 64 rows, so tiled and blocked layouts keep
// their alignment).
static void one_sequence(const duo_handle* h, int32_t layer, int32_t seq, duo::Geom* g, LayerView* lv) {
  *g = h->geom;
  g->B = 1;
  *lv = h->views[layer];
  const bool int4 = h->cfg.kv_format == DUO_KV_INT4_G128;
  const int64_t vec = int4 ? h->cfg.head_dim / 2 : int64_t(h->cfg.head_dim) * (h->cfg.io_dtype == DUO_DTYPE_F32 ? 4 : 2);
  auto shift = [&](CacheRegion& c, int64_t caches) {
    const int64_t rows = caches * c.rows;
    c.k += rows * vec;
    c.v += rows * vec;
    if (c.k_meta) c.k_meta += rows * 2;
    if (c.v_meta) c.v_meta += rows * 2;
  };
  shift(lv->ret, int64_t(seq) * lv->n_ret);
  shift(lv->str, int64_t(seq) * lv->n_str);
}

// Prefill of n_tokens at positions [t0, t0 + n_tokens) for the batch described by (g, lv).
static int run_prefill(duo_handle* h, const duo::Geom& g, const LayerView& lv, const void* q, const void* k,
                       const void* v, int32_t n_tokens, void* out, int64_t t0, hipStream_t st) {
  hipError_t e;
  if (h->use_mfma) {
    // One launch writes the chunk into the retrieval caches (the retrieval kernel reads
    // its keys there) and stages the keys of the first streaming-head queries; the
    // streaming caches, read as they stood before the chunk, are updated last.
    const int nq0 = lv.n_str > 0 ? (n_tokens < h->stage_tokens ? n_tokens : h->stage_tokens) : 0;
    {
      KernelMark m(h, DUO_KERNEL_PREFILL_STAGE, st);
      e = duo::launch_chunk_tiles(g, lv, h->stage, k, v, n_tokens, t0, true, 0, nq0, st);
    }
    if (e != hipSuccess) return hip_fail(e, "prefill append and staging");
    // When every streaming-head query was staged above, the streaming caches' update
    // (nothing later reads them as they stood) joins the attention launch.
    const bool fuse_update = n_tokens <= h->stage_tokens;
    duo::PrefillLaunchInfo info{};
    {  // retrieval heads and the first staged streaming-head queries, one launch
      KernelMark m(h, DUO_KERNEL_PREFILL_RETRIEVAL, st);
      e = duo::launch_prefill_mfma(g, lv, h->stage, q, out, n_tokens, t0, nq0, h->partials, h->partial_floats,
                                   h->prefill_counters, h->num_cu, st, nullptr, fuse_update ? k : nullptr,
                                   fuse_update ? v : nullptr, &info);
    }
    if (e != hipSuccess) return hip_fail(e, "prefill attention");
    if (log_enabled())
      std::fprintf(stderr,
                   "duo: prefill t0=%lld tokens=%d batch=%d workgroups of %d wavefronts (%d heads x %d queries) "
                   "retrieval=%d (key splits %d) streaming=%d (first %d queries, staged passes %d) "
                   "cache update=%s\n",
                   static_cast<long long>(t0), n_tokens, g.B, info.waves, info.pack, info.qrows, info.ret_blocks,
                   info.nsplit, info.str_blocks, nq0,
                   nq0 > 0 ? (n_tokens + h->stage_tokens - 1) / h->stage_tokens : 0,
                   fuse_update ? "in the launch" : "own launch");
    // further streaming-head queries, at most stage_tokens per launch pair (the staging
    // capacity)
    for (int q0 = h->stage_tokens; q0 < n_tokens && nq0 > 0; q0 += h->stage_tokens) {
      const int nq = n_tokens - q0 < h->stage_tokens ? n_tokens - q0 : h->stage_tokens;
      {
        KernelMark m(h, DUO_KERNEL_PREFILL_STAGE, st);
        e = duo::launch_chunk_tiles(g, lv, h->stage, k, v, n_tokens, t0, false, q0, nq, st);
      }
      if (e != hipSuccess) return hip_fail(e, "prefill staging (streaming)");
      {
        KernelMark m(h, DUO_KERNEL_PREFILL_STREAMING, st);
        e = duo::launch_prefill_stream_mfma(g, lv, h->stage, q, out, n_tokens, t0, q0, nq, st);
      }
      if (e != hipSuccess) return hip_fail(e, "prefill attention (streaming)");
    }
    if (!fuse_update) {
      KernelMark m(h, DUO_KERNEL_APPEND, st);
      e = duo::launch_stream_cache_update(g, lv, k, v, n_tokens, t0, st);
    }
    if (e != hipSuccess) return hip_fail(e, "prefill append (streaming)");
  } else {
    {
      KernelMark m(h, DUO_KERNEL_PREFILL_RETRIEVAL, st);
      e = duo::launch_prefill_valu(g, lv, q, k, v, out, n_tokens, t0, st);
    }
    if (e != hipSuccess) return hip_fail(e, "prefill attention");
    {
      KernelMark m(h, DUO_KERNEL_APPEND, st);
      e = duo::launch_append(g, lv, k, v, n_tokens, t0, 3, st);
    }
    if (e != hipSuccess) return hip_fail(e, "prefill append");
  }
  return DUO_OK;
}

int duo_prefill(duo_handle* h, int32_t layer, const void* q, const void* k, const void* v, int32_t n_tokens,
                void* out, void* hip_stream) {
  int rc = check_layer(h, layer);
  if (rc) return rc;
  if ((rc = check_ptr(q, "q")) || (rc = check_ptr(k, "k")) || (rc = check_ptr(v, "v")) || (rc = check_ptr(out, "out")))
    return rc;
  if (h->cfg.kv_format == DUO_KV_INT4_G128) return fail(DUO_E_UNSUPPORTED, "prefill with an int4 cache");
  int64_t t0 = 0;
  if ((rc = batch_len(h, layer, &t0)) || (rc = check_tokens(t0, h->cfg.max_context, n_tokens))) return rc;
  if ((rc = injected_fault("duo_prefill"))) return rc;
  if ((rc = run_prefill(h, h->geom, h->views[layer], q, k, v, n_tokens, out, t0, as_stream(hip_stream)))) return rc;
  for (int32_t b = 0; b < h->cfg.batch; ++b) seq_len(h, layer, b) = t0 + n_tokens;
  return ok();
}

int duo_prefill_seq(duo_handle* h, int32_t layer, int32_t seq, const void* q, const void* k, const void* v,
                    int32_t n_tokens, void* out, void* hip_stream) {
  int rc = check_layer(h, layer);
  if (rc) return rc;
  if (seq < 0 || seq >= h->cfg.batch) return fail(DUO_E_INVALID, "sequence index out of range");
  if ((rc = check_ptr(q, "q")) || (rc = check_ptr(k, "k")) || (rc = check_ptr(v, "v")) || (rc = check_ptr(out, "out")))
    return rc;
  if (h->cfg.kv_format == DUO_KV_INT4_G128) return fail(DUO_E_UNSUPPORTED, "prefill with an int4 cache");
  const int64_t t0 = seq_len(h, layer, seq);
  if ((rc = check_tokens(t0, h->cfg.max_context, n_tokens))) return rc;
  if ((rc = injected_fault("duo_prefill_seq"))) return rc;
  duo::Geom g;
  LayerView lv;
  one_sequence(h, layer, seq, &g, &lv);
  if ((rc = run_prefill(h, g, lv, q, k, v, n_tokens, out, t0, as_stream(hip_stream)))) return rc;
  seq_len(h, layer, seq) = t0 + n_tokens;
  return ok();
}

int duo_prefill_dual(duo_handle* h, int32_t layer, const void* q, const void* k, const void* v, int32_t n_tokens,
                     void* out_full, void* out_streaming, void* hip_stream) {
  int rc = check_layer(h, layer);
  if (rc) return rc;
  if ((rc = check_ptr(q, "q")) || (rc = check_ptr(k, "k")) || (rc = check_ptr(v, "v")) ||
      (rc = check_ptr(out_full, "out_full")) || (rc = check_ptr(out_streaming, "out_streaming")))
    return rc;
  if (!h->use_mfma) return fail(DUO_E_UNSUPPORTED, "both outputs need bf16 I/O, head_dim 128 and bf16 caches");
  const LayerView& lv = h->views[layer];
  if (lv.n_str != 0) return fail(DUO_E_STATE, "every KV head of the layer must be a retrieval head (full caches)");
  int64_t t0 = 0;
  if ((rc = batch_len(h, layer, &t0)) || (rc = check_tokens(t0, h->cfg.max_context, n_tokens))) return rc;
  if ((rc = injected_fault("duo_prefill_dual"))) return rc;
  hipStream_t st = as_stream(hip_stream);
  hipError_t e;
  {
    KernelMark m(h, DUO_KERNEL_PREFILL_STAGE, st);
    e = duo::launch_chunk_tiles(h->geom, lv, h->stage, k, v, n_tokens, t0, true, 0, 0, st);
  }
  if (e != hipSuccess) return hip_fail(e, "prefill append");
  {
    KernelMark m(h, DUO_KERNEL_PREFILL_RETRIEVAL, st);
    e = duo::launch_prefill_mfma(h->geom, lv, h->stage, q, out_full, n_tokens, t0, 0, h->partials,
                                 h->partial_floats, h->prefill_counters, h->num_cu, st, out_streaming);
  }
  if (e != hipSuccess) return hip_fail(e, "prefill attention (both outputs)");
  for (int32_t b = 0; b < h->cfg.batch; ++b) seq_len(h, layer, b) = t0 + n_tokens;
  return ok();
}

int duo_kv_append(duo_handle* h, int32_t layer, const void* k, const void* v, int32_t n_tokens, void* hip_stream) {
  int rc = check_layer(h, layer);
  if (rc) return rc;
  if ((rc = check_ptr(k, "k")) || (rc = check_ptr(v, "v"))) return rc;
  int64_t t0 = 0;
  if ((rc = batch_len(h, layer, &t0)) || (rc = check_tokens(t0, h->cfg.max_context, n_tokens))) return rc;
  if ((rc = injected_fault("duo_kv_append"))) return rc;
  if (log_enabled())
    std::fprintf(stderr, "duo: append layer=%d t0=%lld tokens=%d batch=%d\n", layer, static_cast<long long>(t0),
                 n_tokens, h->cfg.batch);
  hipError_t e;
  {
    KernelMark m(h, DUO_KERNEL_APPEND, as_stream(hip_stream));
    e = duo::launch_append(h->geom, h->views[layer], k, v, n_tokens, t0, 3, as_stream(hip_stream));
  }
  if (e != hipSuccess) return hip_fail(e, "append");
  for (int32_t b = 0; b < h->cfg.batch; ++b) seq_len(h, layer, b) = t0 + n_tokens;
  return ok();
}

int duo_kv_append_seq(duo_handle* h, int32_t layer, int32_t seq, const void* k, const void* v, int32_t n_tokens,
                      void* hip_stream) {
  int rc = check_layer(h, layer);
  if (rc) return rc;
  if (seq < 0 || seq >= h->cfg.batch) return fail(DUO_E_INVALID, "sequence index out of range");
  if ((rc = check_ptr(k, "k")) || (rc = check_ptr(v, "v"))) return rc;
  const int64_t t0 = seq_len(h, layer, seq);
  if ((rc = check_tokens(t0, h->cfg.max_context, n_tokens))) return rc;
  if ((rc = injected_fault("duo_kv_append_seq"))) return rc;
  duo::Geom g;
  LayerView lv;
  one_sequence(h, layer, seq, &g, &lv);
  hipError_t e;
  {
    KernelMark m(h, DUO_KERNEL_APPEND, as_stream(hip_stream));
    e = duo::launch_append(g, lv, k, v, n_tokens, t0, 3, as_stream(hip_stream));
  }
  if (e != hipSuccess) return hip_fail(e, "append");
  seq_len(h, layer, seq) = t0 + n_tokens;
  return ok();
}

// One decoding step (duo_decode) with its split partials and arrival counters in the
// given scratch (the workspace's, or the library's static array).
static int run_decode(const char* call, duo_handle* h, int32_t layer, const void* q, const void* k_new,
                      const void* v_new, void* out, void* hip_stream, float* partials, int* counters,
                      int max_splits) {
  int rc = check_layer(h, layer);
  if (rc) return rc;
  if ((rc = check_ptr(q, "q")) || (rc = check_ptr(out, "out"))) return rc;
  if ((k_new == nullptr) != (v_new == nullptr)) return fail(DUO_E_STATE, "k_new and v_new must both be set or both NULL");
  const bool append = k_new != nullptr;
  if (append && ((rc = check_ptr(k_new, "k_new")) || (rc = check_ptr(v_new, "v_new")))) return rc;
  const int32_t B = h->cfg.batch;
  int64_t tmax = -1;
  bool uniform = true;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t len = seq_len(h, layer, b);
    if (append && len + 1 > h->cfg.max_context) return fail(DUO_E_CAPACITY, "decode append exceeds max_context");
    if (!append && len < 1) return fail(DUO_E_STATE, "decode without new K/V on an empty sequence");
    const int64_t t = append ? len : len - 1;
    if (b > 0 && t != tmax) uniform = false;
    if (t > tmax) tmax = t;
  }
  if (!uniform && B > duo::kMaxVarlen)
    return fail(DUO_E_UNSUPPORTED, "decode of sequences of different lengths with batch > 32");
  const LayerView& lv = h->views[layer];
  hipStream_t st = as_stream(hip_stream);
  hipError_t e;
  duo::DecodePlan p;
  if (!make_plan(h, layer, tmax, partials, counters, max_splits, &p)) return DUO_E_UNSUPPORTED;
  if ((rc = injected_fault(call))) return rc;
  if (log_enabled())
    std::fprintf(stderr,
                 "duo: %s layer=%d t=%lld batch=%d varlen=%d retrieval=%d splits x %d keys streaming=%d splits x %d "
                 "slots max_splits=%d append=%d kernel=%s\n",
                 call, layer, static_cast<long long>(tmax), B, uniform ? 0 : 1, p.nsplit_r, p.chunk_r, p.nsplit_s,
                 p.chunk_s, p.max_splits, append ? 1 : 0, h->use_mfma_decode ? "mfma" : "valu");
  if (!uniform) {
    p.varlen = 1;
    for (int32_t b = 0; b < B; ++b) p.t_seq[b] = seq_len(h, layer, b) - (append ? 0 : 1);
  }
  if (append && h->use_mfma_decode) {
    // the MFMA decode (bf16 or int4 caches) appends the token itself (the workgroup
    // covering its row)
    p.k_new = static_cast<const uint16_t*>(k_new);
    p.v_new = static_cast<const uint16_t*>(v_new);
  } else if (append && uniform) {
    KernelMark m(h, DUO_KERNEL_APPEND, st);
    e = duo::launch_append(h->geom, lv, k_new, v_new, 1, tmax, 3, st);
    if (e != hipSuccess) return hip_fail(e, "decode append");
  } else if (append) {
    // one append per sequence, each at its own position
    const int64_t row_bytes = int64_t(h->cfg.n_kv_heads) * h->cfg.head_dim * (h->cfg.io_dtype == DUO_DTYPE_F32 ? 4 : 2);
    for (int32_t b = 0; b < B; ++b) {
      duo::Geom g1;
      LayerView lv1;
      one_sequence(h, layer, b, &g1, &lv1);
      KernelMark m(h, DUO_KERNEL_APPEND, st);
      e = duo::launch_append(g1, lv1, static_cast<const char*>(k_new) + b * row_bytes,
                             static_cast<const char*>(v_new) + b * row_bytes, 1, p.t_seq[b], 3, st);
      if (e != hipSuccess) return hip_fail(e, "decode append");
    }
  }
  {
    KernelMark m(h, DUO_KERNEL_DECODE, st);
    e = h->use_mfma_decode ? duo::launch_decode_mfma(h->geom, lv, p, q, out, st)
                           : duo::launch_decode_valu(h->geom, lv, p, q, out, st);
  }
  if (e != hipSuccess) return hip_fail(e, "decode attention");
  if (append)
    for (int32_t b = 0; b < B; ++b) ++seq_len(h, layer, b);
  return ok();
}

int duo_decode(duo_handle* h, int32_t layer, const void* q, const void* k_new, const void* v_new, void* out,
               void* hip_stream) {
  if (!h) return fail(DUO_E_INVALID, "handle is NULL");
  return run_decode("duo_decode", h, layer, q, k_new, v_new, out, hip_stream, h->partials, h->counters,
                    duo::kMaxSplits);
}

int duo_decode_static(duo_handle* h, int32_t layer, const void* q, const void* k_new, const void* v_new, void* out,
                      void* hip_stream) {
  if (!h) return fail(DUO_E_INVALID, "handle is NULL");
  StaticScratch sc;
  int rc = static_scratch(h, &sc);
  if (rc) return rc;
  return run_decode("duo_decode_static", h, layer, q, k_new, v_new, out, hip_stream, sc.partials, sc.counters,
                    sc.max_splits);
}

static int check_read(const duo_handle* h, int32_t layer, int32_t b, int32_t kv_head, int32_t which, int64_t pos0,
                      int32_t n, bool* streaming, int64_t* cache) {
  int rc = check_layer(h, layer);
  if (rc) return rc;
  if (b < 0 || b >= h->cfg.batch) return fail(DUO_E_INVALID, "sequence index out of range");
  if (kv_head < 0 || kv_head >= h->cfg.n_kv_heads) return fail(DUO_E_INVALID, "kv_head out of range");
  if (which != 0 && which != 1) return fail(DUO_E_INVALID, "which must be 0 (K) or 1 (V)");
  if (n < 0) return fail(DUO_E_INVALID, "n must be >= 0");
  const LayerView& lv = h->views[layer];
  *streaming = lv.kind[kv_head] == duo::kKindStreaming;
  *cache = int64_t(b) * (*streaming ? lv.n_str : lv.n_ret) + lv.slot[kv_head];
  const int64_t len = seq_len(h, layer, b);
  if (pos0 < 0 || pos0 + n > len) return fail(DUO_E_INVALID, "positions not yet appended");
  if (*streaming && n > 0) {
    const int64_t last = len - 1;
    for (int64_t p = pos0; p < pos0 + n; ++p)
      if (!(p < h->cfg.sink || last - p < h->cfg.recent))
        return fail(DUO_E_INVALID, "position evicted from the streaming cache");
  }
  return DUO_OK;
}

int duo_kv_read(const duo_handle* h, int32_t layer, int32_t b, int32_t kv_head, int32_t which, int64_t pos0,
                int32_t n, float* d_out, void* hip_stream) {
  bool streaming;
  int64_t cache;
  int rc = check_read(h, layer, b, kv_head, which, pos0, n, &streaming, &cache);
  if (rc) return rc;
  if ((rc = check_ptr(d_out, "out"))) return rc;
  if ((rc = injected_fault("duo_kv_read"))) return rc;
  if (n == 0) return ok();
  const LayerView& lv = h->views[layer];
  hipError_t e = duo::launch_read(h->geom, streaming ? lv.str : lv.ret, cache, streaming, pos0, n, which, d_out,
                                  as_stream(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "read");
  return ok();
}

int duo_kv_read_int4(const duo_handle* h, int32_t layer, int32_t b, int32_t kv_head, int32_t which, int64_t pos0,
                     int32_t n, uint8_t* d_codes, uint16_t* d_meta, void* hip_stream) {
  bool streaming;
  int64_t cache;
  int rc = check_read(h, layer, b, kv_head, which, pos0, n, &streaming, &cache);
  if (rc) return rc;
  if (h->cfg.kv_format != DUO_KV_INT4_G128) return fail(DUO_E_STATE, "cache is not int4");
  if ((rc = check_ptr(d_codes, "codes")) || (rc = check_ptr(d_meta, "meta"))) return rc;
  if ((rc = injected_fault("duo_kv_read_int4"))) return rc;
  if (n == 0) return ok();
  const LayerView& lv = h->views[layer];
  hipError_t e = duo::launch_read_int4(h->geom, streaming ? lv.str : lv.ret, cache, streaming, pos0, n, which,
                                       d_codes, d_meta, as_stream(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "read_int4");
  return ok();
}

int duo_profile_enable(duo_handle* h, int32_t on) {
  if (!h) return fail(DUO_E_INVALID, "handle is NULL");
  h->profiling = on != 0;
  return ok();
}

static int collect(Profiler* h, double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return fail(DUO_E_INVALID, "output array is NULL");
  for (int c = 0; c < DUO_KERNEL_CLASSES; ++c) {
    total_ms[c] = 0.0;
    launches[c] = 0;
  }
  int rc = DUO_OK;
  for (Profiler::Mark& m : h->marks) {
    float ms = 0.0f;
    hipError_t e = hipEventSynchronize(m.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, m.start, m.stop);
    if (e != hipSuccess && rc == DUO_OK) rc = hip_fail(e, "profile event");
    total_ms[m.cls] += ms;
    launches[m.cls] += 1;
    h->event_pool.push_back(m.start);
    h->event_pool.push_back(m.stop);
  }
  h->marks.clear();
  return rc == DUO_OK ? ok() : rc;
}

int duo_profile_collect(duo_handle* h, double* total_ms, int64_t* launches) {
  if (!h) return fail(DUO_E_INVALID, "handle is NULL");
  return collect(h, total_ms, launches);
}

// The calls that take no handle record on their host thread's profiler (kept for the
// thread's life; its few events are not released).
static Profiler& thread_profiler() {
  thread_local Profiler* p = new Profiler;
  return *p;
}

int duo_profile_thread_enable(int32_t on) {
  thread_profiler().profiling = on != 0;
  return ok();
}

int duo_profile_thread_collect(double* total_ms, int64_t* launches) {
  return collect(&thread_profiler(), total_ms, launches);
}

int duo_synth_fill(void* d_out, int32_t dtype, uint64_t seed, uint32_t stream, uint64_t counter0, uint64_t n,
                   void* hip_stream) {
  int rc = check_ptr(d_out, "out");
  if (rc) return rc;
  if (dtype != DUO_DTYPE_F32 && dtype != DUO_DTYPE_BF16 && dtype != DUO_SYNTH_INT8)
    return fail(DUO_E_INVALID, "unknown dtype");
  if (seed >> 32) return fail(DUO_E_INVALID, "seed must fit in 32 bits");
  hipError_t e = duo::launch_synth(d_out, dtype, seed, stream, counter0, n, as_stream(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "synth");
  return ok();
}

static int check_w8(const void* x, int64_t M, int32_t K, const int8_t* w, const float* scale, int32_t N) {
  int rc;
  if ((rc = check_ptr(x, "x")) || (rc = check_ptr(w, "w")) || (rc = check_ptr(scale, "scale"))) return rc;
  if (M < 1) return fail(DUO_E_INVALID, "M must be >= 1");
  if (K < 128 || K % 128 != 0) return fail(DUO_E_UNSUPPORTED, "K must be a positive multiple of 128");
  if (N < 256 || N % 256 != 0) return fail(DUO_E_UNSUPPORTED, "N must be a positive multiple of 256");
  if (M > (int64_t(1) << 24) || K > (1 << 20) || N > (1 << 20)) return fail(DUO_E_UNSUPPORTED, "size too large");
  return DUO_OK;
}

int duo_linear_w8(const void* x, int64_t M, int32_t K, const int8_t* w, const float* scale, int32_t N, void* y,
                  void* hip_stream) {
  int rc = check_w8(x, M, K, w, scale, N);
  if (rc || (rc = check_ptr(y, "y"))) return rc;
  duo::W8Args a{};
  a.x = static_cast<const uint16_t*>(x);
  a.w = w;
  a.scale = scale;
  a.pos = nullptr;
  a.y0 = a.y1 = a.y2 = static_cast<uint16_t*>(y);
  a.M = M;
  a.K = K;
  a.N = a.n1 = a.n2 = N;
  a.rope_end = 0;
  hipError_t e;
  {
    KernelMark m(&thread_profiler(), DUO_KERNEL_LINEAR, as_stream(hip_stream));
    e = duo::launch_w8(a, as_stream(hip_stream));
  }
  if (e != hipSuccess) return hip_fail(e, "linear_w8");
  return ok();
}

int duo_qkv_rope_w8(const void* x, int64_t M, int32_t hidden, const int64_t* positions, const int8_t* w_qkv,
                    const float* scale, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float rope_base,
                    void* q, void* k, void* v, void* hip_stream) {
  if (head_dim != 128) return fail(DUO_E_UNSUPPORTED, "head_dim must be 128");
  if (n_q_heads < 1 || n_kv_heads < 1 || n_q_heads > 4096 || n_kv_heads > 4096)
    return fail(DUO_E_INVALID, "head counts out of range");
  if (!(rope_base > 1.0f) || !std::isfinite(rope_base)) return fail(DUO_E_INVALID, "rope_base must be > 1");
  const int32_t N = (n_q_heads + 2 * n_kv_heads) * head_dim;
  int rc = check_w8(x, M, hidden, w_qkv, scale, N);
  if (rc || (rc = check_ptr(q, "q")) || (rc = check_ptr(k, "k")) || (rc = check_ptr(v, "v"))) return rc;
  if (!positions) return fail(DUO_E_INVALID, "positions is NULL");
  if (reinterpret_cast<uintptr_t>(positions) % 8) return fail(DUO_E_INVALID, "positions is not 8-byte aligned");
  duo::W8Args a{};
  a.x = static_cast<const uint16_t*>(x);
  a.w = w_qkv;
  a.scale = scale;
  a.pos = positions;
  a.y0 = static_cast<uint16_t*>(q);
  a.y1 = static_cast<uint16_t*>(k);
  a.y2 = static_cast<uint16_t*>(v);
  a.M = M;
  a.K = hidden;
  a.N = N;
  a.n1 = n_q_heads * head_dim;
  a.n2 = (n_q_heads + n_kv_heads) * head_dim;
  a.rope_end = a.n2;
  for (int j = 0; j < 6; ++j) a.theta_pow[j] = std::pow(static_cast<double>(rope_base), -double(1 << j) / 64.0);
  hipError_t e;
  {
    KernelMark m(&thread_profiler(), DUO_KERNEL_QKV_ROPE, as_stream(hip_stream));
    e = duo::launch_w8(a, as_stream(hip_stream));
  }
  if (e != hipSuccess) return hip_fail(e, "qkv_rope_w8");
  return ok();
}

}  // extern "C"
