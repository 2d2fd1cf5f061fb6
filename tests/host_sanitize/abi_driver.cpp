// Exercises every argument-validation path of libduo_attn's C ABI that returns before
// any HIP call, so it runs on a host without a GPU.  Built with AddressSanitizer and
// UndefinedBehaviorSanitizer over the library's host code (tests/test_host_sanitize.py);
// any sanitizer report or an unexpected return code fails the run.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/duo_attn.h"
#include "../../include/duo_linear.h"
#include "../../include/duo_profile.h"
#include "../../include/duo_synth.h"

static int g_fail = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    std::printf("FAIL %s: got %d want %d (%s)\n", what, got, want, duo_last_error());
    ++g_fail;
  } else if (got != DUO_OK && std::strlen(duo_last_error()) == 0) {
    std::printf("FAIL %s: error %d without a message\n", what, got);
    ++g_fail;
  }
}

struct Cfg {
  std::vector<uint8_t> mask;
  duo_config c;
  Cfg() : mask{1, 0, 1, 0, 0, 0, 1, 1} {
    std::memset(&c, 0, sizeof(c));
    c.n_layers = 2;
    c.batch = 1;
    c.n_q_heads = 8;
    c.n_kv_heads = 4;
    c.head_dim = 128;
    c.sink = 4;
    c.recent = 16;
    c.io_dtype = DUO_DTYPE_BF16;
    c.kv_format = DUO_KV_SAME_AS_IO;
    c.max_context = 1000;
    c.retrieval_mask = mask.data();
  }
};

int main() {
  uint64_t bytes = 0;
  {
    Cfg k;
    expect(duo_kv_bytes(&k.c, &bytes), DUO_OK, "kv_bytes ok");
    expect(duo_kv_bytes(&k.c, nullptr), DUO_E_INVALID, "kv_bytes null out");
    expect(duo_kv_bytes(nullptr, &bytes), DUO_E_INVALID, "kv_bytes null cfg");
  }
  // one bad field at a time
  struct Bad { const char* name; void (*edit)(duo_config&); int want; };
  const Bad bad[] = {
      {"n_layers 0", [](duo_config& c) { c.n_layers = 0; }, DUO_E_INVALID},
      {"batch 0", [](duo_config& c) { c.batch = 0; }, DUO_E_INVALID},
      {"q heads not a multiple", [](duo_config& c) { c.n_q_heads = 6; }, DUO_E_INVALID},
      {"group above 16", [](duo_config& c) { c.n_q_heads = 4 * 17; }, DUO_E_UNSUPPORTED},
      {"head_dim 96", [](duo_config& c) { c.head_dim = 96; }, DUO_E_UNSUPPORTED},
      {"sink < 0", [](duo_config& c) { c.sink = -1; }, DUO_E_INVALID},
      {"recent 0", [](duo_config& c) { c.recent = 0; }, DUO_E_INVALID},
      {"sink above bound", [](duo_config& c) { c.sink = DUO_MAX_WINDOW + 1; }, DUO_E_UNSUPPORTED},
      {"recent at int32 max", [](duo_config& c) { c.recent = 0x7fffffff; }, DUO_E_UNSUPPORTED},
      {"max_context 0", [](duo_config& c) { c.max_context = 0; }, DUO_E_INVALID},
      {"max_context huge", [](duo_config& c) { c.max_context = int64_t(1) << 50; }, DUO_E_INVALID},
      {"io dtype", [](duo_config& c) { c.io_dtype = 7; }, DUO_E_INVALID},
      {"kv format", [](duo_config& c) { c.kv_format = 3; }, DUO_E_INVALID},
      {"int4 with fp32", [](duo_config& c) { c.kv_format = DUO_KV_INT4_G128; c.io_dtype = DUO_DTYPE_F32; }, DUO_E_UNSUPPORTED},
      {"reserved", [](duo_config& c) { c.reserved = 1; }, DUO_E_INVALID},
      {"scale nan", [](duo_config& c) { c.scale = __builtin_nanf(""); }, DUO_E_INVALID},
      {"scale negative", [](duo_config& c) { c.scale = -1.0f; }, DUO_E_INVALID},
      {"mask null", [](duo_config& c) { c.retrieval_mask = nullptr; }, DUO_E_INVALID},
  };
  for (const Bad& b : bad) {
    Cfg k;
    b.edit(k.c);
    expect(duo_kv_bytes(&k.c, &bytes), b.want, b.name);
    duo_handle* h = nullptr;
    expect(duo_kv_init(&k.c, reinterpret_cast<void*>(4096), uint64_t(1) << 40, nullptr, &h), b.want, b.name);
    if (h) { std::printf("FAIL %s: handle returned\n", b.name); ++g_fail; }
  }
  {
    Cfg k;
    k.mask[3] = 2;
    expect(duo_kv_bytes(&k.c, &bytes), DUO_E_INVALID, "mask entry 2");
  }
  {  // the largest windows: layout arithmetic in range
    Cfg k;
    k.c.sink = DUO_MAX_WINDOW;
    k.c.recent = DUO_MAX_WINDOW;
    k.c.max_context = 64;
    expect(duo_kv_bytes(&k.c, &bytes), DUO_OK, "largest window");
  }
  {  // workspace checks happen before any device work
    Cfg k;
    uint64_t need = 0;
    duo_kv_bytes(&k.c, &need);
    duo_handle* h = nullptr;
    expect(duo_kv_init(&k.c, reinterpret_cast<void*>(4096), need - 1, nullptr, &h), DUO_E_CAPACITY, "small ws");
    expect(duo_kv_init(&k.c, reinterpret_cast<void*>(4096 + 16), need, nullptr, &h), DUO_E_INVALID, "misaligned ws");
    expect(duo_kv_init(&k.c, nullptr, need, nullptr, &h), DUO_E_INVALID, "null ws");
    expect(duo_kv_init(&k.c, reinterpret_cast<void*>(4096), need, nullptr, nullptr), DUO_E_INVALID, "null out");
    // an injected fault fails the call after validation, before any HIP call
    setenv("DUO_FAULT_INJECT", "duo_prefill,duo_kv_init", 1);
    expect(duo_kv_init(&k.c, reinterpret_cast<void*>(4096), need, nullptr, &h), DUO_E_HIP, "injected init fault");
    if (h) { std::printf("FAIL injected init fault: handle returned\n"); ++g_fail; }
    expect(duo_kv_init(&k.c, reinterpret_cast<void*>(4096), need - 1, nullptr, &h), DUO_E_CAPACITY,
           "validation before the injected fault");
    unsetenv("DUO_FAULT_INJECT");
    // resume over a saved workspace: lengths are checked before anything else happens
    std::vector<int64_t> lens(size_t(k.c.n_layers) * k.c.batch, 3);
    expect(duo_kv_attach(&k.c, reinterpret_cast<void*>(4096), need, nullptr, &h), DUO_E_INVALID, "attach null lengths");
    lens[1] = k.c.max_context + 1;
    expect(duo_kv_attach(&k.c, reinterpret_cast<void*>(4096), need, lens.data(), &h), DUO_E_INVALID,
           "attach length past max_context");
    lens[1] = 3;
    expect(duo_kv_attach(&k.c, reinterpret_cast<void*>(4096), need - 1, lens.data(), &h), DUO_E_CAPACITY,
           "attach small ws");
    if (h) { std::printf("FAIL attach: handle returned\n"); ++g_fail; }
  }
  // calls on a NULL handle
  void* p = reinterpret_cast<void*>(4096);
  int64_t n = 0;
  float* fp = reinterpret_cast<float*>(4096);
  expect(duo_prefill(nullptr, 0, p, p, p, 4, p, nullptr), DUO_E_INVALID, "prefill null handle");
  expect(duo_prefill_dual(nullptr, 0, p, p, p, 4, p, p, nullptr), DUO_E_INVALID, "dual null handle");
  expect(duo_kv_append(nullptr, 0, p, p, 4, nullptr), DUO_E_INVALID, "append null handle");
  expect(duo_decode(nullptr, 0, p, p, p, p, nullptr), DUO_E_INVALID, "decode null handle");
  expect(duo_decode_static(nullptr, 0, p, p, p, p, nullptr), DUO_E_INVALID, "decode_static null handle");
  expect(duo_kv_length(nullptr, 0, &n), DUO_E_INVALID, "length null handle");
  expect(duo_prefill_seq(nullptr, 0, 0, p, p, p, 4, p, nullptr), DUO_E_INVALID, "prefill_seq null handle");
  expect(duo_kv_append_seq(nullptr, 0, 0, p, p, 4, nullptr), DUO_E_INVALID, "append_seq null handle");
  expect(duo_kv_length_seq(nullptr, 0, 0, &n), DUO_E_INVALID, "length_seq null handle");
  expect(duo_kv_read(nullptr, 0, 0, 0, 0, 0, 1, fp, nullptr), DUO_E_INVALID, "read null handle");
  expect(duo_kv_read_int4(nullptr, 0, 0, 0, 0, 0, 1, reinterpret_cast<uint8_t*>(4096),
                          reinterpret_cast<uint16_t*>(4096), nullptr),
         DUO_E_INVALID, "read_int4 null handle");
  int32_t nb = 0;
  expect(duo_kv_guard_bands(nullptr, nullptr, 0, &nb), DUO_E_INVALID, "guard_bands null handle");
  expect(duo_profile_enable(nullptr, 1), DUO_E_INVALID, "profile_enable null handle");
  double ms[DUO_KERNEL_CLASSES];
  int64_t cnt[DUO_KERNEL_CLASSES];
  expect(duo_profile_collect(nullptr, ms, cnt), DUO_E_INVALID, "profile_collect null handle");
  duo_kv_free(nullptr);
  // handle-free calls
  expect(duo_synth_fill(nullptr, DUO_DTYPE_BF16, 1, 0, 0, 10, nullptr), DUO_E_INVALID, "synth null");
  expect(duo_synth_fill(reinterpret_cast<void*>(4098), DUO_DTYPE_BF16, 1, 0, 0, 10, nullptr), DUO_E_INVALID,
         "synth misaligned");
  expect(duo_synth_fill(p, 5, 1, 0, 0, 10, nullptr), DUO_E_INVALID, "synth dtype");
  expect(duo_synth_fill(p, DUO_DTYPE_BF16, uint64_t(1) << 40, 0, 0, 10, nullptr), DUO_E_INVALID, "synth seed");
  const int8_t* w = reinterpret_cast<const int8_t*>(4096);
  expect(duo_linear_w8(p, 0, 4096, w, fp, 4096, p, nullptr), DUO_E_INVALID, "linear M 0");
  expect(duo_linear_w8(p, 4, 100, w, fp, 4096, p, nullptr), DUO_E_UNSUPPORTED, "linear K");
  expect(duo_linear_w8(p, 4, 4096, w, fp, 100, p, nullptr), DUO_E_UNSUPPORTED, "linear N");
  expect(duo_linear_w8(nullptr, 4, 4096, w, fp, 4096, p, nullptr), DUO_E_INVALID, "linear null x");
  expect(duo_qkv_rope_w8(p, 4, 4096, reinterpret_cast<const int64_t*>(4096), w, fp, 32, 8, 64, 1e4f, p, p, p,
                         nullptr),
         DUO_E_UNSUPPORTED, "qkv head_dim");
  expect(duo_qkv_rope_w8(p, 4, 4096, reinterpret_cast<const int64_t*>(4096), w, fp, 32, 8, 128, 0.5f, p, p, p,
                         nullptr),
         DUO_E_INVALID, "qkv rope base");
  expect(duo_qkv_rope_w8(p, 4, 4096, nullptr, w, fp, 32, 8, 128, 1e4f, p, p, p, nullptr), DUO_E_INVALID,
         "qkv null positions");
  expect(duo_profile_thread_collect(nullptr, cnt), DUO_E_INVALID, "thread collect null");
  std::printf("%s: %d failure(s)\n", g_fail ? "FAILED" : "ok", g_fail);
  return g_fail ? 1 : 0;
}
