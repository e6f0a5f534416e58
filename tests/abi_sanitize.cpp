// Host-side checks of libkvr's C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer.  The library sources are compiled with both
// sanitizers on their host side (the device code is built but never runs
// here); this driver calls every entry
// point with arguments that must be rejected before any device work, and a
// few that reach the HIP runtime (which, without a GPU, reports an error
// that the library must turn into KVR_ERR_HIP).  Pointers are fake, aligned
// addresses that the host side must never dereference.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "kvr.h"

namespace {

int g_checks = 0, g_fails = 0;

void check(int got, int want, const char* what, int line) {
  ++g_checks;
  if (got != want) {
    std::fprintf(stderr, "abi_sanitize.cpp:%d: %s returned %d, expected %d (%s)\n", line, what,
                 got, want, kvr_last_error());
    ++g_fails;
  }
}
#define CHECK(expr, want) check(static_cast<int>(expr), (want), #expr, __LINE__)

void* fake(uintptr_t off = 0) { return reinterpret_cast<void*>((uintptr_t{1} << 20) + off); }
template <class T> T* fk(uintptr_t off = 0) { return static_cast<T*>(fake(off)); }

kvr_config cfg(int head_dim = 64, int hq = 4, int hkv = 2, int hidden = 256, int inter = 512,
               kvr_dtype dt = KVR_F32) {
  kvr_config c{};
  c.hidden = hidden;
  c.n_q_heads = hq;
  c.n_kv_heads = hkv;
  c.head_dim = head_dim;
  c.intermediate = inter;
  c.rms_eps = 1e-6f;
  c.rope_theta = 1e6;
  c.alpha = -1.f;
  c.beta = -2.f;
  c.dtype = dt;
  return c;
}

kvr_layer_weights weights() {
  kvr_layer_weights w{};
  w.attn_norm = fake(0x100);
  w.wq = fake(0x200);
  w.wk = fake(0x300);
  w.wv = fake(0x400);
  w.wo = fake(0x500);
  w.mlp_norm = fake(0x600);
  w.w_gate = fake(0x700);
  w.w_up = fake(0x800);
  w.w_down = fake(0x900);
  return w;
}

void layer_and_stack() {
  kvr_config c = cfg();
  kvr_layer_weights w = weights();
  kvr_kv kv{fake(0x1000), fake(0x2000)};
  kvr_meta meta{fk<uint8_t>(0x3000), nullptr, nullptr, 512};
  const int32_t* T = fk<int32_t>(0x4000);
  const float* x = fk<float>(0x5000);
  float* y = fk<float>(0x6000);
  auto layer = [&](const kvr_config* cc, const kvr_layer_weights* ww, int B, int rows,
                   size_t ws, const kvr_meta* mm) {
    return kvr_layer_repair(cc, ww, kv, mm, T, B, x, rows, y, fake(0x7000), ws, nullptr);
  };
  const size_t big = size_t{1} << 40;
  CHECK(layer(nullptr, &w, 4, 4, big, &meta), KVR_ERR_INVALID_ARGUMENT);
  for (int hd : {0, 32, 96, 256}) {
    kvr_config b = cfg(hd);
    CHECK(layer(&b, &w, 4, 4, big, &meta), KVR_ERR_UNSUPPORTED);
  }
  {
    kvr_config b = cfg(64, 5, 2);
    CHECK(layer(&b, &w, 4, 4, big, &meta), KVR_ERR_UNSUPPORTED);
    b = cfg(64, 4, 2, 200);
    CHECK(layer(&b, &w, 4, 4, big, &meta), KVR_ERR_UNSUPPORTED);
    b = cfg(64, 4, 2, 256, 500);
    CHECK(layer(&b, &w, 4, 4, big, &meta), KVR_ERR_UNSUPPORTED);
    b = cfg(64, 4, 2, 16384);
    CHECK(layer(&b, &w, 4, 4, big, &meta), KVR_ERR_UNSUPPORTED);
    b = cfg(64, 0, 2);
    CHECK(layer(&b, &w, 4, 4, big, &meta), KVR_ERR_INVALID_ARGUMENT);
    b = cfg();
    b.alpha = std::numeric_limits<float>::quiet_NaN();
    CHECK(layer(&b, &w, 4, 4, big, &meta), KVR_ERR_INVALID_ARGUMENT);
    b = cfg();
    b.beta = std::numeric_limits<float>::infinity();
    CHECK(layer(&b, &w, 4, 4, big, &meta), KVR_ERR_INVALID_ARGUMENT);
    b = cfg();
    b.rms_eps = -1.f;
    CHECK(layer(&b, &w, 4, 4, big, &meta), KVR_ERR_INVALID_ARGUMENT);
    b = cfg();
    b.rope_theta = 0.0;
    CHECK(layer(&b, &w, 4, 4, big, &meta), KVR_ERR_INVALID_ARGUMENT);
    b = cfg();
    b.dtype = static_cast<kvr_dtype>(9);
    CHECK(layer(&b, &w, 4, 4, big, &meta), KVR_ERR_INVALID_ARGUMENT);
  }
  CHECK(layer(&c, &w, -1, 4, big, &meta), KVR_ERR_INVALID_ARGUMENT);
  CHECK(layer(&c, &w, 600, 600, big, &meta), KVR_ERR_INVALID_ARGUMENT);
  CHECK(layer(&c, &w, 4, 7, big, &meta), KVR_ERR_INVALID_ARGUMENT);
  CHECK(layer(&c, &w, 4, 4, 1024, &meta), KVR_ERR_WORKSPACE);
  CHECK(layer(&c, &w, 0, 0, big, &meta), KVR_OK);
  CHECK(layer(&c, &w, 4, 4, big, nullptr), KVR_ERR_INVALID_ARGUMENT);
  {
    kvr_layer_weights b = w;
    b.wq = nullptr;
    CHECK(layer(&c, &b, 4, 4, big, &meta), KVR_ERR_INVALID_ARGUMENT);
    b = w;
    b.w_down = fake(0x901);   // misaligned
    CHECK(layer(&c, &b, 4, 4, big, &meta), KVR_ERR_INVALID_ARGUMENT);
    b = w;
    b.bq = fake(0xA00);       // one bias without the others
    CHECK(layer(&c, &b, 4, 4, big, &meta), KVR_ERR_INVALID_ARGUMENT);
    b.bk = fake(0xB00);
    b.bv = fake(0xC04);       // all three, one misaligned
    CHECK(layer(&c, &b, 4, 4, big, &meta), KVR_ERR_INVALID_ARGUMENT);
  }
  {
    kvr_meta m2 = meta;
    m2.gpos = fk<int32_t>(0x8004);   // misaligned position map
    CHECK(layer(&c, &w, 4, 4, 1024, &m2), KVR_ERR_INVALID_ARGUMENT);
    m2 = meta;
    m2.n_tokens = 0;
    CHECK(layer(&c, &w, 0, 0, big, &m2), KVR_ERR_INVALID_ARGUMENT);
  }
  // gather into the input buffer itself
  CHECK(kvr_layer_repair(&c, &w, kv, &meta, T, 4, x, 512, const_cast<float*>(x), fake(0x7000),
                         big, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  // stack: n_layers, arrays, per-layer checks
  kvr_layer_weights ws[3] = {w, w, w};
  kvr_kv kvs[3] = {kv, kv, kv};
  CHECK(kvr_stack_repair(&c, 0, ws, kvs, &meta, T, 4, x, 4, y, fake(0x7000), big, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_stack_repair(&c, 3, nullptr, kvs, &meta, T, 4, x, 4, y, fake(0x7000), big, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  ws[2].w_up = nullptr;
  CHECK(kvr_stack_repair(&c, 3, ws, kvs, &meta, T, 4, x, 4, y, fake(0x7000), big, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  ws[2] = w;
  kvs[1].v = fake(0x2008);
  CHECK(kvr_stack_repair(&c, 3, ws, kvs, &meta, T, 4, x, 4, y, fake(0x7000), big, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
}

void workspace_sizes() {
  // the layout arithmetic for the workload shapes (no device involved)
  struct S { int hd, hq, hkv, hidden, inter; kvr_dtype dt; int B, N; } shapes[] = {
      {64, 4, 2, 256, 512, KVR_F32, 24, 512},        {128, 12, 2, 1536, 8960, KVR_BF16, 240, 4096},
      {128, 28, 4, 3584, 18944, KVR_BF16, 756, 16384}, {128, 28, 4, 3584, 18944, KVR_BF16, 646, 32768},
      {128, 12, 2, 1536, 8960, KVR_BF16, 16128, 16384}, {128, 32, 8, 4096, 12288, KVR_BF16, 64, 8192},
      {64, 8, 2, 256, 512, KVR_BF16, 1, 1},           {128, 28, 4, 3584, 18944, KVR_BF16, 0, 16}};
  for (const S& s : shapes) {
    kvr_config c = cfg(s.hd, s.hq, s.hkv, s.hidden, s.inter, s.dt);
    ++g_checks;
    const size_t a = kvr_workspace_bytes(&c, s.B, s.N);
    const size_t b = kvr_attention_workspace_bytes(&c, s.B, s.N);
    if (a == 0 || b == 0) {
      std::fprintf(stderr, "workspace sizes for B=%d N=%d: %zu, %zu\n", s.B, s.N, a, b);
      ++g_fails;
    }
  }
  kvr_config c = cfg();
  CHECK(kvr_workspace_bytes(&c, 600, 512) == 0, 1);
  CHECK(kvr_workspace_bytes(&c, -1, 512) == 0, 1);
  CHECK(kvr_workspace_bytes(nullptr, 1, 512) == 0, 1);
  CHECK(kvr_attention_workspace_bytes(&c, 1, 0) == 0, 1);
}

void index_calls() {
  kvr_repair_set out{fk<int32_t>(0x100), fk<int32_t>(0x200), fk<int32_t>(0x300),
                     fk<int32_t>(0x400), 16};
  const int32_t* s = fk<int32_t>(0x500);
  const int32_t* e = fk<int32_t>(0x600);
  CHECK(kvr_build_repair_set(s, e, 0, 8, 1, 1, nullptr, &out, nullptr, nullptr), KVR_ERR_BAD_BLOCKS);
  CHECK(kvr_build_repair_set(s, e, 2, 0, 1, 1, nullptr, &out, nullptr, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_build_repair_set(s, e, 2, 8, -1, 1, nullptr, &out, nullptr, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_build_repair_set(s, e, 2, 8, 1, 8, nullptr, &out, nullptr, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_build_repair_set(nullptr, e, 2, 8, 1, 1, nullptr, &out, nullptr, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_build_repair_set(s, e, 2, 8, 1, 3, nullptr, &out, nullptr, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  kvr_meta bad{fk<uint8_t>(0x700), nullptr, nullptr, 9};
  CHECK(kvr_build_repair_set(s, e, 2, 8, 1, 3, &bad, &out, nullptr, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  kvr_repair_set neg = out;
  neg.cap = -1;
  CHECK(kvr_build_repair_set(s, e, 2, 8, 1, 1, nullptr, &neg, nullptr, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  // a valid request reaches the HIP runtime, which has no GPU here
  int32_t h[3] = {0, 0, 0};
  CHECK(kvr_build_repair_set(s, e, 2, 8, 1, 1, nullptr, &out, h, nullptr), KVR_ERR_HIP);

  CHECK(kvr_check_support(fk<int32_t>(), 5, 4, 0, nullptr, fk<int32_t>(0x40), nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_check_support(fk<int32_t>(), 1, 4, 0, nullptr, nullptr, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_check_support(fk<int32_t>(), 1, 4, 0, fk<int32_t>(0x44), fk<int32_t>(0x80), nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_check_support(fk<int32_t>(), 1, 4, 0, nullptr, fk<int32_t>(0x80), nullptr), KVR_ERR_HIP);

  kvr_repair_set runs{nullptr, fk<int32_t>(0x200), fk<int32_t>(0x300), fk<int32_t>(0x400), 16};
  CHECK(kvr_build_runs(fk<int32_t>(), -1, 8, 0, &runs, nullptr, nullptr), KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_build_runs(fk<int32_t>(), 9, 8, 0, &runs, nullptr, nullptr), KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_build_runs(nullptr, 4, 8, 0, &runs, nullptr, nullptr), KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_build_runs(fk<int32_t>(4), 4, 8, 0, &runs, nullptr, nullptr), KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_build_runs(fk<int32_t>(), 17, 40, 0, &runs, nullptr, nullptr), KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_build_runs(fk<int32_t>(), 4, 8, 0, nullptr, nullptr, nullptr), KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_build_runs(fk<int32_t>(), 4, 8, 0, &runs, h, nullptr), KVR_ERR_HIP);

  CHECK(kvr_build_plan(fk<int32_t>(), 4, 0, fk<int32_t>(0x40), fk<int32_t>(0x80), nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_build_plan(fk<int32_t>(), 0, 7, fk<int32_t>(0x40), fk<int32_t>(0x80), nullptr), KVR_OK);
  CHECK(kvr_build_plan(fk<int32_t>(), 4, 7, nullptr, fk<int32_t>(0x80), nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_build_tile_map(fk<int32_t>(), 5, 4, fk<int32_t>(0x40), nullptr), KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_build_tile_map(fk<int32_t>(), 0, 0, fk<int32_t>(0x40), nullptr), KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_build_tile_map(fk<int32_t>(), 3, 40, nullptr, nullptr), KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_build_tile_map(fk<int32_t>(4), 3, 40, fk<int32_t>(0x40), nullptr), KVR_ERR_INVALID_ARGUMENT);
}

void attention_calls() {
  kvr_config c = cfg(128, 28, 4, 3584, 18944, KVR_BF16);
  kvr_kv kv{fake(0x1000), fake(0x2000)};
  const uint8_t* f = fk<uint8_t>(0x3000);
  const float* q = fk<float>(0x4000);
  const int32_t* pos = fk<int32_t>(0x5000);
  float* o = fk<float>(0x6000);
  const size_t big = size_t{1} << 40;
  CHECK(kvr_biased_attention(&c, kv, f, 16384, q, pos, 1, o, fake(0x7000), 16, nullptr),
        KVR_ERR_WORKSPACE);
  CHECK(kvr_biased_attention(&c, kv, f, 16384, q, pos, -1, o, fake(0x7000), big, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_biased_attention(&c, kv, f, 16384, q, pos, 16385, o, fake(0x7000), big, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_biased_attention(&c, kv, f, 16384, q, pos, 1, const_cast<float*>(q), fake(0x7000), big,
                             nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_biased_attention(&c, kv, f, 16384, q, pos, 1, o, nullptr, big, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_biased_attention(&c, kv, f, 0, q, pos, 0, o, fake(0x7000), big, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_biased_attention(&c, kv, f, 16384, q, pos, 0, o, fake(0x7000), big, nullptr), KVR_OK);
  // the allocation-free variant: same checks, then its scratch limit, then
  // the runtime (no GPU here)
  CHECK(kvr_biased_attention_noalloc(&c, kv, f, 16384, q, pos, -1, o, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_biased_attention_noalloc(&c, kv, f, 16384, q, pos, 1, const_cast<float*>(q), nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_biased_attention_noalloc(&c, kv, f, 16384, q, pos, 64, o, nullptr), KVR_ERR_WORKSPACE);
  CHECK(kvr_biased_attention_noalloc(&c, kv, f, 16384, q, pos, 1, o, nullptr), KVR_ERR_HIP);
}

void shift_and_sur_calls() {
  kvr_config c = cfg(128, 28, 4, 3584, 18944, KVR_BF16);
  kvr_kv src[2] = {{fake(0x100000), fake(0x200000)}, {fake(0x300000), fake(0x400000)}};
  kvr_kv dst[2] = {{fake(0x500000), fake(0x600000)}, {fake(0x700000), fake(0x800000)}};
  const int N = 16;
  CHECK(kvr_shift_cache(&c, 0, src, dst, nullptr, nullptr, nullptr, nullptr, N, 2, 3, 0, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_shift_cache(&c, 2, src, dst, nullptr, nullptr, nullptr, nullptr, N, 10, 7, 0, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_shift_cache(&c, 2, src, dst, fk<uint8_t>(0x900000), nullptr, nullptr, nullptr, N, 2, 3,
                        0, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  kvr_kv overlap[2] = {{fake(0x100000 + 256), fake(0x600000)}, {fake(0x700000), fake(0x800000)}};
  CHECK(kvr_shift_cache(&c, 2, src, overlap, nullptr, nullptr, nullptr, nullptr, N, 2, 3, 0, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  kvr_config t = c;
  t.rope_theta = -1.0;
  CHECK(kvr_shift_cache(&t, 2, src, dst, nullptr, nullptr, nullptr, nullptr, N, 2, 3, 0, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_shift_cache(&c, 2, src, dst, nullptr, nullptr, nullptr, nullptr, N, 0, N, 0, nullptr),
        KVR_OK);   // everything deleted: nothing to move

  const int32_t* ids = fk<int32_t>(0x1000);
  float* r = fk<float>(0x2000);
  CHECK(kvr_sur_scores(fake(), KVR_BF16, 0, 256, ids, 4, ids, 2, r, nullptr), KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_sur_scores(fake(), KVR_BF16, 10, 256, ids, 4, ids, 0, r, nullptr), KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_sur_scores(fake(), KVR_BF16, 10, 256, ids, 4, ids, 257, r, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_sur_scores(fake(), KVR_BF16, 10, 100, ids, 4, ids, 2, r, nullptr), KVR_ERR_UNSUPPORTED);
  CHECK(kvr_sur_scores(fake(), KVR_F32, 10, 8256, ids, 4, ids, 2, r, nullptr), KVR_ERR_UNSUPPORTED);
  CHECK(kvr_sur_scores(fake(), KVR_BF16, 10, 256, ids, 0, ids, 2, r, nullptr), KVR_OK);
  kvr_repair_set out{fk<int32_t>(0x100), fk<int32_t>(0x200), fk<int32_t>(0x300), fk<int32_t>(0x400),
                     8};
  float* us = fk<float>(0x3000);
  float* wsf = fk<float>(0x4000);
  CHECK(kvr_sur_select(r, 0, ids, 1, 0, 0, us, &out, wsf, 1 << 20, nullptr, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_sur_select(r, 100, ids, 101, 4, 0, us, &out, wsf, 1 << 20, nullptr, nullptr),
        KVR_ERR_INVALID_ARGUMENT);
  CHECK(kvr_sur_select(r, 100, ids, 4, 9, 0, us, &out, wsf, 1 << 20, nullptr, nullptr),
        KVR_ERR_INVALID_ARGUMENT);   // cap < budget
  CHECK(kvr_sur_select(r, 100, ids, 4, 4, 0, us, &out, wsf, 16, nullptr, nullptr), KVR_ERR_WORKSPACE);
  CHECK(kvr_sur_select(r, 20000, ids, 9000, 4, 0, us, &out, wsf, 1 << 20, nullptr, nullptr),
        KVR_ERR_UNSUPPORTED);
}

void misc_calls() {
  for (int s = -7; s <= 0; ++s) {
    ++g_checks;
    const char* name = kvr_status_string(static_cast<kvr_status>(s));
    if (!name || std::strncmp(name, "KVR_", 4) != 0) ++g_fails;
  }
  ++g_checks;
  if (std::strcmp(kvr_status_string(static_cast<kvr_status>(5)), "KVR_UNKNOWN_STATUS") != 0) ++g_fails;
  CHECK(kvr_timing_begin(0xFFFFFFFFu), KVR_OK);
  double ms[KVR_KERNEL_COUNT];
  int32_t n[KVR_KERNEL_COUNT];
  CHECK(kvr_timing_end(ms, n), KVR_OK);
  CHECK(kvr_timing_end(nullptr, nullptr), KVR_OK);
}

}  // namespace

int main() {
  layer_and_stack();
  workspace_sizes();
  index_calls();
  attention_calls();
  shift_and_sur_calls();
  misc_calls();
  std::printf("%d checks, %d failed\n", g_checks, g_fails);
  return g_fails == 0 ? 0 : 1;
}
