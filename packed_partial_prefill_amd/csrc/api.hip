// Host side of libkvr: the extern "C" entry points declared in kvr.h.
// Validates arguments before touching the device, carves the caller's
// workspace, and enqueues the per-layer kernel sequence on the caller's
// stream (no synchronisation, no device allocation).
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "kvr_internal.h"

namespace {

thread_local char g_err[512] = "";

kvr_status fail(kvr_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

kvr_status hip_fail(hipError_t e, const char* what) {
  return fail(KVR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dev_ok(const void* p) { return p != nullptr && aligned16(p); }

// ---------------------------------------------------------------- timing
struct Timing {
  uint32_t mask = 0;
  std::vector<hipEvent_t> ev;  // pairs
  std::vector<int> id;
  size_t used = 0;
} g_timing;

struct Launch {
  int id;
  hipStream_t stream;
  bool on;
  Launch(int kernel_id, hipStream_t s) : id(kernel_id), stream(s), on(false) {
    if (!(g_timing.mask & (1u << kernel_id))) return;
    if (g_timing.used * 2 + 2 > g_timing.ev.size()) {
      hipEvent_t a, b;
      if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return;
      g_timing.ev.push_back(a);
      g_timing.ev.push_back(b);
      g_timing.id.push_back(-1);
    }
    g_timing.id[g_timing.used] = kernel_id;
    on = hipEventRecord(g_timing.ev[g_timing.used * 2], stream) == hipSuccess;
  }
  void done() {
    if (!on) return;
    hipEventRecord(g_timing.ev[g_timing.used * 2 + 1], stream);
    ++g_timing.used;
  }
};

#define KVR_RUN(kid, stream, what, expr)          \
  do {                                            \
    Launch _l((kid), (stream));                   \
    hipError_t _e = (expr);                       \
    _l.done();                                    \
    if (_e != hipSuccess) return hip_fail(_e, what); \
  } while (0)

// ---------------------------------------------------------------- config
// dtype and attention heads: what every entry point reads.
// The value of a dtype field as its bytes hold it: a C caller may store any
// int there, and reading a value outside the enumerators through the enum
// type is undefined in C++.
int raw_dtype(const kvr_dtype* p) {
  int v = 0;
  static_assert(sizeof(kvr_dtype) == sizeof(int), "kvr_dtype is int-sized");
  std::memcpy(&v, p, sizeof(v));
  return v;
}

kvr_status check_heads(const kvr_config* c, kvr::Shape* sh) {
  if (!c) return fail(KVR_ERR_INVALID_ARGUMENT, "cfg is NULL");
  const int dt = raw_dtype(&c->dtype);
  if (dt != KVR_F32 && dt != KVR_BF16)
    return fail(KVR_ERR_INVALID_ARGUMENT, "unknown dtype %d", dt);
  if (c->n_q_heads <= 0 || c->n_kv_heads <= 0)
    return fail(KVR_ERR_INVALID_ARGUMENT, "non-positive head counts");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(KVR_ERR_UNSUPPORTED, "head_dim %d (64 or 128 supported)", c->head_dim);
  if (c->n_q_heads % c->n_kv_heads)
    return fail(KVR_ERR_UNSUPPORTED, "n_q_heads %% n_kv_heads != 0");
  *sh = kvr::Shape{};
  sh->hq = c->n_q_heads;
  sh->hkv = c->n_kv_heads;
  sh->d = c->head_dim;
  sh->group = c->n_q_heads / c->n_kv_heads;
  return KVR_OK;
}

kvr_status check_config(const kvr_config* c, kvr::Shape* sh) {
  kvr_status st = check_heads(c, sh);
  if (st != KVR_OK) return st;
  if (c->hidden <= 0 || c->intermediate <= 0)
    return fail(KVR_ERR_INVALID_ARGUMENT, "non-positive shape");
  if (c->hidden % 64 || c->intermediate % 64)
    return fail(KVR_ERR_UNSUPPORTED, "hidden and intermediate must be multiples of 64");
  if (c->hidden > 8192) return fail(KVR_ERR_UNSUPPORTED, "hidden > 8192");
  if (!std::isfinite(c->alpha) || !std::isfinite(c->beta) || !std::isfinite(c->rms_eps) ||
      c->rms_eps < 0.f)
    return fail(KVR_ERR_INVALID_ARGUMENT, "alpha, beta and rms_eps must be finite (eps >= 0)");
  if (!std::isfinite(c->rope_theta) || c->rope_theta <= 0.0)
    return fail(KVR_ERR_INVALID_ARGUMENT, "rope_theta must be finite and positive");
  sh->hidden = c->hidden;
  sh->hq = c->n_q_heads;
  sh->hkv = c->n_kv_heads;
  sh->d = c->head_dim;
  sh->inter = c->intermediate;
  sh->group = c->n_q_heads / c->n_kv_heads;
  return KVR_OK;
}

size_t esize(kvr_dtype dt) { return dt == KVR_BF16 ? 2 : 4; }

// Workspace layout; offsets are 256-byte aligned from an aligned base.
struct Layout {
  size_t tab, n_full, n_total, nbuf, part, q, o, mlp, attn, total;
  kvr::GemmPlan g_qkv, g_o, g_gateup, g_down;
};

size_t up256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

Layout layout_for(const kvr_config* c, const kvr::Shape& sh, int B, int n_tokens) {
  Layout L{};
  const size_t es = esize(c->dtype);
  const int nt = kvr::plan_tiles(B, sh.group);
  L.g_qkv = kvr::gemm_plan_for(c->dtype, B, sh.qkv_cols(), sh.hidden, false);
  L.g_o = kvr::gemm_plan_for(c->dtype, B, sh.hidden, sh.hq * sh.d, false);
  L.g_gateup = kvr::gemm_plan_for(c->dtype, B, sh.inter, sh.hidden, true);
  L.g_down = kvr::gemm_plan_for(c->dtype, B, sh.hidden, sh.inter, false);
  size_t part_floats = static_cast<size_t>(L.g_qkv.splits) * B * sh.qkv_cols();
  part_floats = std::max(part_floats, static_cast<size_t>(L.g_o.splits) * B * sh.hidden);
  part_floats = std::max(part_floats, static_cast<size_t>(L.g_down.splits) * B * sh.hidden);
  if (!L.g_gateup.fused)
    part_floats = std::max(part_floats, static_cast<size_t>(L.g_gateup.splits) * B * 2 * sh.inter);
  size_t off = 0;
  L.tab = off;     off = up256(off + static_cast<size_t>(B) * (sh.d / 2) * sizeof(float2));
  L.n_full = off;  off = up256(off + static_cast<size_t>(nt) * 4);
  L.n_total = off; off = up256(off + static_cast<size_t>(nt) * 4);
  L.nbuf = off;    off = up256(off + static_cast<size_t>(B) * sh.hidden * es);
  L.part = off;    off = up256(off + part_floats * 4);
  L.q = off;       off = up256(off + static_cast<size_t>(B) * sh.hq * sh.d * es);
  L.o = off;       off = up256(off + static_cast<size_t>(B) * sh.hq * sh.d * es);
  L.mlp = off;     off = up256(off + static_cast<size_t>(B) * sh.inter * es);
  L.attn = off;    off = up256(off + kvr::attention_workspace_bytes(c->dtype, B, n_tokens, sh));
  L.total = off;
  return L;
}

// Workspace of kvr_biased_attention: plan, scaled queries, split-KV partials.
struct AttnLayout {
  size_t n_full, n_total, q, attn, total;
};

AttnLayout attn_layout_for(const kvr_config* c, const kvr::Shape& sh, int B, int n_tokens) {
  AttnLayout L{};
  if (kvr::decode_supported(c->dtype, B, sh)) {   // few pairs: chunk partials only
    L.attn = 0;
    L.total = up256(kvr::decode_workspace_bytes(B, n_tokens, sh));
    return L;
  }
  const int nt = kvr::plan_tiles(B, sh.group);
  size_t off = 0;
  L.n_full = off;  off = up256(off + static_cast<size_t>(nt) * 4);
  L.n_total = off; off = up256(off + static_cast<size_t>(nt) * 4);
  L.q = off;
  if (c->dtype == KVR_BF16) off = up256(off + static_cast<size_t>(B) * sh.hq * sh.d * 2);
  L.attn = off;    off = up256(off + kvr::attention_workspace_bytes(c->dtype, B, n_tokens, sh));
  L.total = off;
  return L;
}

kvr_status check_weights(const kvr_layer_weights& w, int layer) {
  const void* req[] = {w.attn_norm, w.wq, w.wk, w.wv, w.wo, w.mlp_norm, w.w_gate, w.w_up, w.w_down};
  for (const void* p : req)
    if (!dev_ok(p)) return fail(KVR_ERR_INVALID_ARGUMENT, "layer %d: weight pointer NULL or not 16-byte aligned", layer);
  const int nb = (w.bq != nullptr) + (w.bk != nullptr) + (w.bv != nullptr);
  if (nb != 0 && nb != 3)
    return fail(KVR_ERR_INVALID_ARGUMENT, "layer %d: bq, bk, bv must be all NULL or all set", layer);
  if (nb == 3 && (!aligned16(w.bq) || !aligned16(w.bk) || !aligned16(w.bv)))
    return fail(KVR_ERR_INVALID_ARGUMENT, "layer %d: bias pointers not 16-byte aligned", layer);
  return KVR_OK;
}

// The device-side support check of kvr_check_support (also run first by the
// repair and attention entries in validation mode): launch, copy the result
// word back, synchronise, map it to a status.
kvr_status check_support_sync(const int32_t* d_T, int B, int n_tokens, int first_selectable,
                              const int32_t* d_gpos, int32_t* d_result, hipStream_t stream) {
  hipError_t e = kvr::launch_check_support(d_T, B, n_tokens, first_selectable, d_gpos, d_result,
                                           stream);
  if (e != hipSuccess) return hip_fail(e, "check support");
  int32_t h = 0;
  e = hipMemcpyAsync(&h, d_result, sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return hip_fail(e, "copy result");
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "synchronize");
  if (h == KVR_ERR_BAD_SUPPORT)
    return fail(KVR_ERR_BAD_SUPPORT, "support not strictly increasing or outside [%d, %d)",
                first_selectable, n_tokens);
  if (h != KVR_OK)
    return fail(KVR_ERR_INVALID_ARGUMENT,
                "global position map not non-negative and strictly increasing");
  return KVR_OK;
}

// Validation mode: KVR_VALIDATE set in the environment to anything but "0"
// (read on every call).  The repair and attention entries then check their
// support (and position map) on the device before any other launch, which
// synchronises the stream, and return the check's error instead of running.
bool validate_mode() {
  const char* v = std::getenv("KVR_VALIDATE");
  return v && v[0] && !(v[0] == '0' && v[1] == '\0');
}

kvr_status run_stack(const kvr_config* cfg, int n_layers, const kvr_layer_weights* w,
                     const kvr_kv* caches, const kvr_meta* meta, const int32_t* d_T, int B,
                     const float* x_in, int x_in_rows, float* x_out, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  g_err[0] = '\0';
  kvr::Shape sh;
  kvr_status st = check_config(cfg, &sh);
  if (st != KVR_OK) return st;
  if (n_layers < 1) return fail(KVR_ERR_INVALID_ARGUMENT, "n_layers must be >= 1");
  if (!w || !caches) return fail(KVR_ERR_INVALID_ARGUMENT, "weights / caches arrays are NULL");
  if (!meta) return fail(KVR_ERR_INVALID_ARGUMENT, "meta is NULL");
  const int N = meta->n_tokens;
  if (N <= 0) return fail(KVR_ERR_INVALID_ARGUMENT, "meta->n_tokens must be positive");
  if (B < 0 || B > N) return fail(KVR_ERR_INVALID_ARGUMENT, "B=%d outside [0, N=%d]", B, N);
  if (x_in_rows != B && x_in_rows != N)
    return fail(KVR_ERR_INVALID_ARGUMENT, "x_in_rows=%d must be B=%d or N=%d", x_in_rows, B, N);
  if (B == 0) return KVR_OK;
  if (!dev_ok(d_T) || !dev_ok(x_in) || !dev_ok(x_out) || !dev_ok(ws) || !dev_ok(meta->flags))
    return fail(KVR_ERR_INVALID_ARGUMENT, "T, x_in, x_out, ws and flags must be non-NULL and 16-byte aligned");
  if (meta->gpos && !aligned16(meta->gpos))
    return fail(KVR_ERR_INVALID_ARGUMENT, "meta->gpos not 16-byte aligned");
  const bool gather = (x_in_rows == N) && !(B == N);
  if (gather && x_in == x_out)
    return fail(KVR_ERR_INVALID_ARGUMENT, "x_out may alias x_in only when x_in_rows == B");
  for (int l = 0; l < n_layers; ++l) {
    if ((st = check_weights(w[l], l)) != KVR_OK) return st;
    if (!dev_ok(caches[l].k) || !dev_ok(caches[l].v))
      return fail(KVR_ERR_INVALID_ARGUMENT, "layer %d: cache pointers NULL or not 16-byte aligned", l);
  }
  const Layout L = layout_for(cfg, sh, B, N);
  uint8_t* base = reinterpret_cast<uint8_t*>(up256(reinterpret_cast<uintptr_t>(ws)));
  const size_t slack = static_cast<size_t>(base - static_cast<uint8_t*>(ws));
  if (ws_bytes < L.total + slack)
    return fail(KVR_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, L.total + slack);
  // (the result word borrows the plan's first slot, written after the check)
  if (validate_mode() &&
      (st = check_support_sync(d_T, B, N, 0, meta->gpos, reinterpret_cast<int32_t*>(base + L.n_full),
                               stream)) != KVR_OK)
    return st;

  const kvr_dtype dt = cfg->dtype;
  float2* tab = reinterpret_cast<float2*>(base + L.tab);
  int32_t* n_full = reinterpret_cast<int32_t*>(base + L.n_full);
  int32_t* n_total = reinterpret_cast<int32_t*>(base + L.n_total);
  void* nbuf = base + L.nbuf;
  float* part = reinterpret_cast<float*>(base + L.part);
  void* qbuf = base + L.q;
  void* obuf = base + L.o;
  void* mlp = base + L.mlp;
  void* attn_ws = base + L.attn;
  const int qkv_n = sh.qkv_cols();

  // gather the selected rows once; RMSNorm for layer 0; in the same launch,
  // once per call, the plan (Eq. 23-24) and the RoPE table for the fixed
  // positions
  const kvr::LayerTables tabs{d_T,     meta->gpos, B,       sh.group, kvr::plan_tiles(B, sh.group),
                              n_full,  n_total,    sh.d / 2, cfg->rope_theta, tab};
  KVR_RUN(KVR_KERNEL_NORM, stream, "gather+norm, plan and rope table",
          kvr::launch_gather_norm(dt, x_in, gather ? d_T : nullptr, x_out,
                                  static_cast<const float*>(w[0].attn_norm), cfg->rms_eps, nbuf, B,
                                  sh.hidden, &tabs, stream));
  for (int l = 0; l < n_layers; ++l) {
    const kvr_layer_weights& W = w[l];
    kvr::WeightSegs qkv{{W.wq, W.wk, W.wv},
                        {0, sh.hq * sh.d, (sh.hq + sh.hkv) * sh.d, qkv_n}, 3};
    KVR_RUN(KVR_KERNEL_QKV, stream, "qkv gemm",
            kvr::launch_gemm_partial(dt, nbuf, qkv, B, qkv_n, sh.hidden, L.g_qkv, part, stream));
    KVR_RUN(KVR_KERNEL_ROPE, stream, "rope+writeback",
            kvr::launch_rope_writeback(dt, part, L.g_qkv.splits, static_cast<size_t>(B) * qkv_n,
                                       static_cast<const float*>(W.bq),
                                       static_cast<const float*>(W.bk),
                                       static_cast<const float*>(W.bv), tab, d_T, B, sh,
                                       kvr::attention_q_scale(dt, sh.d), qbuf,
                                       caches[l].k, caches[l].v, meta->flags, stream));
    KVR_RUN(KVR_KERNEL_ATTN, stream, "attention",
            kvr::launch_attention(dt, qbuf, caches[l].k, caches[l].v, meta->flags, d_T, B, N, sh,
                                  cfg->alpha, cfg->beta, n_full, n_total, attn_ws, obuf, stream));
    if (kvr::attention_needs_merge(dt))
      KVR_RUN(KVR_KERNEL_ATTN_MERGE, stream, "attention merge",
              kvr::launch_attention_merge(dt, B, N, sh, n_total, attn_ws, obuf, false, stream));
    kvr::WeightSegs wo{{W.wo, nullptr, nullptr}, {0, sh.hidden, sh.hidden, sh.hidden}, 1};
    KVR_RUN(KVR_KERNEL_OPROJ, stream, "o gemm",
            kvr::launch_gemm_partial(dt, obuf, wo, B, sh.hidden, sh.hq * sh.d, L.g_o, part,
                                     stream));
    KVR_RUN(KVR_KERNEL_NORM, stream, "residual+norm",
            kvr::launch_residual_norm(dt, x_out, part, L.g_o.splits,
                                      static_cast<size_t>(B) * sh.hidden,
                                      static_cast<const float*>(W.mlp_norm), cfg->rms_eps, nbuf,
                                      B, sh.hidden, stream));
    KVR_RUN(KVR_KERNEL_GATEUP, stream, "gate/up gemm",
            kvr::launch_gemm_swiglu(dt, nbuf, W.w_gate, W.w_up, B, sh.inter, sh.hidden, L.g_gateup,
                                    part, mlp, stream));
    kvr::WeightSegs wd{{W.w_down, nullptr, nullptr}, {0, sh.hidden, sh.hidden, sh.hidden}, 1};
    KVR_RUN(KVR_KERNEL_DOWN, stream, "down gemm",
            kvr::launch_gemm_partial(dt, mlp, wd, B, sh.hidden, sh.inter, L.g_down, part,
                                     stream));
    const bool last = (l + 1 == n_layers);
    KVR_RUN(last ? KVR_KERNEL_FINAL : KVR_KERNEL_NORM, stream, "residual+norm",
            kvr::launch_residual_norm(
                dt, x_out, part, L.g_down.splits, static_cast<size_t>(B) * sh.hidden,
                last ? nullptr : static_cast<const float*>(w[l + 1].attn_norm), cfg->rms_eps,
                nbuf, B, sh.hidden, stream));
  }
  return KVR_OK;
}


// Argument checks shared by both inference-mode entry points.
kvr_status check_attention_args(const kvr_config* cfg, const kvr_kv& cache, const uint8_t* flags,
                                int n_tokens, const float* q, const int32_t* d_pos, int B,
                                const float* o, kvr::Shape* sh) {
  kvr_status st = check_heads(cfg, sh);
  if (st != KVR_OK) return st;
  if (!std::isfinite(cfg->alpha) || !std::isfinite(cfg->beta))
    return fail(KVR_ERR_INVALID_ARGUMENT, "alpha and beta must be finite");
  if (n_tokens <= 0) return fail(KVR_ERR_INVALID_ARGUMENT, "n_tokens must be positive");
  if (B < 0 || B > n_tokens)
    return fail(KVR_ERR_INVALID_ARGUMENT, "B=%d outside [0, n_tokens=%d]", B, n_tokens);
  if (B == 0) return KVR_OK;
  if (!dev_ok(q) || !dev_ok(d_pos) || !dev_ok(o) || !dev_ok(flags) || !dev_ok(cache.k) ||
      !dev_ok(cache.v))
    return fail(KVR_ERR_INVALID_ARGUMENT,
                "q, d_pos, o, flags and cache pointers must be non-NULL and 16-byte aligned");
  if (static_cast<const void*>(o) == static_cast<const void*>(q))
    return fail(KVR_ERR_INVALID_ARGUMENT, "o must not alias q");
  return KVR_OK;
}

// The launches of inference-mode attention over a workspace at `base`
// (256-byte aligned, at least L.total bytes).
kvr_status run_biased_attention(const kvr_config* cfg, const kvr::Shape& sh, const AttnLayout& L,
                                const kvr_kv& cache, const uint8_t* flags, int n_tokens,
                                const float* q, const int32_t* d_pos, int B, float* o,
                                uint8_t* base, hipStream_t stream) {
  const kvr_dtype dt = cfg->dtype;
  // (the result word borrows the first word of the workspace, written after
  // the check)
  kvr_status st;
  if (validate_mode() &&
      (st = check_support_sync(d_pos, B, n_tokens, 0, nullptr, reinterpret_cast<int32_t*>(base),
                               stream)) != KVR_OK)
    return st;
  if (kvr::decode_supported(dt, B, sh)) {
    // decode sizes: one streaming pass over the cache plus a chunk merge
    KVR_RUN(KVR_KERNEL_ATTN, stream, "decode attention",
            kvr::launch_attention_decode(q, d_pos, B, n_tokens, cache.k, cache.v, flags, sh,
                                         cfg->alpha, cfg->beta, base + L.attn, o, stream));
    KVR_RUN(KVR_KERNEL_ATTN_MERGE, stream, "decode merge",
            kvr::launch_attention_decode_merge(B, n_tokens, sh, base + L.attn, o, stream));
    return KVR_OK;
  }
  int32_t* n_full = reinterpret_cast<int32_t*>(base + L.n_full);
  int32_t* n_total = reinterpret_cast<int32_t*>(base + L.n_total);
  void* attn_ws = base + L.attn;
  // float32 storage attends on the caller's queries directly (the row kernel
  // applies 1/sqrt(d) itself); bf16 takes them scaled and rounded once
  // (bf16: the query prep launch also builds the attention plan)
  const void* qk = q;
  if (dt == KVR_BF16) {
    qk = base + L.q;
    KVR_RUN(KVR_KERNEL_QPREP, stream, "query prep and plan",
            kvr::launch_prep_queries(dt, q, static_cast<size_t>(B) * sh.hq * sh.d,
                                     kvr::attention_q_scale(dt, sh.d), base + L.q, d_pos, B,
                                     sh.group, n_full, n_total, stream));
  } else {
    KVR_RUN(KVR_KERNEL_PLAN, stream, "plan",
            kvr::launch_build_plan(d_pos, B, sh.group, n_full, n_total, stream));
  }
  KVR_RUN(KVR_KERNEL_ATTN, stream, "attention",
          kvr::launch_attention(dt, qk, cache.k, cache.v, flags, d_pos, B, n_tokens, sh,
                                cfg->alpha, cfg->beta, n_full, n_total, attn_ws, o, stream));
  if (kvr::attention_needs_merge(dt))
    KVR_RUN(KVR_KERNEL_ATTN_MERGE, stream, "attention merge",
            kvr::launch_attention_merge(dt, B, n_tokens, sh, n_total, attn_ws, o, true, stream));
  return KVR_OK;
}

// Scratch of kvr_biased_attention_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol); it uses the device address that hipGetSymbolAddress returns,
// looked up once per device with that device current.
static __device__ __align__(256) uint8_t scratch[KVR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};

kvr_status noalloc_scratch(uint8_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(KVR_ERR_UNSUPPORTED, "device index %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (reinterpret_cast<uintptr_t>(ptr) & 255u)
      return fail(KVR_ERR_HIP, "static scratch is not 256-byte aligned");
    g_scratch_ptr[dev] = static_cast<uint8_t*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return KVR_OK;
}

}  // namespace

extern "C" {

kvr_status kvr_build_repair_set(const int32_t* d_s, const int32_t* d_e, int32_t m,
                                int32_t n_tokens, int32_t tau, uint32_t mode,
                                const kvr_meta* meta, const kvr_repair_set* out,
                                int32_t* h_counts, hipStream_t stream) {
  g_err[0] = '\0';
  if (m < 1) return fail(KVR_ERR_BAD_BLOCKS, "m must be >= 1");
  if (n_tokens < 1) return fail(KVR_ERR_INVALID_ARGUMENT, "n_tokens must be >= 1");
  if (tau < 0) return fail(KVR_ERR_INVALID_ARGUMENT, "tau must be >= 0");
  if (mode & ~static_cast<uint32_t>(KVR_SEAM_ASYMMETRIC | KVR_INIT_META))
    return fail(KVR_ERR_INVALID_ARGUMENT, "unknown mode bits 0x%x", mode);
  if (!dev_ok(d_s) || !dev_ok(d_e)) return fail(KVR_ERR_INVALID_ARGUMENT, "d_s / d_e NULL or misaligned");
  if (!out || !dev_ok(out->T) || !dev_ok(out->run_start) || !dev_ok(out->run_len) ||
      !dev_ok(out->counts) || out->cap < 0)
    return fail(KVR_ERR_INVALID_ARGUMENT, "repair-set outputs NULL, misaligned or cap < 0");
  const bool init = (mode & KVR_INIT_META) != 0;
  if (init) {
    if (!meta || !dev_ok(meta->flags) || meta->n_tokens != n_tokens ||
        (meta->block_id && !aligned16(meta->block_id)))
      return fail(KVR_ERR_INVALID_ARGUMENT, "KVR_INIT_META needs meta with flags and n_tokens == N");
  }
  hipError_t e = kvr::launch_build_repair_set(d_s, d_e, m, n_tokens, tau,
                                              (mode & KVR_SEAM_ASYMMETRIC) != 0, out->T,
                                              out->run_start, out->run_len, out->counts, out->cap,
                                              stream);
  if (e != hipSuccess) return hip_fail(e, "build repair set");
  if (init) {
    e = kvr::launch_init_meta(d_s, d_e, m, n_tokens, out->counts, meta->flags, meta->block_id,
                              stream);
    if (e != hipSuccess) return hip_fail(e, "init meta");
  }
  if (!h_counts) return KVR_OK;
  e = hipMemcpyAsync(h_counts, out->counts, 3 * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return hip_fail(e, "copy counts");
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "synchronize");
  if (h_counts[2] == KVR_ERR_BAD_BLOCKS) return fail(KVR_ERR_BAD_BLOCKS, "blocks do not tile [0, N)");
  if (h_counts[2] == KVR_ERR_CAPACITY)
    return fail(KVR_ERR_CAPACITY, "|T| = %d exceeds cap %d", h_counts[0], out->cap);
  return KVR_OK;
}

kvr_status kvr_check_support(const int32_t* d_T, int32_t B, int32_t n_tokens,
                             int32_t first_selectable, const int32_t* d_gpos,
                             int32_t* d_result, hipStream_t stream) {
  g_err[0] = '\0';
  if (B < 0 || n_tokens < 0 || B > n_tokens)
    return fail(KVR_ERR_INVALID_ARGUMENT, "B=%d, n_tokens=%d", B, n_tokens);
  if (!dev_ok(d_result) || (B > 0 && !dev_ok(d_T)) || (d_gpos && !aligned16(d_gpos)))
    return fail(KVR_ERR_INVALID_ARGUMENT, "d_T / d_gpos / d_result NULL or misaligned");
  return check_support_sync(d_T, B, n_tokens, first_selectable, d_gpos, d_result, stream);
}


kvr_status kvr_build_runs(const int32_t* d_T, int32_t B, int32_t n_tokens,
                          int32_t first_selectable, const kvr_repair_set* out,
                          int32_t* h_counts, hipStream_t stream) {
  g_err[0] = '\0';
  if (B < 0 || n_tokens < 0 || B > n_tokens)
    return fail(KVR_ERR_INVALID_ARGUMENT, "B=%d, n_tokens=%d", B, n_tokens);
  if (!out || !dev_ok(out->run_start) || !dev_ok(out->run_len) || !dev_ok(out->counts) ||
      (B > 0 && !dev_ok(d_T)))
    return fail(KVR_ERR_INVALID_ARGUMENT, "d_T / run outputs NULL or misaligned");
  if (out->cap < B) return fail(KVR_ERR_INVALID_ARGUMENT, "cap %d < B %d", out->cap, B);
  hipError_t e = kvr::launch_build_runs(d_T, B, n_tokens, first_selectable, out->run_start,
                                        out->run_len, out->counts, stream);
  if (e != hipSuccess) return hip_fail(e, "build runs");
  if (!h_counts) return KVR_OK;
  e = hipMemcpyAsync(h_counts, out->counts, 3 * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return hip_fail(e, "copy counts");
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "synchronize");
  if (h_counts[2] != KVR_OK)
    return fail(KVR_ERR_BAD_SUPPORT, "support not strictly increasing or outside [%d, %d)",
                first_selectable, n_tokens);
  return KVR_OK;
}

kvr_status kvr_build_tile_map(const int32_t* d_T, int32_t B, int32_t n_tokens,
                              int32_t* d_first_q, hipStream_t stream) {
  g_err[0] = '\0';
  if (n_tokens < 1 || B < 0 || B > n_tokens)
    return fail(KVR_ERR_INVALID_ARGUMENT, "B=%d, n_tokens=%d", B, n_tokens);
  if (!dev_ok(d_first_q) || (B > 0 && !dev_ok(d_T)))
    return fail(KVR_ERR_INVALID_ARGUMENT, "d_T / d_first_q NULL or misaligned");
  hipError_t e = kvr::launch_tile_map(d_T, B, n_tokens, d_first_q, stream);
  if (e != hipSuccess) return hip_fail(e, "tile map");
  return KVR_OK;
}

kvr_status kvr_build_plan(const int32_t* d_T, int32_t B, int32_t group, int32_t* d_n_full,
                          int32_t* d_n_total, hipStream_t stream) {
  g_err[0] = '\0';
  if (B < 0 || group < 1) return fail(KVR_ERR_INVALID_ARGUMENT, "B < 0 or group < 1");
  if (B == 0) return KVR_OK;
  if (!dev_ok(d_T) || !dev_ok(d_n_full) || !dev_ok(d_n_total))
    return fail(KVR_ERR_INVALID_ARGUMENT, "pointers NULL or misaligned");
  hipError_t e = kvr::launch_build_plan(d_T, B, group, d_n_full, d_n_total, stream);
  return e == hipSuccess ? KVR_OK : hip_fail(e, "build plan");
}

size_t kvr_workspace_bytes(const kvr_config* cfg, int32_t B, int32_t n_tokens) {
  kvr::Shape sh;
  if (check_config(cfg, &sh) != KVR_OK || B < 0 || n_tokens <= 0 || B > n_tokens) return 0;
  return layout_for(cfg, sh, B, n_tokens).total + 256;
}

kvr_status kvr_layer_repair(const kvr_config* cfg, const kvr_layer_weights* w, kvr_kv cache,
                            const kvr_meta* meta, const int32_t* d_T, int32_t B,
                            const float* x_in, int32_t x_in_rows, float* x_out, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  return run_stack(cfg, 1, w, &cache, meta, d_T, B, x_in, x_in_rows, x_out, ws, ws_bytes, stream);
}

kvr_status kvr_stack_repair(const kvr_config* cfg, int32_t n_layers, const kvr_layer_weights* w,
                            const kvr_kv* caches, const kvr_meta* meta, const int32_t* d_T,
                            int32_t B, const float* x_in, int32_t x_in_rows, float* x_out,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  return run_stack(cfg, n_layers, w, caches, meta, d_T, B, x_in, x_in_rows, x_out, ws, ws_bytes,
                   stream);
}

size_t kvr_attention_workspace_bytes(const kvr_config* cfg, int32_t B, int32_t n_tokens) {
  kvr::Shape sh;
  if (check_heads(cfg, &sh) != KVR_OK || B < 0 || n_tokens <= 0 || B > n_tokens) return 0;
  return attn_layout_for(cfg, sh, B, n_tokens).total + 256;
}

kvr_status kvr_biased_attention(const kvr_config* cfg, kvr_kv cache, const uint8_t* flags,
                                int32_t n_tokens, const float* q, const int32_t* d_pos,
                                int32_t B, float* o, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  g_err[0] = '\0';
  kvr::Shape sh;
  kvr_status st = check_attention_args(cfg, cache, flags, n_tokens, q, d_pos, B, o, &sh);
  if (st != KVR_OK || B == 0) return st;
  if (!dev_ok(ws)) return fail(KVR_ERR_INVALID_ARGUMENT, "ws must be non-NULL and 16-byte aligned");
  const AttnLayout L = attn_layout_for(cfg, sh, B, n_tokens);
  uint8_t* base = reinterpret_cast<uint8_t*>(up256(reinterpret_cast<uintptr_t>(ws)));
  const size_t slack = static_cast<size_t>(base - static_cast<uint8_t*>(ws));
  if (ws_bytes < L.total + slack)
    return fail(KVR_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, L.total + slack);
  return run_biased_attention(cfg, sh, L, cache, flags, n_tokens, q, d_pos, B, o, base, stream);
}

kvr_status kvr_biased_attention_noalloc(const kvr_config* cfg, kvr_kv cache, const uint8_t* flags,
                                        int32_t n_tokens, const float* q, const int32_t* d_pos,
                                        int32_t B, float* o, hipStream_t stream) {
  g_err[0] = '\0';
  kvr::Shape sh;
  kvr_status st = check_attention_args(cfg, cache, flags, n_tokens, q, d_pos, B, o, &sh);
  if (st != KVR_OK || B == 0) return st;
  const AttnLayout L = attn_layout_for(cfg, sh, B, n_tokens);
  if (L.total > static_cast<size_t>(KVR_NOALLOC_SCRATCH_BYTES))
    return fail(KVR_ERR_WORKSPACE,
                "this call needs %zu bytes of scratch; the static scratch holds %d "
                "(use kvr_biased_attention with a workspace)",
                L.total, static_cast<int>(KVR_NOALLOC_SCRATCH_BYTES));
  uint8_t* base = nullptr;
  if ((st = noalloc_scratch(&base)) != KVR_OK) return st;
  return run_biased_attention(cfg, sh, L, cache, flags, n_tokens, q, d_pos, B, o, base, stream);
}

kvr_status kvr_shift_cache(const kvr_config* cfg, int32_t n_layers, const kvr_kv* src,
                           const kvr_kv* dst, const uint8_t* flags_src, uint8_t* flags_dst,
                           const int32_t* block_src, int32_t* block_dst, int32_t n_tokens,
                           int32_t del_start, int32_t del_len, uint8_t mark,
                           hipStream_t stream) {
  g_err[0] = '\0';
  kvr::Shape sh;
  kvr_status st = check_heads(cfg, &sh);
  if (st != KVR_OK) return st;
  if (!std::isfinite(cfg->rope_theta) || cfg->rope_theta <= 0.0)
    return fail(KVR_ERR_INVALID_ARGUMENT, "rope_theta must be finite and positive");
  if (n_layers < 1 || !src || !dst)
    return fail(KVR_ERR_INVALID_ARGUMENT, "n_layers must be >= 1 with src and dst arrays");
  if (n_tokens < 0 || del_start < 0 || del_len < 0 ||
      static_cast<int64_t>(del_start) + del_len > n_tokens)
    return fail(KVR_ERR_INVALID_ARGUMENT, "span [%d, %d + %d) outside [0, %d)", del_start,
                del_start, del_len, n_tokens);
  if ((flags_src == nullptr) != (flags_dst == nullptr) ||
      (block_src == nullptr) != (block_dst == nullptr))
    return fail(KVR_ERR_INVALID_ARGUMENT, "flags and block ids: both src and dst, or neither");
  if ((flags_dst && (!aligned16(flags_src) || !aligned16(flags_dst))) ||
      (block_dst && (!aligned16(block_src) || !aligned16(block_dst))))
    return fail(KVR_ERR_INVALID_ARGUMENT, "metadata pointers not 16-byte aligned");
  const int n_out = n_tokens - del_len;
  const size_t row_bytes = static_cast<size_t>(sh.hkv) * sh.d * esize(cfg->dtype);
  struct Range { uintptr_t lo, hi; };
  std::vector<Range> srcs, dsts;
  for (int l = 0; l < n_layers; ++l) {
    if (!dev_ok(src[l].k) || !dev_ok(src[l].v) || !dev_ok(dst[l].k) || !dev_ok(dst[l].v))
      return fail(KVR_ERR_INVALID_ARGUMENT, "layer %d: cache pointers NULL or not 16-byte aligned", l);
    for (const void* p : {src[l].k, src[l].v}) {
      const uintptr_t a = reinterpret_cast<uintptr_t>(p);
      srcs.push_back({a, a + row_bytes * n_tokens});
    }
    for (const void* p : {static_cast<const void*>(dst[l].k), static_cast<const void*>(dst[l].v)}) {
      const uintptr_t a = reinterpret_cast<uintptr_t>(p);
      dsts.push_back({a, a + row_bytes * n_out});
    }
  }
  if (flags_dst) {
    srcs.push_back({reinterpret_cast<uintptr_t>(flags_src), reinterpret_cast<uintptr_t>(flags_src) + n_tokens});
    dsts.push_back({reinterpret_cast<uintptr_t>(flags_dst), reinterpret_cast<uintptr_t>(flags_dst) + n_out});
  }
  if (block_dst) {
    srcs.push_back({reinterpret_cast<uintptr_t>(block_src), reinterpret_cast<uintptr_t>(block_src) + 4u * n_tokens});
    dsts.push_back({reinterpret_cast<uintptr_t>(block_dst), reinterpret_cast<uintptr_t>(block_dst) + 4u * n_out});
  }
  for (const Range& d : dsts)
    for (const Range& s : srcs)
      if (d.lo < s.hi && s.lo < d.hi && d.lo < d.hi && s.lo < s.hi)
        return fail(KVR_ERR_INVALID_ARGUMENT, "a destination buffer overlaps a source buffer");
  if (n_out == 0) return KVR_OK;

  for (int l0 = 0; l0 < n_layers; l0 += kvr::kShiftMaxLayers) {
    const int nl = std::min(kvr::kShiftMaxLayers, n_layers - l0);
    kvr::ShiftLayers L{};
    for (int j = 0; j < nl; ++j) {
      L.src_k[j] = src[l0 + j].k;
      L.src_v[j] = src[l0 + j].v;
      L.dst_k[j] = dst[l0 + j].k;
      L.dst_v[j] = dst[l0 + j].v;
    }
    KVR_RUN(KVR_KERNEL_SHIFT, stream, "shift",
            kvr::launch_shift(cfg->dtype, L, nl, n_out, sh, del_start, del_len, cfg->rope_theta,
                              stream));
  }
  KVR_RUN(KVR_KERNEL_SHIFT, stream, "shift metadata",
          kvr::launch_shift_meta(flags_src, flags_dst, block_src, block_dst, n_out, del_start,
                                 del_len, mark, stream));
  return KVR_OK;
}

kvr_status kvr_sur_scores(const void* d_E, kvr_dtype dtype, int32_t vocab, int32_t hidden,
                          const int32_t* d_suffix_ids, int32_t S, const int32_t* d_query_ids,
                          int32_t Q, float* d_r, hipStream_t stream) {
  g_err[0] = '\0';
  if (raw_dtype(&dtype) != KVR_F32 && raw_dtype(&dtype) != KVR_BF16)
    return fail(KVR_ERR_INVALID_ARGUMENT, "unknown dtype %d", raw_dtype(&dtype));
  if (vocab < 1 || S < 0 || Q < 1 || Q > kvr::kSurMaxQuery)
    return fail(KVR_ERR_INVALID_ARGUMENT, "vocab=%d, S=%d, Q=%d (1 <= Q <= %d)", vocab, S, Q,
                kvr::kSurMaxQuery);
  if (hidden <= 0 || hidden % 64 || (dtype == KVR_F32 && hidden > 8192))
    return fail(KVR_ERR_UNSUPPORTED, "hidden=%d (a positive multiple of 64; <= 8192 for float32)",
                hidden);
  if (S == 0) return KVR_OK;
  if (!dev_ok(d_E) || !dev_ok(d_suffix_ids) || !dev_ok(d_query_ids) || !dev_ok(d_r))
    return fail(KVR_ERR_INVALID_ARGUMENT, "pointers must be non-NULL and 16-byte aligned");
  KVR_RUN(KVR_KERNEL_SUR_SCORE, stream, "sur scores",
          kvr::launch_sur_scores(dtype, d_E, vocab, hidden, d_suffix_ids, S, d_query_ids, Q, d_r,
                                 stream));
  return KVR_OK;
}

kvr_status kvr_sur_select(const float* d_r, int32_t S, const int32_t* d_unit_start,
                          int32_t n_units, int32_t budget, int32_t pos0, float* d_unit_scores,
                          const kvr_repair_set* out, float* d_ws, size_t ws_bytes,
                          int32_t* h_counts, hipStream_t stream) {
  g_err[0] = '\0';
  if (S < 1 || n_units < 1 || n_units > S || budget < 0 || budget > S || pos0 < 0)
    return fail(KVR_ERR_INVALID_ARGUMENT, "S=%d, n_units=%d, budget=%d, pos0=%d", S, n_units,
                budget, pos0);
  if (n_units > kvr::kSurMaxUnitCount)
    return fail(KVR_ERR_UNSUPPORTED, "n_units=%d > %d", n_units, kvr::kSurMaxUnitCount);
  if (!dev_ok(d_r) || !dev_ok(d_unit_start) || !dev_ok(d_unit_scores) || !dev_ok(d_ws))
    return fail(KVR_ERR_INVALID_ARGUMENT, "pointers must be non-NULL and 16-byte aligned");
  if (!out || !dev_ok(out->T) || !dev_ok(out->run_start) || !dev_ok(out->run_len) ||
      !dev_ok(out->counts) || out->cap < budget)
    return fail(KVR_ERR_INVALID_ARGUMENT, "outputs NULL, misaligned or cap < budget");
  if (ws_bytes < 2 * sizeof(float) * static_cast<size_t>(S))
    return fail(KVR_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes,
                2 * sizeof(float) * static_cast<size_t>(S));
  KVR_RUN(KVR_KERNEL_SUR_SELECT, stream, "sur select",
          kvr::launch_sur_select(d_r, S, d_unit_start, n_units, d_unit_scores, budget, pos0, d_ws,
                                 out->T, out->run_start, out->run_len, out->counts, out->cap,
                                 stream));
  if (!h_counts) return KVR_OK;
  hipError_t e = hipMemcpyAsync(h_counts, out->counts, 3 * sizeof(int32_t),
                                hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return hip_fail(e, "copy counts");
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "synchronize");
  if (h_counts[2] == KVR_ERR_BAD_BLOCKS)
    return fail(KVR_ERR_BAD_BLOCKS, "unit starts do not partition [0, S)");
  if (h_counts[2] != KVR_OK)
    return fail(static_cast<kvr_status>(h_counts[2]), "selection failed (|T| = %d)", h_counts[0]);
  return KVR_OK;
}

const char* kvr_status_string(kvr_status s) {
  switch (s) {
    case KVR_OK: return "KVR_OK";
    case KVR_ERR_INVALID_ARGUMENT: return "KVR_ERR_INVALID_ARGUMENT";
    case KVR_ERR_UNSUPPORTED: return "KVR_ERR_UNSUPPORTED";
    case KVR_ERR_BAD_BLOCKS: return "KVR_ERR_BAD_BLOCKS";
    case KVR_ERR_BAD_SUPPORT: return "KVR_ERR_BAD_SUPPORT";
    case KVR_ERR_CAPACITY: return "KVR_ERR_CAPACITY";
    case KVR_ERR_WORKSPACE: return "KVR_ERR_WORKSPACE";
    case KVR_ERR_HIP: return "KVR_ERR_HIP";
  }
  return "KVR_UNKNOWN_STATUS";
}

const char* kvr_last_error(void) { return g_err; }

kvr_status kvr_timing_begin(uint32_t mask) {
  g_timing.mask = mask & ((1u << KVR_KERNEL_COUNT) - 1u);
  g_timing.used = 0;
  return KVR_OK;
}

kvr_status kvr_timing_end(double* total_ms, int32_t* launches) {
  g_err[0] = '\0';
  if (total_ms) for (int i = 0; i < KVR_KERNEL_COUNT; ++i) total_ms[i] = 0.0;
  if (launches) for (int i = 0; i < KVR_KERNEL_COUNT; ++i) launches[i] = 0;
  kvr_status st = KVR_OK;
  for (size_t i = 0; i < g_timing.used; ++i) {
    hipEvent_t a = g_timing.ev[2 * i], b = g_timing.ev[2 * i + 1];
    hipError_t e = hipEventSynchronize(b);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
    if (e != hipSuccess) { st = hip_fail(e, "timing events"); break; }
    const int id = g_timing.id[i];
    if (total_ms) total_ms[id] += ms;
    if (launches) launches[id] += 1;
  }
  g_timing.mask = 0;
  g_timing.used = 0;
  return st;
}

}  // extern "C"
