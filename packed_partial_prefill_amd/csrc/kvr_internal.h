// Internal launch interface of libkvr (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvr.h"

namespace kvr {

// Model shape of one call, validated by the host layer.
struct Shape {
  int hidden, hq, hkv, d, inter, group;
  __host__ __device__ int qkv_cols() const { return (hq + 2 * hkv) * d; }
};

// ---- index.hip --------------------------------------------------------------
hipError_t launch_build_repair_set(const int32_t* s, const int32_t* e, int m, int n_tokens,
                                   int tau, bool asym, int32_t* T, int32_t* run_start,
                                   int32_t* run_len, int32_t* counts, int cap, hipStream_t stream);
hipError_t launch_init_meta(const int32_t* s, const int32_t* e, int m, int n_tokens,
                            const int32_t* counts, uint8_t* flags, int32_t* block_id,
                            hipStream_t stream);
hipError_t launch_check_support(const int32_t* T, int B, int n_tokens, int first,
                                const int32_t* gpos, int32_t* result, hipStream_t stream);
// Support check plus maximal runs of an explicit support; counts = (B, R, status).
hipError_t launch_build_runs(const int32_t* T, int B, int n_tokens, int first,
                             int32_t* run_start, int32_t* run_len, int32_t* counts,
                             hipStream_t stream);
int plan_tiles(int B, int group);
// first_q[c] (c < ceil(n_tokens / KV_TILE)): first row r with T[r] >= c * KV_TILE.
hipError_t launch_tile_map(const int32_t* T, int B, int n_tokens, int32_t* first_q,
                           hipStream_t stream);
hipError_t launch_build_plan(const int32_t* T, int B, int group, int32_t* n_full,
                             int32_t* n_total, hipStream_t stream);
// The per-call tables of a layer repair: the attention plan (n_full and
// n_total of each of n_tiles query tiles) and the RoPE table (cos, sin of
// g_r * theta^(-2i/d) as float32 pairs [B][half], computed in float64,
// g_r = gpos[T[r]] or T[r] when gpos is NULL).  Entries 0 .. n_tiles - 1 are
// plan entries, the next B * half the table's.
struct LayerTables {
  const int32_t* T;
  const int32_t* gpos;
  int B, group, n_tiles;
  int32_t* n_full;
  int32_t* n_total;
  int half;
  double theta;
  float2* tab;
  int entries() const { return n_tiles + B * half; }
};

// ---- norm.hip ---------------------------------------------------------------
// x_res[r] = x_in[gather ? T[r] : r]; n_out[r] = RMSNorm(x_res[r]) * gamma.
// With tabs, further workgroups of the same launch build those tables.
hipError_t launch_gather_norm(kvr_dtype dt, const float* x_in, const int32_t* gather_T,
                              float* x_res, const float* gamma, float eps, void* n_out, int B,
                              int hidden, const LayerTables* tabs, hipStream_t stream);
// x_res[r] += sum_s part[s][r]; if gamma: n_out[r] = RMSNorm(x_res[r]) * gamma.
hipError_t launch_residual_norm(kvr_dtype dt, float* x_res, const float* part, int splits,
                                size_t split_stride, const float* gamma, float eps, void* n_out,
                                int B, int hidden, hipStream_t stream);

// ---- gemm.hip ---------------------------------------------------------------
// Weight matrix given as up to three row segments (e.g. Wq | Wk | Wv):
// output column n belongs to segment j with n_begin[j] <= n < n_begin[j+1].
struct WeightSegs {
  const void* w[3];
  int n_begin[4];
  int nseg;
};
// How one projection is launched: tile shape (variant), K split, and for the
// gate/up pair whether SwiGLU runs in the GEMM epilogue (fused, no split) or
// in a reduction of float32 partials.
struct GemmPlan {
  int variant;
  int splits;
  bool fused;
};
GemmPlan gemm_plan_for(kvr_dtype dt, int M, int N, int K, bool swiglu);
// part[s][M][N] (float32) = A[M, K-slice s] * W[N, K-slice s]^T for
// s < plan.splits (K split evenly in multiples of 32).
hipError_t launch_gemm_partial(kvr_dtype dt, const void* A, const WeightSegs& W, int M, int N,
                               int K, const GemmPlan& plan, float* part, hipStream_t stream);
// out[M][N] = SiLU(A Wg^T) * (A Wu^T), stored in dtype dt; part holds
// plan.splits * M * 2N floats when the plan is not fused.
hipError_t launch_gemm_swiglu(kvr_dtype dt, const void* A, const void* Wg, const void* Wu, int M,
                              int N, int K, const GemmPlan& plan, float* part, void* out,
                              hipStream_t stream);

// ---- rope.hip -----------------------------------------------------------------
hipError_t launch_rope_writeback(kvr_dtype dt, const float* qkv_part, int splits,
                                 size_t split_stride, const float* bq, const float* bk,
                                 const float* bv, const float2* tab, const int32_t* T, int B,
                                 const Shape& sh, float q_scale, void* q_out, void* k_cache,
                                 void* v_cache, uint8_t* flags, hipStream_t stream);

// q_out[i] = q[i] * scale stored in dtype dt (n elements, a multiple of 4).
// also builds the attention plan (n_full, n_total) of the query positions
hipError_t launch_prep_queries(kvr_dtype dt, const float* q, size_t n, float scale, void* q_out,
                               const int32_t* pos, int B, int group, int32_t* n_full,
                               int32_t* n_total, hipStream_t stream);

// ---- shift.hip ----------------------------------------------------------------
constexpr int kShiftMaxLayers = 32;   // layers per launch (kernel-argument arrays)
struct ShiftLayers {
  const void* src_k[kShiftMaxLayers];
  const void* src_v[kShiftMaxLayers];
  void* dst_k[kShiftMaxLayers];
  void* dst_v[kShiftMaxLayers];
};
// Cache rows [0, n_out) of each layer's dst from src with rows
// [del_start, del_start + del_len) deleted; moved keys re-rotated by -del_len.
hipError_t launch_shift(kvr_dtype dt, const ShiftLayers& L, int n_layers, int n_out,
                        const Shape& sh, int del_start, int del_len, double theta,
                        hipStream_t stream);
hipError_t launch_shift_meta(const uint8_t* f_src, uint8_t* f_dst, const int32_t* b_src,
                             int32_t* b_dst, int n_out, int del_start, int del_len, uint8_t mark,
                             hipStream_t stream);

// ---- sur.hip ------------------------------------------------------------------
constexpr int kSurMaxQuery = 256;
constexpr int kSurMaxUnitCount = 8192;
hipError_t launch_sur_scores(kvr_dtype dt, const void* E, int vocab, int hidden,
                             const int32_t* sid, int S, const int32_t* qid, int Q, float* r,
                             hipStream_t stream);
// ws: 2 * S floats (envelope and window sums of the unit that takes a window)
hipError_t launch_sur_select(const float* r, int S, const int32_t* ustart, int U,
                             float* uscore, int budget, int pos0, float* ws, int32_t* T,
                             int32_t* run_start, int32_t* run_len, int32_t* counts, int cap,
                             hipStream_t stream);

// ---- attention.hip ----------------------------------------------------------
size_t attention_workspace_bytes(kvr_dtype dt, int B, int n_tokens, const Shape& sh);
hipError_t launch_attention(kvr_dtype dt, const void* q, const void* k_cache,
                            const void* v_cache, const uint8_t* flags, const int32_t* T, int B,
                            int n_tokens, const Shape& sh, float alpha, float beta,
                            const int32_t* plan_n_full, const int32_t* plan_n_total, void* ws,
                            void* o_out, hipStream_t stream);
bool attention_needs_merge(kvr_dtype dt);
// Inference-mode decode path (bf16, B * group <= 64 pairs per KV head):
// float32 queries in; chunk partials in ws, then the merge writes float32
// o [B, Hq, d].
bool decode_supported(kvr_dtype dt, int B, const Shape& sh);
size_t decode_workspace_bytes(int B, int n_tokens, const Shape& sh);
hipError_t launch_attention_decode(const float* q, const int32_t* pos, int B, int n_tokens,
                                   const void* k_cache, const void* v_cache,
                                   const uint8_t* flags, const Shape& sh, float alpha, float beta,
                                   void* ws, float* o, hipStream_t stream);
hipError_t launch_attention_decode_merge(int B, int n_tokens, const Shape& sh, void* ws,
                                         float* o, hipStream_t stream);
// o_out: [B, Hq, d] in bf16, or float32 when out_f32.
hipError_t launch_attention_merge(kvr_dtype dt, int B, int n_tokens, const Shape& sh,
                                  const int32_t* plan_n_total, void* ws, void* o_out,
                                  bool out_f32, hipStream_t stream);
// Factor the RoPE kernel folds into the stored queries for this path.
float attention_q_scale(kvr_dtype dt, int head_dim);

}  // namespace kvr
