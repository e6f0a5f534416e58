/*
 * kvr.h - C ABI of libkvr: layer-packed selective recompute of a mixed
 * KV cache (budgeted KV-cache repair) on AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources cited by page title and section):
 *   - "Budgeted KV-Cache Repair for Evolving Contexts", section 13.2
 *     (mixed-cache recurrence, Eq. 21-22; reusable execution plan,
 *     Eq. 23-24), section 3.3 (layer-major packed schedule), section 7.1
 *     (exact budget, Eq. 3; only retained-suffix positions are selectable).
 *   - The cross-attention reuse specification page, sections 6.1-6.4:
 *     blocks [s_i, e_i), mixed cache L[t,l] = (K, V, m_t) with
 *     m_t = (type, block id, global position), the seam set T_tau with the
 *     asymmetric true-prefix rule, and the biased operator F whose logits
 *     are <q,k>/sqrt(d) + alpha*[type=local] + beta*[key in S'].
 *
 * Conventions shared by every entry point:
 *   - Every buffer is owned by the caller.  The library allocates no device
 *     memory; scratch comes from the caller's workspace.  It keeps no pointer
 *     after a call returns.
 *   - "device" pointers point to GPU memory of the current HIP device;
 *     "host" pointers to CPU memory.  Device pointers must be 16-byte
 *     aligned.
 *   - Calls enqueue work on `stream` (0 = the null stream) in order and
 *     return; only the calls that say so synchronise.
 *   - Host-side validation runs first and returns an error without touching
 *     the device.  A failed HIP call returns KVR_ERR_HIP; the HIP error text
 *     is then in kvr_last_error().
 *   - The cache row index t is the global position g_t unless kvr_meta
 *     carries a position map (then g_t = gpos[t], strictly increasing);
 *     RoPE angles and causal visibility both use it.
 */
#ifndef KVR_H
#define KVR_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVR_OK = 0,
  KVR_ERR_INVALID_ARGUMENT = -1, /* null/misaligned pointer, bad size, non-finite scalar */
  KVR_ERR_UNSUPPORTED = -2,      /* shape outside what the kernels implement        */
  KVR_ERR_BAD_BLOCKS = -3,       /* blocks do not tile [0, N)                        */
  KVR_ERR_BAD_SUPPORT = -4,      /* support not strictly increasing / out of range   */
  KVR_ERR_CAPACITY = -5,         /* output arrays too small                          */
  KVR_ERR_WORKSPACE = -6,        /* workspace smaller than kvr_workspace_bytes()     */
  KVR_ERR_HIP = -7               /* a HIP runtime call or launch failed              */
} kvr_status;

/* Storage type of layer weights and the KV cache.  Activations crossing the
 * boundary (x_in, x_out), RMSNorm gains and q/k/v biases are always float32.
 * KVR_BF16 computes matrix products on bf16 operands with float32
 * accumulation; KVR_F32 is float32 end to end. */
typedef enum { KVR_F32 = 0, KVR_BF16 = 1 } kvr_dtype;

/* Per-position metadata byte m_t (cross-attention reuse page, 6.2 / 6.4):
 * bit 0 set = type local (KV does not match a full prefill), clear = global;
 * bit 1 set = position is in the spurious-sink set S'. */
enum { KVR_FLAG_LOCAL = 1u, KVR_FLAG_SINK = 2u };

/* mode bits of kvr_build_repair_set */
enum {
  KVR_SEAM_ASYMMETRIC = 1u, /* true-prefix rule: skip B_1's trailing window, add B_m's (6.3) */
  KVR_INIT_META = 2u        /* also write load-time metadata for all N positions           */
};

/* Attention tiling used by kvr_build_plan and the packed attention kernel:
 * a query tile holds KVR_ATTN_QROWS (packed row, query head) pairs of one KV
 * head group (pair p = r*G + h with G = n_q_heads / n_kv_heads), keys are
 * visited in tiles of KVR_ATTN_KV_TILE positions. */
enum { KVR_ATTN_QROWS = 128, KVR_ATTN_KV_TILE = 64 };

typedef struct {
  int32_t hidden;        /* model width; multiple of 64                            */
  int32_t n_q_heads;     /* query heads Hq                                          */
  int32_t n_kv_heads;    /* KV heads Hkv; Hq % Hkv == 0 (query head h reads h/(Hq/Hkv)) */
  int32_t head_dim;      /* d: 64 or 128                                            */
  int32_t intermediate;  /* SwiGLU width; multiple of 64                            */
  float rms_eps;         /* RMSNorm epsilon (finite, >= 0)                          */
  double rope_theta;     /* RoPE base; rotate-half pairing (i, i + d/2)             */
  float alpha;           /* logit bias on local keys (finite)                       */
  float beta;            /* logit bias on spurious-sink keys (finite)               */
  kvr_dtype dtype;       /* storage of weights and cache                            */
} kvr_config;

/* One decoder layer.  Matrices are device, row-major [out, in] (PyTorch
 * Linear), in cfg.dtype: wq [Hq*d, hidden] (head h owns rows h*d..h*d+d-1),
 * wk / wv [Hkv*d, hidden], wo [hidden, Hq*d], w_gate / w_up
 * [intermediate, hidden], w_down [hidden, intermediate].  attn_norm and
 * mlp_norm are float32 [hidden]; bq [Hq*d], bk / bv [Hkv*d] are float32 and
 * may all be NULL (no projection bias). */
typedef struct {
  const void *attn_norm, *wq, *wk, *wv, *bq, *bk, *bv, *wo, *mlp_norm, *w_gate, *w_up, *w_down;
} kvr_layer_weights;

/* One layer's cache: device K and V, each [N, Hkv, d] contiguous, cfg.dtype.
 * Keys are stored after RoPE; values are not rotated. */
typedef struct {
  void *k, *v;
} kvr_kv;

/* Mixed-cache metadata m_t = (type, block id, global position) shared by all
 * layers (cross-attention reuse page, 6.2; m_t has no layer index).
 *   flags     device uint8 [n_tokens] (KVR_FLAG_* bits: the type, and
 *             membership of the spurious-sink set).
 *   block_id  device int32 [n_tokens] or NULL (only written by KVR_INIT_META).
 *   gpos      device int32 [n_tokens] or NULL: the global position g_t of
 *             cache row t, which RoPE and the causal rule of F use (6.2).
 *             NULL means g_t = t.  A non-NULL map must be non-negative and
 *             strictly increasing (kvr_check_support verifies it); causal
 *             visibility g_j <= g_u is then visibility by row, j <= u, and
 *             the repair rotates row r's query and key at g_{T[r]}.
 *   n_tokens  N, the number of cache rows. */
typedef struct {
  uint8_t* flags;
  int32_t* block_id;
  const int32_t* gpos;
  int32_t n_tokens;
} kvr_meta;

/* Output of kvr_build_repair_set; all device arrays.  T, run_start and
 * run_len hold `cap` int32 each; counts holds 3 int32:
 * counts[0] = |T|, counts[1] = R (number of maximal runs), counts[2] =
 * status of the build (KVR_OK, KVR_ERR_BAD_BLOCKS or KVR_ERR_CAPACITY). */
typedef struct {
  int32_t *T, *run_start, *run_len, *counts;
  int32_t cap;
} kvr_repair_set;

/*
 * kvr_build_repair_set - recomputation set T_tau from block boundaries
 * (cross-attention reuse page, 6.3), its maximal runs (the execution
 * intervals of Budgeted KV-Cache Repair, section 3.2), and optionally the
 * load-time metadata (6.2).
 *
 *   d_s, d_e   device int32 [m]: block starts / exclusive ends.  They must
 *              tile [0, n_tokens): s_1 = 0, e_i = s_{i+1}, e_m = n_tokens,
 *              every block non-empty; otherwise counts[2] = BAD_BLOCKS.
 *   tau        seam half-width (>= 0).  Window at seam i|i+1: the last tau
 *              positions of B_i and the first tau of B_{i+1}, each clipped to
 *              its block.  With KVR_SEAM_ASYMMETRIC, B_1's trailing window is
 *              dropped and B_m's trailing tau positions are added.  T is the
 *              ascending set union.  m = 1 or tau = 0 gives T empty.
 *   meta       needed (non-NULL, meta->n_tokens == n_tokens) with
 *              KVR_INIT_META: flags[t] = LOCAL for t >= e_1, plus SINK at
 *              every s_i with i >= 2; block_id[t] = i - 1 (when non-NULL).
 *   out        device arrays (see kvr_repair_set).  |T| > out->cap gives
 *              counts[2] = CAPACITY with T, runs and counts[0..1] undefined.
 *   h_counts   host int32 [3] or NULL.  When given, counts are copied back,
 *              the stream is synchronised and the device status is returned.
 *              When NULL the call does not synchronise and returns KVR_OK
 *              after the launch; the status is then only in counts[2].
 */
kvr_status kvr_build_repair_set(const int32_t* d_s, const int32_t* d_e, int32_t m,
                                int32_t n_tokens, int32_t tau, uint32_t mode,
                                const kvr_meta* meta, const kvr_repair_set* out,
                                int32_t* h_counts, hipStream_t stream);

/*
 * kvr_check_support - checks an explicit support before execution, as the
 * budgeted-repair page requires (section 13.2 / 7.1): d_T (device int32 [B])
 * strictly increasing (hence unique) and inside [first_selectable,
 * n_tokens), the retained suffix being the only selectable part.  d_gpos
 * (device int32 [n_tokens], or NULL for the identity g_t = t) is the global
 * position map of kvr_meta (cross-attention reuse page, 6.2); when given it
 * is checked in the same pass to be non-negative and strictly increasing.
 * d_result is a device int32 scratch word.  Synchronises the stream.
 * Returns KVR_OK, KVR_ERR_BAD_SUPPORT (support), or KVR_ERR_INVALID_ARGUMENT
 * (position map; also for B > n_tokens or NULL / misaligned pointers).
 * B = 0 is valid.
 */
kvr_status kvr_check_support(const int32_t* d_T, int32_t B, int32_t n_tokens,
                             int32_t first_selectable, const int32_t* d_gpos,
                             int32_t* d_result, hipStream_t stream);

/*
 * Validation mode.  With KVR_VALIDATE set in the environment to anything but
 * "0" (read on every call), kvr_layer_repair and kvr_stack_repair run this
 * check on d_T over [0, n_tokens) together with meta->gpos, and
 * kvr_biased_attention / kvr_biased_attention_noalloc run it on d_pos, on
 * the device before any other launch (the result word lives in the
 * workspace or scratch).  A bad support then returns KVR_ERR_BAD_SUPPORT (a
 * bad position map KVR_ERR_INVALID_ARGUMENT) with the cache, flags and
 * outputs untouched.  The check synchronises the stream, so calls made in
 * validation mode cannot be captured into a HIP graph.  Off by default:
 * callers that build their supports with kvr_build_repair_set,
 * kvr_build_runs or kvr_sur_select already hold checked supports.
 */

/*
 * kvr_build_runs - checks an explicit support like kvr_check_support and
 * coalesces it into its maximal runs of consecutive positions, the execution
 * intervals that Budgeted KV-Cache Repair sorts and coalesces a support into
 * (section 3.2, the end of Algorithm 1) and that sequential maximal-interval
 * replay (section 7.1) traverses one at a time.  Seam sets get their runs
 * from kvr_build_repair_set; this call covers every other support (isolated
 * tokens, intervals, supports chosen by Semantic-Unit Refresh elsewhere).
 *
 *   d_T        device int32 [B], the support (not modified).
 *   out        out->run_start and out->run_len: device int32 [out->cap]
 *              each, out->cap >= B; out->counts: device int32 [3] receives
 *              (B, R, status) with status KVR_OK or KVR_ERR_BAD_SUPPORT (then
 *              the runs are undefined).  out->T is not used (may be NULL).
 *   h_counts   host int32 [3] or NULL.  When given, counts are copied back,
 *              the stream is synchronised and the device status is returned.
 *              When NULL the call does not synchronise.
 * Errors (before any device work): B < 0 or B > n_tokens, NULL or
 * misaligned pointers, cap < B -> INVALID_ARGUMENT.  B = 0 gives R = 0.
 */
kvr_status kvr_build_runs(const int32_t* d_T, int32_t B, int32_t n_tokens,
                          int32_t first_selectable, const kvr_repair_set* out,
                          int32_t* h_counts, hipStream_t stream);

/*
 * kvr_build_plan - reusable attention plan (Budgeted KV-Cache Repair,
 * section 13.2, Eq. 23-24) for a sorted support d_T [B] and GQA group size
 * `group` (= Hq/Hkv).  Query tile t covers pairs [t*QROWS, min(B*group,
 * (t+1)*QROWS)); with u_min / u_max the positions of its first / last pair:
 * d_n_full[t] = floor((u_min+1)/KV_TILE), d_n_total[t] =
 * ceil((u_max+1)/KV_TILE).  Both outputs are device int32
 * [ceil(B*group/QROWS)].  kvr_layer_repair / kvr_stack_repair build the
 * same plan in their workspace; this entry point exposes it for checking.
 */
kvr_status kvr_build_plan(const int32_t* d_T, int32_t B, int32_t group, int32_t* d_n_full,
                          int32_t* d_n_total, hipStream_t stream);

/*
 * kvr_build_tile_map - the key-tile-major view of the same plan: for each
 * KV_TILE-key tile c of an n_tokens cache, d_first_q[c] is the index of the
 * first packed row r whose position d_T[r] is at or after the tile's first
 * key, i.e. the first query of the sorted support that sees any key of the
 * tile (every later row sees it too), or B when no row reaches the tile.
 * It inverts Eq. 24 (Budgeted KV-Cache Repair, section 13.2): query tile t
 * touches key tile c exactly when its last row index is >= d_first_q[c].
 * The attention kernels walk query tiles with n_full / n_total; this table
 * serves a traversal by key tile and inspection.
 *
 *   d_T        device int32 [B], strictly increasing (checked by
 *              kvr_check_support, not here); may be NULL when B = 0.
 *   d_first_q  device int32 [ceil(n_tokens / KV_TILE)].
 * Errors (before any device work): n_tokens < 1, B < 0 or B > n_tokens,
 * NULL or misaligned pointers -> INVALID_ARGUMENT.  Does not synchronise.
 */
kvr_status kvr_build_tile_map(const int32_t* d_T, int32_t B, int32_t n_tokens,
                              int32_t* d_first_q, hipStream_t stream);

/* Workspace bytes needed by kvr_layer_repair / kvr_stack_repair for this
 * shape, support size B and context length; 0 on invalid arguments. */
size_t kvr_workspace_bytes(const kvr_config* cfg, int32_t B, int32_t n_tokens);

/*
 * kvr_layer_repair - one layer of the layer-major packed recurrence
 * (Budgeted KV-Cache Repair, section 13.2) with the biased operator F in
 * physical-repair mode (cross-attention reuse page, 6.4):
 *
 *   n = RMSNorm(x) * attn_norm; q, k, v = n Wq^T (+bq), n Wk^T (+bk),
 *   n Wv^T (+bv); RoPE on q, k at each row's global position
 *   g_{u_r} (meta->gpos[T[r]], or u_r = T[r] itself when gpos is NULL);
 *   before attention: cache.k[u_r] = k, cache.v[u_r] = v (rounded to
 *   cfg.dtype), flags[u_r] &= ~(LOCAL | SINK)  (Eq. 21; type <- global);
 *   o = softmax_j(<q, k_j>/sqrt(d) + alpha*local_j + beta*sink_j) v_j over
 *   j = 0..u_r inclusive (Eq. 22 with the 6.4 logit form), query head h
 *   reading KV head h / (Hq/Hkv);
 *   h1 = x + o Wo^T;  y = h1 + Wdown(SiLU(n2 Wgate^T) * (n2 Wup^T)),
 *   n2 = RMSNorm(h1) * mlp_norm.
 *
 *   d_T        device int32 [B], strictly increasing, in [0, N) (checked by
 *              kvr_check_support, or here in validation mode).
 *   x_in       device float32 [x_in_rows, hidden]: x_in_rows == B means the
 *              rows are already packed in the order of T; x_in_rows ==
 *              meta->n_tokens means row r is gathered from x_in[T[r]].
 *   x_out      device float32 [B, hidden], packed in the order of T.  It may
 *              alias x_in when x_in_rows == B.
 *   cache, meta  updated in place at the rows T only; every other cache row
 *              and flag byte is left bit-identical.
 *   ws         device workspace of at least kvr_workspace_bytes() bytes.
 *
 * Errors (before any device work): null or misaligned pointers;
 * head_dim not 64/128, Hq % Hkv != 0, hidden or intermediate not a multiple
 * of 64 -> UNSUPPORTED; B < 0, B > N, x_in_rows not in {B, N}, non-finite
 * alpha/beta/eps -> INVALID_ARGUMENT; ws_bytes too small -> WORKSPACE.
 * B = 0 is a successful no-op.
 */
kvr_status kvr_layer_repair(const kvr_config* cfg, const kvr_layer_weights* w, kvr_kv cache,
                            const kvr_meta* meta, const int32_t* d_T, int32_t B,
                            const float* x_in, int32_t x_in_rows, float* x_out, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/*
 * kvr_stack_repair - the layer-major traversal (Budgeted KV-Cache Repair,
 * section 3.3): rows T are gathered once and advance through layers
 * 0..n_layers-1 together, each layer as in kvr_layer_repair, reusing one
 * plan and one RoPE table built once per call.  w and caches are host
 * arrays of n_layers entries.  x_out receives the last layer's packed output
 * and is also the packed residual stream between layers.  Same argument
 * rules and errors as kvr_layer_repair.
 */
kvr_status kvr_stack_repair(const kvr_config* cfg, int32_t n_layers, const kvr_layer_weights* w,
                            const kvr_kv* caches, const kvr_meta* meta, const int32_t* d_T,
                            int32_t B, const float* x_in, int32_t x_in_rows, float* x_out,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes needed by kvr_biased_attention for B query rows over an
 * n_tokens-position cache; 0 on invalid arguments. */
size_t kvr_attention_workspace_bytes(const kvr_config* cfg, int32_t B, int32_t n_tokens);

/*
 * kvr_biased_attention - the operator F in inference mode (cross-attention
 * reuse page, 6.4, "prefill / decode, inference mode"): attention only, over
 * the mixed cache with the metadata logit bias, and no write-back:
 *
 *   o[r, h] = sum_j softmax_j(<q[r, h], k_j>/sqrt(d) + alpha*local_j +
 *             beta*sink_j) v_j   over j = 0..d_pos[r] inclusive,
 *
 * keys and values of KV head h / (Hq/Hkv).  The query at position u sees
 * its own position, as the repair's attention does; a decode step writes
 * the new token's K/V at u (and its flags byte) before calling.
 *
 *   q        device float32 [B, Hq, d], post-RoPE (rotated at d_pos[r]).
 *   d_pos    device int32 [B], strictly increasing, in [0, n_tokens)
 *            (checkable with kvr_check_support, not checked here).
 *   cache    K, V [n_tokens, Hkv, d] in cfg->dtype; read only.
 *   flags    device uint8 [n_tokens] (KVR_FLAG_LOCAL | KVR_FLAG_SINK); read only.
 *   o        device float32 [B, Hq, d]; must not alias q.
 *   ws       device workspace of at least kvr_attention_workspace_bytes() bytes.
 *
 * Only cfg's dtype, head counts, head_dim, alpha and beta are read.
 * Errors (before any device work): null or misaligned (16-byte) pointers,
 * o == q, B < 0, B > n_tokens -> INVALID_ARGUMENT; head_dim not 64/128 or
 * Hq % Hkv != 0 -> UNSUPPORTED; ws_bytes too small -> WORKSPACE.  B = 0 is a
 * successful no-op.
 */
kvr_status kvr_biased_attention(const kvr_config* cfg, kvr_kv cache, const uint8_t* flags,
                                int32_t n_tokens, const float* q, const int32_t* d_pos,
                                int32_t B, float* o, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/*
 * kvr_biased_attention_noalloc - kvr_biased_attention without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops (a decode step per token), harnesses
 * that forbid hipMalloc.  The call allocates nothing; its scratch is a
 * static device array of KVR_NOALLOC_SCRATCH_BYTES held by the library on
 * every GPU it runs on until the process ends (looked up once per device on
 * the first call there).  Same arguments, results and errors as
 * kvr_biased_attention, plus KVR_ERR_WORKSPACE when the shape needs more
 * scratch than that (kvr_attention_workspace_bytes() - 256 >
 * KVR_NOALLOC_SCRATCH_BYTES).  A bf16 decode call (B * Hq/Hkv <= 64) needs
 * at most 256 * B * (Hq/Hkv) * (d + 2) * 4 bytes whatever N (8.5 MB at 64
 * pairs per KV head, d = 128), so every decode call fits; larger B take the
 * packed attention path, whose scratch grows with B and N (33 MB for B = 64
 * over N = 16384 at the 7B shape, beyond the limit).  All calls on one GPU
 * share that GPU's scratch, which keeps
 * the last call's contents: calls that overlap in time on one GPU
 * (different streams or threads) race and must be serialised by the caller.
 */
enum { KVR_NOALLOC_SCRATCH_BYTES = 32 << 20 };
kvr_status kvr_biased_attention_noalloc(const kvr_config* cfg, kvr_kv cache,
                                        const uint8_t* flags, int32_t n_tokens, const float* q,
                                        const int32_t* d_pos, int32_t B, float* o,
                                        hipStream_t stream);

/*
 * kvr_shift_cache - the Shift step that precedes a repair (Budgeted KV-Cache
 * Repair, section 7.1, Eq. 2): delete positions [del_start, del_start +
 * del_len) of the cached sequence and position-correct the retained suffix.
 * For every layer, destination row r is
 *   r <  del_start:  src row r, copied bit for bit;
 *   r >= del_start:  src row i = r + del_len with K~ = R_{i-d} R_i^{-1} K_i
 *                    and V~ = V_i, where d = del_len and R_i is the rotary
 *                    map with rope_theta, rotate-half pairing (j, j + d_h/2).
 * R_{i-d} R_i^{-1} turns pair j by -d * theta^(-2j/d_h) whatever i is; the
 * cosine and sine are evaluated in float64 and the rotation in float32, then
 * rounded to cfg->dtype.
 *
 *   src, dst        host arrays [n_layers] of caches: src K, V [n_tokens, Hkv,
 *                   d_h], dst K, V [n_tokens - del_len, Hkv, d_h], cfg->dtype.
 *                   No dst buffer may overlap any src buffer (not in place).
 *   flags_src/dst   device uint8 [n_tokens] -> [n_tokens - del_len], moved
 *                   with their rows; `mark` is OR-ed into every moved suffix
 *                   row (e.g. KVR_FLAG_LOCAL: the shifted keys still carry
 *                   the deleted span's influence).  Both NULL: no flags.
 *   block_src/dst   device int32 block ids, moved likewise (both NULL or both set).
 *
 * Only cfg's dtype, head counts, head_dim and rope_theta are read.
 * Errors (before any device work): null or misaligned (16-byte) pointers,
 * overlapping src/dst, n_layers < 1, del_start < 0, del_len < 0,
 * del_start + del_len > n_tokens, non-positive rope_theta ->
 * INVALID_ARGUMENT; head_dim not 64/128 -> UNSUPPORTED.  del_len = 0 copies.
 */
kvr_status kvr_shift_cache(const kvr_config* cfg, int32_t n_layers, const kvr_kv* src,
                           const kvr_kv* dst, const uint8_t* flags_src, uint8_t* flags_dst,
                           const int32_t* block_src, int32_t* block_dst, int32_t n_tokens,
                           int32_t del_start, int32_t del_len, uint8_t mark,
                           hipStream_t stream);

/*
 * kvr_sur_scores - token relevance of Semantic-Unit Refresh (Budgeted
 * KV-Cache Repair, section 3.2, Eq. 1, and section 7.3, Eq. 7), in float32
 * as the page prescribes for normalisation and cosine scoring:
 *
 *   r[i] = max_{j < Q} <E[s_i], E[q_j]> / (||E[s_i]||_2 ||E[q_j]||_2)
 *          + 0.25 * 1[s_i occurs among the query ids]
 *
 * A zero-norm row scores cosine 0.  bf16 tables are contracted on the MFMA
 * (products exact in float32, float32 sums); float32 tables in float32 FMA.
 *
 *   d_E           device [vocab, hidden] embedding table in `dtype`.
 *   d_suffix_ids  device int32 [S]: token ids of the retained suffix.
 *   d_query_ids   device int32 [Q], 1 <= Q <= 256.
 *   d_r           device float32 [S] out.  A token id outside [0, vocab)
 *                 gives r = NaN for that token (no row is read out of range).
 * Errors (before any device work): null or misaligned (16-byte) pointers,
 * vocab < 1, S < 0, Q outside [1, 256] -> INVALID_ARGUMENT; hidden not a
 * positive multiple of 64, or above 8192 for a float32 table -> UNSUPPORTED.
 * S = 0 is a successful no-op.
 */
kvr_status kvr_sur_scores(const void* d_E, kvr_dtype dtype, int32_t vocab, int32_t hidden,
                          const int32_t* d_suffix_ids, int32_t S, const int32_t* d_query_ids,
                          int32_t Q, float* d_r, hipStream_t stream);

/*
 * kvr_sur_select - the selection of Semantic-Unit Refresh under an exact
 * budget (Budgeted KV-Cache Repair, section 7.3, the selection part of
 * Algorithm 1): each unit scores the mean of its four largest token scores
 * (all of them below four); units are ranked by score, the earlier unit
 * winning a tie; whole units are admitted in ranked order while they fit the
 * remaining allowance w = budget - |A|; the first that does not fit
 * contributes the width-w window with the largest sum of the forward-decay
 * envelope u_t = max(e^(r_t - r_max), e^(-1/16) u_{t-1}), u_0 = 0 (Eq. 8),
 * the earliest on ties, which fills the allowance exactly; the chosen
 * positions are sorted and coalesced into runs.
 *
 *   d_r            device float32 [S] token scores (kvr_sur_scores).
 *   d_unit_start   device int32 [n_units]: the suffix partition into units,
 *                  unit u = [start[u], start[u+1]) with start[n_units] = S.
 *                  start[0] = 0 and strictly increasing below S, checked on
 *                  the device (KVR_ERR_BAD_BLOCKS in counts[2]).
 *   budget         |A|, 0 <= budget <= S (the exact budget of Eq. 3 is the
 *                  caller's: min(S, ceil(S * b / 100))).
 *   pos0           global position of suffix token 0: T holds pos0 + i.
 *   d_unit_scores  device float32 [n_units] out: the unit scores.
 *   out            T, run_start, run_len: device int32 [cap] each; counts:
 *                  device int32 [3] = (|T|, R, status); cap >= budget.
 *   d_ws           device workspace of at least 2 * S floats.
 *   h_counts       host int32 [3] or NULL: when given the call synchronises
 *                  the stream, copies counts and returns their status.
 * Errors (before any device work): null or misaligned pointers, S < 1,
 * n_units outside [1, S], budget outside [0, S], cap < budget, ws_bytes too
 * small -> INVALID_ARGUMENT / WORKSPACE; n_units > 8192 -> UNSUPPORTED.
 */
kvr_status kvr_sur_select(const float* d_r, int32_t S, const int32_t* d_unit_start,
                          int32_t n_units, int32_t budget, int32_t pos0, float* d_unit_scores,
                          const kvr_repair_set* out, float* d_ws, size_t ws_bytes,
                          int32_t* h_counts, hipStream_t stream);

/* Human-readable name of a status. */
const char* kvr_status_string(kvr_status s);
/* Detail of the last error returned on the calling thread ("" if none). */
const char* kvr_last_error(void);

/*
 * Kernel timing probe.  kvr_timing_begin(mask) makes the library bracket
 * every later launch of the kernels whose KVR_KERNEL_* bit is in `mask` with
 * a pair of HIP events on the launch stream.  kvr_timing_end() waits for
 * them and writes, for each of the KVR_KERNEL_COUNT kernels, the summed
 * elapsed milliseconds (host double [KVR_KERNEL_COUNT]) and the number of
 * launches (host int32 [KVR_KERNEL_COUNT]); either may be NULL.  Timing is
 * process-wide and not thread-safe.
 */
enum {
  KVR_KERNEL_PLAN = 0,      /* attention plan (kvr_biased_attention, float32) */
  KVR_KERNEL_NORM = 1,      /* gather / residual sum + RMSNorm (the first
                               launch of a repair also builds its plan and
                               RoPE table)                               */
  KVR_KERNEL_QKV = 2,       /* QKV projection GEMM                         */
  KVR_KERNEL_ROPE = 3,      /* RoPE + K/V write-back + flags               */
  KVR_KERNEL_ATTN = 4,      /* packed causal attention                     */
  KVR_KERNEL_ATTN_MERGE = 5,/* split-KV merge                              */
  KVR_KERNEL_OPROJ = 6,     /* O projection GEMM                           */
  KVR_KERNEL_GATEUP = 7,    /* gate/up GEMM with SwiGLU epilogue           */
  KVR_KERNEL_DOWN = 8,      /* down projection GEMM                        */
  KVR_KERNEL_FINAL = 9,     /* last residual sum into x_out                */
  KVR_KERNEL_QPREP = 10,    /* query scaling and attention plan
                               (kvr_biased_attention, bf16)                 */
  KVR_KERNEL_SHIFT = 11,    /* Shift re-rotation / move (kvr_shift_cache)  */
  KVR_KERNEL_SUR_SCORE = 12,/* SUR token relevance (kvr_sur_scores)        */
  KVR_KERNEL_SUR_SELECT = 13,/* SUR unit scores + selection (kvr_sur_select) */
  KVR_KERNEL_COUNT = 14
};
kvr_status kvr_timing_begin(uint32_t mask);
kvr_status kvr_timing_end(double* total_ms, int32_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* KVR_H */
