// Integer kernels of the repair: the seam set T_tau and its runs, load-time
// metadata, support validation, the per-query-tile attention plan (the
// layer path builds it, with the per-row RoPE table, inside its first row
// kernel: tables.h) and the key-tile map.
//
// Seam windows and the asymmetric true-prefix rule: cross-attention reuse
// specification page, section 6.3.  Runs are the execution intervals of
// "Budgeted KV-Cache Repair", section 3.2.  Plan: same page, section 13.2,
// Eq. 23-24.
#include "kvr_internal.h"
#include "tables.h"

namespace kvr {

namespace {

constexpr int kBuildThreads = 1024;
// T and the run openings are also kept in LDS up to this many entries, so
// the run pass reads them back without a round trip to memory.
constexpr int kBuildLds = 4096;

// Exclusive prefix sum over a 1024-thread workgroup; *total gets the sum.
__device__ int block_exclusive_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wid] = x;
  __syncthreads();
  int pre = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    const int w = wsum[i];
    pre += (i < wid) ? w : 0;
    tot += w;
  }
  __syncthreads();
  *total = tot;
  return pre + x - v;
}

// Maximal runs of the sorted positions t_at(0..total-1): T[k] opens a run
// unless T[k] == T[k-1] + 1 (the execution intervals of "Budgeted KV-Cache
// Repair", section 3.2).  Writes run_start / run_len and returns R; every
// thread of the 1024-thread workgroup gets R.  run_len first holds each run's
// opening index in T, then its length; the openings are also kept in LDS
// (sOpen) while R <= kBuildLds, else the lengths are fixed up chunk by chunk
// from global memory between barriers.
template <class TAt>
__device__ int emit_runs(TAt t_at, int total, int32_t* __restrict__ run_start,
                         int32_t* __restrict__ run_len, int* sOpen, int* wsum) {
  const int tid = threadIdx.x;
  int nruns = 0;
  for (int base = 0; base < total; base += blockDim.x) {
    const int k = base + tid;
    const int open = (k < total) && (k == 0 || t_at(k) != t_at(k - 1) + 1);
    int chunk;
    const int id = nruns + block_exclusive_scan(open, wsum, &chunk);
    if (open) {
      run_start[id] = t_at(k);
      if (id < kBuildLds) sOpen[id] = k;
      run_len[id] = k;
    }
    nruns += chunk;
  }
  __threadfence_block();
  __syncthreads();
  if (nruns <= kBuildLds) {
    for (int j = tid; j < nruns; j += blockDim.x)
      run_len[j] = ((j + 1 < nruns) ? sOpen[j + 1] : total) - sOpen[j];
  } else {
    for (int base = 0; base < nruns; base += blockDim.x) {
      const int j = base + tid;
      int len = 0;
      if (j < nruns) len = ((j + 1 < nruns) ? run_len[j + 1] : total) - run_len[j];
      __syncthreads();
      if (j < nruns) run_len[j] = len;
      __threadfence_block();
      __syncthreads();
    }
  }
  return nruns;
}

// Positions of block i that belong to T_tau: at most two half-open ranges
// [a0, a1) (leading window, merged with the trailing one when they touch)
// and [b0, b1) (trailing window).
struct BlockRanges {
  int a0, a1, b0, b1;
  __device__ int count() const { return (a1 - a0) + (b1 - b0); }
};

__device__ BlockRanges block_ranges(int i, int m, int si, int ei, int tau, bool asym) {
  const bool lead = i >= 1;
  const bool trail = (i < m - 1 && !(asym && i == 0)) || (asym && m >= 2 && i == m - 1);
  const int la = si, lb = lead ? min(ei, si + tau) : si;
  const int ta = trail ? max(si, ei - tau) : ei, tb = ei;
  BlockRanges r;
  if (lb >= ta) {  // windows overlap or touch: one range
    r.a0 = la; r.a1 = tb; r.b0 = tb; r.b1 = tb;
  } else {
    r.a0 = la; r.a1 = lb; r.b0 = ta; r.b1 = tb;
  }
  return r;
}

__global__ __launch_bounds__(kBuildThreads) void k_build_repair_set(
    const int32_t* __restrict__ s, const int32_t* __restrict__ e, int m, int n_tokens, int tau,
    int asym, int32_t* __restrict__ T, int32_t* __restrict__ run_start,
    int32_t* __restrict__ run_len, int32_t* __restrict__ counts, int cap) {
  __shared__ int wsum[16];
  __shared__ int s_bad;
  __shared__ int sT[kBuildLds];      // T, when it fits
  __shared__ int sOpen[kBuildLds];   // index in T of each run's first position, when they fit
  const int tid = threadIdx.x;
  if (tid == 0) s_bad = 0;
  __syncthreads();

  // 1. the blocks must tile [0, N): s_1 = 0, e_i = s_{i+1}, e_m = N, non-empty
  for (int i = tid; i < m; i += blockDim.x) {
    const int si = s[i], ei = e[i];
    const bool bad = !(si < ei) || (i == 0 && si != 0) || (i == m - 1 && ei != n_tokens) ||
                     (i + 1 < m && ei != s[i + 1]);
    if (bad) atomicOr(&s_bad, 1);
  }
  __syncthreads();
  if (s_bad) {
    if (tid == 0) { counts[0] = 0; counts[1] = 0; counts[2] = KVR_ERR_BAD_BLOCKS; }
    return;
  }

  // 2. |T| = sum of per-block counts; check capacity before writing
  int total = 0;
  for (int base = 0; base < m; base += blockDim.x) {
    const int i = base + tid;
    const int c = i < m ? block_ranges(i, m, s[i], e[i], tau, asym != 0).count() : 0;
    int chunk;
    block_exclusive_scan(c, wsum, &chunk);
    total += chunk;
  }
  if (total > cap) {
    if (tid == 0) { counts[0] = total; counts[1] = 0; counts[2] = KVR_ERR_CAPACITY; }
    return;
  }

  // 3. fill T: block i writes its ranges at its exclusive offset
  const bool lds_t = total <= kBuildLds;
  int off0 = 0;
  for (int base = 0; base < m; base += blockDim.x) {
    const int i = base + tid;
    BlockRanges r{0, 0, 0, 0};
    if (i < m) r = block_ranges(i, m, s[i], e[i], tau, asym != 0);
    int chunk;
    int off = off0 + block_exclusive_scan(i < m ? r.count() : 0, wsum, &chunk);
    for (int t = r.a0; t < r.a1; ++t) {
      if (lds_t) sT[off] = t;
      T[off++] = t;
    }
    for (int t = r.b0; t < r.b1; ++t) {
      if (lds_t) sT[off] = t;
      T[off++] = t;
    }
    off0 += chunk;
  }
  __threadfence_block();
  __syncthreads();
  auto t_at = [&](int k) { return lds_t ? sT[k] : T[k]; };

  // 4. maximal runs
  const int nruns = emit_runs(t_at, total, run_start, run_len, sOpen, wsum);
  if (tid == 0) { counts[0] = total; counts[1] = nruns; counts[2] = KVR_OK; }
}

// Load-time metadata (6.2): block 1 global, later blocks local; the first
// token of every block after the first is a spurious sink.  Skipped when the
// build reported bad blocks.
__global__ void k_init_meta(const int32_t* __restrict__ s, const int32_t* __restrict__ e, int m,
                            int n_tokens, const int32_t* __restrict__ counts,
                            uint8_t* __restrict__ flags, int32_t* __restrict__ block_id) {
  if (counts[2] == KVR_ERR_BAD_BLOCKS) return;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_tokens) return;
  int lo = 0, hi = m - 1;  // largest i with s[i] <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s[mid] <= t) lo = mid; else hi = mid - 1;
  }
  uint8_t f = 0;
  if (t >= e[0]) f |= KVR_FLAG_LOCAL;
  if (lo >= 1 && t == s[lo]) f |= KVR_FLAG_SINK;
  flags[t] = f;
  if (block_id) block_id[t] = lo;
}

// An explicit support (any sorted selection, e.g. isolated tokens or a
// contiguous interval): check it as kvr_check_support does, then coalesce it
// into its maximal runs.  counts = (B, R, status).
__global__ __launch_bounds__(kBuildThreads) void k_build_runs(
    const int32_t* __restrict__ T, int B, int n_tokens, int first,
    int32_t* __restrict__ run_start, int32_t* __restrict__ run_len,
    int32_t* __restrict__ counts) {
  __shared__ int wsum[16];
  __shared__ int s_bad;
  __shared__ int sOpen[kBuildLds];
  const int tid = threadIdx.x;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  for (int k = tid; k < B; k += blockDim.x) {
    const int t = T[k];
    if (t < first || t < 0 || t >= n_tokens || (k > 0 && T[k - 1] >= t))
      atomicOr(&s_bad, 1);
  }
  __syncthreads();
  if (s_bad) {
    if (tid == 0) { counts[0] = B; counts[1] = 0; counts[2] = KVR_ERR_BAD_SUPPORT; }
    return;
  }
  const int nruns = emit_runs([&](int k) { return T[k]; }, B, run_start, run_len, sOpen, wsum);
  if (tid == 0) { counts[0] = B; counts[1] = nruns; counts[2] = KVR_OK; }
}

// Support check (strictly increasing, inside [first, n_tokens)) and, when
// gpos is given, the global-position map: non-negative and strictly
// increasing over all n_tokens rows, so that causal visibility by global
// position (g_j <= g_u) is visibility by row (j <= u).
__global__ __launch_bounds__(kBuildThreads) void k_check_support(
    const int32_t* __restrict__ T, int B, int n_tokens, int first,
    const int32_t* __restrict__ gpos, int32_t* __restrict__ result) {
  __shared__ int s_bad, s_bad_pos;
  if (threadIdx.x == 0) { s_bad = 0; s_bad_pos = 0; }
  __syncthreads();
  for (int k = threadIdx.x; k < B; k += blockDim.x) {
    const int t = T[k];
    if (t < first || t < 0 || t >= n_tokens || (k > 0 && T[k - 1] >= t))
      atomicOr(&s_bad, 1);
  }
  if (gpos) {
    for (int t = threadIdx.x; t < n_tokens; t += blockDim.x) {
      const int g = gpos[t];
      if (g < 0 || (t > 0 && gpos[t - 1] >= g)) atomicOr(&s_bad_pos, 1);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0)
    result[0] = s_bad ? KVR_ERR_BAD_SUPPORT : (s_bad_pos ? KVR_ERR_INVALID_ARGUMENT : KVR_OK);
}

__global__ void k_build_plan(const int32_t* __restrict__ T, int B, int group, int n_tiles,
                             int32_t* __restrict__ n_full, int32_t* __restrict__ n_total) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n_tiles) plan_entry(T, B, group, t, n_full, n_total);
}

// Key tile c's first packed row: the left insertion point of c * KV_TILE
// into the sorted support (one thread per key tile, binary search).
__global__ void k_tile_map(const int32_t* __restrict__ T, int B, int n_kv,
                           int32_t* __restrict__ first_q) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= n_kv) return;
  const long long key0 = static_cast<long long>(c) * KVR_ATTN_KV_TILE;
  int lo = 0, hi = B;   // first r in [lo, hi) with T[r] >= key0
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (T[mid] < key0) lo = mid + 1; else hi = mid;
  }
  first_q[c] = lo;
}


}  // namespace

hipError_t launch_build_repair_set(const int32_t* s, const int32_t* e, int m, int n_tokens,
                                   int tau, bool asym, int32_t* T, int32_t* run_start,
                                   int32_t* run_len, int32_t* counts, int cap,
                                   hipStream_t stream) {
  hipLaunchKernelGGL(k_build_repair_set, dim3(1), dim3(kBuildThreads), 0, stream, s, e, m,
                     n_tokens, tau, asym ? 1 : 0, T, run_start, run_len, counts, cap);
  return hipGetLastError();
}

hipError_t launch_init_meta(const int32_t* s, const int32_t* e, int m, int n_tokens,
                            const int32_t* counts, uint8_t* flags, int32_t* block_id,
                            hipStream_t stream) {
  if (n_tokens <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_init_meta, dim3((n_tokens + 255) / 256), dim3(256), 0, stream, s, e, m,
                     n_tokens, counts, flags, block_id);
  return hipGetLastError();
}

hipError_t launch_check_support(const int32_t* T, int B, int n_tokens, int first,
                                const int32_t* gpos, int32_t* result, hipStream_t stream) {
  hipLaunchKernelGGL(k_check_support, dim3(1), dim3(kBuildThreads), 0, stream, T, B, n_tokens,
                     first, gpos, result);
  return hipGetLastError();
}

hipError_t launch_build_runs(const int32_t* T, int B, int n_tokens, int first,
                             int32_t* run_start, int32_t* run_len, int32_t* counts,
                             hipStream_t stream) {
  hipLaunchKernelGGL(k_build_runs, dim3(1), dim3(kBuildThreads), 0, stream, T, B, n_tokens,
                     first, run_start, run_len, counts);
  return hipGetLastError();
}

int plan_tiles(int B, int group) { return (B * group + KVR_ATTN_QROWS - 1) / KVR_ATTN_QROWS; }

hipError_t launch_build_plan(const int32_t* T, int B, int group, int32_t* n_full,
                             int32_t* n_total, hipStream_t stream) {
  const int nt = plan_tiles(B, group);
  if (nt == 0) return hipSuccess;
  hipLaunchKernelGGL(k_build_plan, dim3((nt + 255) / 256), dim3(256), 0, stream, T, B, group, nt,
                     n_full, n_total);
  return hipGetLastError();
}

hipError_t launch_tile_map(const int32_t* T, int B, int n_tokens, int32_t* first_q,
                           hipStream_t stream) {
  const int n_kv = (n_tokens + KVR_ATTN_KV_TILE - 1) / KVR_ATTN_KV_TILE;
  if (n_kv == 0) return hipSuccess;
  hipLaunchKernelGGL(k_tile_map, dim3((n_kv + 255) / 256), dim3(256), 0, stream, T, B, n_kv,
                     first_q);
  return hipGetLastError();
}

}  // namespace kvr
