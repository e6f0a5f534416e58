// Numeric core of Semantic-Unit Refresh ("Budgeted KV-Cache Repair",
// sections 3.2 and 7.3): token relevance from the frozen embedding table
// (Eq. 1 / 7), unit scores and ranking, the exact-budget fill of Algorithm 1
// with the forward-decay envelope window (Eq. 8) for the unit that does not
// fit, and the sort-and-coalesce of the chosen positions into T and its runs.
//
// Scoring is float32 as the page prescribes: bf16 tables feed the MFMA,
// whose products are exact in float32 and whose sums are float32; float32
// tables take a float32 FMA path.
#include <cmath>

#include "common.h"
#include "kvr_internal.h"

namespace kvr {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kScoreThreads = 256;   // 4 waves: 32 suffix tokens, hidden in quarters
constexpr int kSurMaxQ = 256;        // query tokens (8 blocks of 32)

__device__ __forceinline__ bool id_ok(int id, int vocab) { return id >= 0 && id < vocab; }

// bf16 table, general shapes (any hidden multiple of 64, Q up to 256):
// workgroup = 32 suffix tokens, its 4 waves splitting the
// hidden dimension in quarters.  The MFMA forms D[query][token] (A = query
// rows, B = token rows, k along hidden), so a lane owns one token column and
// 16 query rows per 32-query block.  Both operands are read straight from
// global memory in MFMA layout (16 bytes per lane per k step): the token
// rows are streamed once, the query rows come from L2.  Squared norms
// accumulate from the same operand registers; the quarters are summed
// through LDS one query block at a time.
template <int QB>
__global__ __launch_bounds__(kScoreThreads) void k_sur_scores_mfma(
    const bf16_t* __restrict__ E, int vocab, int hidden, const int32_t* __restrict__ sid, int S,
    const int32_t* __restrict__ qid, int Q, float* __restrict__ r) {
  __shared__ int qids[kSurMaxQ];
  __shared__ float red[3][16][64];
  __shared__ float red_ss[3][QB + 1][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  for (int j = tid; j < Q; j += kScoreThreads) qids[j] = qid[j];
  __syncthreads();
  const int tok = blockIdx.x * 32 + (lane & 31);
  const int tc = min(tok, S - 1);
  const int id = sid[tc];
  const bool bad = !id_ok(id, vocab);
  const int quarter = hidden >> 2;
  const int k0 = wave * quarter;
  const bf16_t* trow = E + static_cast<size_t>(bad ? 0 : id) * hidden + k0 + 8 * half;
  const bf16_t* qrow[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qj = qids[min(qb * 32 + (lane & 31), Q - 1)];
    qrow[qb] = E + static_cast<size_t>(id_ok(qj, vocab) ? qj : 0) * hidden + k0 + 8 * half;
  }
  f32x16_t acc[QB];
  float tss = 0.f, qss[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    qss[qb] = 0.f;
#pragma unroll
    for (int t = 0; t < 16; ++t) acc[qb][t] = 0.f;
  }
#pragma unroll 4
  for (int k = 0; k < quarter; k += 16) {
    const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(trow + k);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = static_cast<float>(b[i]);
      tss = fmaf(x, x, tss);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(qrow[qb] + k);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = static_cast<float>(a[i]);
        qss[qb] = fmaf(x, x, qss[qb]);
      }
      acc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[qb], 0, 0, 0);
    }
  }
  // sum the quarters into wave 0
  if (wave > 0) {
    red_ss[wave - 1][QB][lane] = tss;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) red_ss[wave - 1][qb][lane] = qss[qb];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < 3; ++w) {
      tss += red_ss[w][QB][lane];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) qss[qb] += red_ss[w][qb][lane];
    }
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    if (wave > 0)
#pragma unroll
      for (int t = 0; t < 16; ++t) red[wave - 1][t][lane] = acc[qb][t];
    __syncthreads();
    if (wave == 0)
#pragma unroll
      for (int t = 0; t < 16; ++t) acc[qb][t] += red[0][t][lane] + red[1][t][lane] + red[2][t][lane];
    __syncthreads();
  }
  if (wave != 0) return;
  const float tn = sqrtf(xor32_add(tss));
  float best = -INFINITY;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float qn_mine = sqrtf(qss[qb] + __shfl_xor(qss[qb], 32, 64));   // query row lane % 32
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int row = 8 * (t >> 2) + 4 * half + (t & 3);
      const float qn = __shfl(qn_mine, row, 64);
      const float den = qn * tn;
      const float c = den > 0.f ? acc[qb][t] / den : 0.f;
      if (qb * 32 + row < Q) best = fmaxf(best, c);
    }
  }
  best = xor32_max(best);
  if (half == 0 && tok < S) {
    bool in_q = false;
    for (int j = 0; j < Q; ++j) in_q |= (qids[j] == id);
    r[tok] = bad ? NAN : best + (in_q ? 0.25f : 0.f);
  }
}

// bf16 table, query-stationary (hidden a multiple of kStatChunk, Q <= 128):
// a workgroup of 8 waves scores 64 suffix tokens.  The query rows are staged
// in LDS one hidden chunk of kStatChunk at a time (double-buffered; loaded
// with coalesced 16-byte lanes and shared by all 8 waves), so each query byte
// crosses L2 once per 64 tokens instead of once per 32, in whole lines.  Wave
// w owns tokens 16 (w % 4) .. +15 and the half w / 4 of every chunk; the
// token rows are read directly in 16x16x32 MFMA layout (4 lanes cover 64
// contiguous bytes of one row) through a register ring that prefetches the
// same steps of the next chunk.  D[query][token] accumulates in float32; the
// two halves meet in LDS at the end.  The query squared norms accumulate from
// the staging registers: the kStatChunk / 8 consecutive threads of a staging
// slot cover one query row.
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
constexpr int kStatWaves = 8;
constexpr int kStatThreads = 64 * kStatWaves;
constexpr int kStatTokens = 16 * kStatWaves / 2;      // 64 tokens per workgroup
constexpr int kStatChunk = 256;                        // hidden elements per staged chunk
constexpr int kStatHalf = kStatChunk / 2;              // per wave half
constexpr int kStatSteps = kStatHalf / 32;             // 16x16x32 k-steps per half chunk
constexpr int kStatRow16 = kStatChunk / 8;             // 16-byte pieces per staged row

// 16-byte piece c of staged query row r; the XOR keeps the MFMA operand
// reads (16 rows x 2 pieces per 32 lanes) and the staging writes free of
// LDS bank conflicts.
__device__ __forceinline__ int stat_off(int row, int c) {
  return row * kStatChunk + 8 * (c ^ ((2 * row) & 31));
}

template <int QB16>
__global__ __launch_bounds__(kStatThreads) void k_sur_scores_stat(
    const bf16_t* __restrict__ E, int vocab, int hidden, const int32_t* __restrict__ sid, int S,
    const int32_t* __restrict__ qid, int Q, float* __restrict__ r) {
  constexpr int QP = 16 * QB16;
  constexpr int SLOTS = QP * kStatRow16 / kStatThreads;
  static_assert(QP * kStatRow16 % kStatThreads == 0 && kStatThreads % kStatRow16 == 0, "staging map");
  constexpr int kXr = (kStatWaves / 2) * (4 * QB16 + 1) * 64;   // floats of the half exchange
  static_assert(kXr <= QP * kStatChunk, "exchange fits the staging buffers");
  __shared__ __attribute__((aligned(16))) bf16_t qs[2][QP * kStatChunk];
  __shared__ int qids[kSurMaxQ];
  __shared__ float qss_s[QP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g4 = lane >> 4;
  const int tg = wave % (kStatWaves / 2), h = wave / (kStatWaves / 2);
  for (int j = tid; j < Q; j += kStatThreads) qids[j] = qid[j];
  __syncthreads();
  // staging slot i of this thread: query row lin / kStatRow16, piece lin % kStatRow16
  const bf16_t* srow[SLOTS];
  int soff[SLOTS];
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const int lin = i * kStatThreads + tid, row = lin / kStatRow16, c = lin % kStatRow16;
    const int qj = qids[min(row, Q - 1)];
    srow[i] = E + static_cast<size_t>(id_ok(qj, vocab) ? qj : 0) * hidden + 8 * c;
    soff[i] = stat_off(row, c);
  }
  float qss[SLOTS];
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) qss[i] = 0.f;
  const int tok = blockIdx.x * kStatTokens + tg * 16 + (lane & 15);
  const int id = sid[min(tok, S - 1)];
  const bool bad = !id_ok(id, vocab);
  const int nch = hidden / kStatChunk;
  const bf16_t* trow = E + static_cast<size_t>(bad ? 0 : id) * hidden + h * kStatHalf + 8 * g4;
  bf16x8_t ring[kStatSteps];
#pragma unroll
  for (int u = 0; u < kStatSteps; ++u) ring[u] = *reinterpret_cast<const bf16x8_t*>(trow + 32 * u);
  {
    bf16x8_t st[SLOTS];
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) st[i] = *reinterpret_cast<const bf16x8_t*>(srow[i]);
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      *reinterpret_cast<bf16x8_t*>(&qs[0][soff[i]]) = st[i];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = static_cast<float>(st[i][e]);
        qss[i] = fmaf(x, x, qss[i]);
      }
    }
  }
  __syncthreads();
  f32x4_t acc[QB16];
#pragma unroll
  for (int qb = 0; qb < QB16; ++qb) acc[qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float tss = 0.f;
  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1;
    const bool more = c + 1 < nch;
    bf16x8_t st[SLOTS];
    if (more) {
#pragma unroll
      for (int i = 0; i < SLOTS; ++i)
        st[i] = *reinterpret_cast<const bf16x8_t*>(srow[i] + (c + 1) * kStatChunk);
    }
    const bf16_t* qb_base = qs[buf];
    const int nxt = min(c + 1, nch - 1) * kStatChunk;
#pragma unroll
    for (int u = 0; u < kStatSteps; ++u) {
      const bf16x8_t cur = ring[u];
      ring[u] = *reinterpret_cast<const bf16x8_t*>(trow + nxt + 32 * u);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = static_cast<float>(cur[e]);
        tss = fmaf(x, x, tss);
      }
      const int cq = 4 * (h * kStatSteps + u) + g4;
#pragma unroll
      for (int qb = 0; qb < QB16; ++qb) {
        const int row = qb * 16 + (lane & 15);
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(qb_base + stat_off(row, cq));
        acc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, cur, acc[qb], 0, 0, 0);
      }
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < SLOTS; ++i) {
        *reinterpret_cast<bf16x8_t*>(&qs[buf ^ 1][soff[i]]) = st[i];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = static_cast<float>(st[i][e]);
          qss[i] = fmaf(x, x, qss[i]);
        }
      }
    }
    __syncthreads();
  }
  // query norms: a slot's kStatRow16 consecutive threads share its row
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    float v = qss[i];
#pragma unroll
    for (int o = 1; o < kStatRow16; o <<= 1) v += __shfl_xor(v, o, 64);
    const int lin = i * kStatThreads + tid;
    if (lin % kStatRow16 == 0) qss_s[lin / kStatRow16] = v;
  }
  // the second half's partial products join the first half's through LDS
  // (the staging buffers are free after the loop's last barrier)
  float* xr = reinterpret_cast<float*>(&qs[0][0]) + tg * (4 * QB16 + 1) * 64;
  if (h == 1) {
#pragma unroll
    for (int qb = 0; qb < QB16; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) xr[(qb * 4 + i) * 64 + lane] = acc[qb][i];
    xr[4 * QB16 * 64 + lane] = tss;
  }
  __syncthreads();
  if (h != 0) return;
#pragma unroll
  for (int qb = 0; qb < QB16; ++qb)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[qb][i] += xr[(qb * 4 + i) * 64 + lane];
  tss += xr[4 * QB16 * 64 + lane];
  tss += __shfl_xor(tss, 16, 64);
  tss = xor32_add(tss);
  const float tn = sqrtf(tss);
  // D layout: lane holds token lane % 16, query rows 4 (lane / 16) + i
  float best = -INFINITY;
#pragma unroll
  for (int qb = 0; qb < QB16; ++qb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = qb * 16 + 4 * g4 + i;
      const float den = sqrtf(qss_s[row]) * tn;
      const float cv = den > 0.f ? acc[qb][i] / den : 0.f;
      if (row < Q) best = fmaxf(best, cv);
    }
  best = fmaxf(best, __shfl_xor(best, 16, 64));
  best = xor32_max(best);
  if (lane < 16 && tok < S) {
    bool in_q = false;
    for (int j = 0; j < Q; ++j) in_q |= (qids[j] == id);
    r[tok] = bad ? NAN : best + (in_q ? 0.25f : 0.f);
  }
}

// float32 table: one workgroup per suffix token; the token row is staged in
// LDS, each wave takes query tokens wave, wave + 4, ... with the lanes
// splitting the hidden dimension.
constexpr int kScoreMaxHidden = 8192;
__global__ __launch_bounds__(kScoreThreads) void k_sur_scores_f32(
    const float* __restrict__ E, int vocab, int hidden, const int32_t* __restrict__ sid,
    const int32_t* __restrict__ qid, int Q, float* __restrict__ r) {
  __shared__ float row[kScoreMaxHidden];
  __shared__ float wbest[4];
  __shared__ float red[16];
  const int i = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int id = sid[i];
  const bool bad = !id_ok(id, vocab);
  const float* trow = E + static_cast<size_t>(bad ? 0 : id) * hidden;
  float ss = 0.f;
  for (int k = tid; k < hidden; k += kScoreThreads) {
    row[k] = trow[k];
    ss = fmaf(row[k], row[k], ss);
  }
  const float tn = sqrtf(block_sum(ss, red));   // block_sum synchronises: row[] is complete
  float best = -INFINITY;
  bool in_q = false;
  for (int j = wave; j < Q; j += 4) {
    const int qj = qid[j];
    in_q |= (qj == id);
    const float* qr = E + static_cast<size_t>(id_ok(qj, vocab) ? qj : 0) * hidden;
    float dot = 0.f, qs = 0.f;
    for (int k = lane; k < hidden; k += 64) {
      const float x = qr[k];
      dot = fmaf(row[k], x, dot);
      qs = fmaf(x, x, qs);
    }
    dot = wave_sum(dot);
    qs = wave_sum(qs);
    const float den = sqrtf(qs) * tn;
    best = fmaxf(best, den > 0.f ? dot / den : 0.f);
  }
  if (lane == 0) wbest[wave] = best;
  const bool any_q = __syncthreads_or(in_q ? 1 : 0) != 0;
  if (tid == 0)
    r[i] = bad ? NAN
               : fmaxf(fmaxf(wbest[0], wbest[1]), fmaxf(wbest[2], wbest[3])) + (any_q ? 0.25f : 0.f);
}

// Unit score = mean of the unit's four largest token scores (all of them when
// it has fewer): one wave per unit, four rounds of a wave maximum, each
// removing one occurrence (the lowest index among equal values).  The sum
// runs from the largest down, as the reference does.
constexpr int kUnitWaves = 4;
__global__ __launch_bounds__(64 * kUnitWaves) void k_sur_unit_scores(
    const float* __restrict__ r, int S, const int32_t* __restrict__ ustart, int U,
    float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int u = blockIdx.x * kUnitWaves + (threadIdx.x >> 6);
  if (u >= U) return;
  const int a = ustart[u], b = (u + 1 < U) ? ustart[u + 1] : S;
  const int n = b - a;
  const int take = min(n, 4);
  float sum = 0.f;
  int rm0 = -1, rm1 = -1, rm2 = -1;   // indices taken by earlier rounds
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (k >= take) break;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int i = a + lane; i < b; i += 64) {
      const bool skip = (i == rm0) || (i == rm1) || (i == rm2);
      const float v = r[i];
      if (!skip && (v > bv || (v == bv && i < bi))) { bv = v; bi = i; }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (k == 0) rm0 = bi;
    else if (k == 1) rm1 = bi;
    else if (k == 2) rm2 = bi;
    sum += bv;
  }
  if (lane == 0) out[u] = sum / static_cast<float>(take);
}

// Selection (the selection part of Algorithm 1) in one workgroup.
constexpr int kSelThreads = 1024;
constexpr int kSurMaxUnits = 8192;

__device__ __forceinline__ uint32_t order_desc(float x) {
  // maps larger floats to smaller keys (total order on non-NaN values;
  // -0 is read as +0 so that equal scores tie)
  const uint32_t u = __float_as_uint(x + 0.f);
  const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;
}

// Block-wide primitives for the 1024-thread selection workgroup: a wave-level
// pass (shuffles), 16 per-wave partials in LDS, one more wave-level pass.
// Each costs two barriers, where a tree over 1024 LDS slots costs twenty.
constexpr int kSelWaves = kSelThreads / 64;

// inclusive block scan of one value per thread; *total receives the sum
__device__ __forceinline__ int block_scan_incl(int v, int* sh, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(v, off, 64);
    if (lane >= off) v += y;
  }
  if (lane == 63) sh[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int t = lane < kSelWaves ? sh[lane] : 0;
#pragma unroll
    for (int off = 1; off < kSelWaves; off <<= 1) {
      const int y = __shfl_up(t, off, 64);
      if (lane >= off) t += y;
    }
    if (lane < kSelWaves) sh[kSelWaves + lane] = t;   // inclusive wave totals
  }
  __syncthreads();
  const int res = v + (wave > 0 ? sh[kSelWaves + wave - 1] : 0);
  *total = sh[2 * kSelWaves - 1];
  __syncthreads();
  return res;
}

__device__ __forceinline__ float block_max(float v, float* sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  v = wave_max(v);
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  float m = sh[0];
#pragma unroll
  for (int w = 1; w < kSelWaves; ++w) m = fmaxf(m, sh[w]);
  __syncthreads();
  return m;
}

// the largest v, the lowest i among equal largest values
__device__ __forceinline__ int block_argmax_first(float v, int i, float* shv, int* shi) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(v, off, 64);
    const int oi = __shfl_xor(i, off, 64);
    if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
  }
  if (lane == 0) { shv[wave] = v; shi[wave] = i; }
  __syncthreads();
  float bv = shv[0];
  int bi = shi[0];
#pragma unroll
  for (int w = 1; w < kSelWaves; ++w)
    if (shv[w] > bv || (shv[w] == bv && shi[w] < bi)) { bv = shv[w]; bi = shi[w]; }
  __syncthreads();
  return bi;
}

__global__ __launch_bounds__(kSelThreads) void k_sur_select(
    const float* __restrict__ r, int S, const int32_t* __restrict__ ustart, int U,
    const float* __restrict__ uscore, int budget, int pos0, float* __restrict__ env,
    float* __restrict__ wsum, int32_t* __restrict__ T, int32_t* __restrict__ run_start,
    int32_t* __restrict__ run_len, int32_t* __restrict__ counts, int cap) {
  __shared__ unsigned long long key[kSurMaxUnits];   // (order_desc(score), unit)
  __shared__ int rank[kSurMaxUnits];
  __shared__ int scan[kSelThreads];
  __shared__ int s_incl[kSelThreads], s_st[kSelThreads];   // T layout when U <= kSelThreads
  __shared__ int s_k, s_w, s_ws, s_err, s_bad;
  __shared__ float s_best[kSelThreads];
  const int tid = threadIdx.x;
  if (tid == 0) { s_err = 0; s_bad = 0; }
  __syncthreads();
  // units must partition [0, S): first start 0, strictly increasing, below S
  for (int u = tid; u < U; u += kSelThreads) {
    const int a = ustart[u];
    const bool ok = (u == 0 ? a == 0 : a > ustart[u - 1]) && a < S;
    if (!ok) atomicOr(&s_err, 1);
  }
  __syncthreads();
  if (s_err) {
    if (tid == 0) { counts[0] = 0; counts[1] = 0; counts[2] = KVR_ERR_BAD_BLOCKS; }
    return;
  }
  // rank the units by (score descending, unit ascending); key[i] becomes the
  // i-th unit in that order.  Up to kSelThreads units: each unit counts the
  // keys below its own (keys are distinct); beyond: bitonic sort.
  if (U <= kSelThreads) {
    unsigned long long mine = 0;
    if (tid < U) {
      mine = (static_cast<unsigned long long>(order_desc(uscore[tid])) << 32) | static_cast<unsigned>(tid);
      key[tid] = mine;
    }
    __syncthreads();
    // tpu threads per unit (a power of two up to 64) share the counting
    int tpu = 1;
    while (tpu < 64 && 2 * tpu * U <= kSelThreads) tpu *= 2;
    const int cu = tid / tpu, cq = tid % tpu;
    const unsigned long long ck = cu < U ? key[cu] : 0ull;
    int below = 0;
    if (cu < U) {
#pragma unroll 8
      for (int v = cq; v < U; v += tpu) below += key[v] < ck ? 1 : 0;
    }
    for (int off = 1; off < tpu; off <<= 1) below += __shfl_xor(below, off, 64);
    __syncthreads();
    if (cu < U && cq == 0) {
      key[below] = ck;
      rank[cu] = below;
    }
    __syncthreads();
  } else {
    int P2 = 1;
    while (P2 < U) P2 <<= 1;
    for (int i = tid; i < P2; i += kSelThreads)
      key[i] = i < U ? (static_cast<unsigned long long>(order_desc(uscore[i])) << 32) | static_cast<unsigned>(i)
                     : ~0ull;
    __syncthreads();
    for (int k = 2; k <= P2; k <<= 1)
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < P2; i += kSelThreads) {
          const int l = i ^ j;
          if (l > i) {
            const unsigned long long x = key[i], y = key[l];
            const bool up = (i & k) == 0;
            if ((x > y) == up) { key[i] = y; key[l] = x; }
          }
        }
        __syncthreads();
      }
    for (int i = tid; i < U; i += kSelThreads) rank[static_cast<int>(key[i] & 0xffffffffu)] = i;
    __syncthreads();
  }
  // fill: the first ranked unit whose length exceeds the remaining allowance
  if (tid == 0) { s_k = U; s_w = 0; }
  __syncthreads();
  int carry = 0;
  for (int base = 0; base < U; base += kSelThreads) {
    const int i = base + tid;
    int len = 0;
    if (i < U) {
      const int u = static_cast<int>(key[i] & 0xffffffffu);
      len = ((u + 1 < U) ? ustart[u + 1] : S) - ustart[u];
    }
    int chunk;
    const int incl = block_scan_incl(len, scan, &chunk) + carry;
    if (i < U && incl > budget && incl - len <= budget) {   // exactly one such i
      s_k = i;
      s_w = budget - (incl - len);
    }
    carry += chunk;
  }
  __syncthreads();
  const int k = s_k, w = s_w;   // units of rank < k are whole; rank k gets a width-w window
  int wu = -1, wa = 0, wlen = 0;
  if (k < U && w > 0) {
    wu = static_cast<int>(key[k] & 0xffffffffu);
    wa = ustart[wu];
    wlen = ((wu + 1 < U) ? ustart[wu + 1] : S) - wa;
    __syncthreads();   // key[] is free from here on: it holds the envelope when it fits
    const bool in_lds = wlen <= kSurMaxUnits;
    float* e = in_lds ? reinterpret_cast<float*>(key) : env;
    float* sums = in_lds ? reinterpret_cast<float*>(key) + kSurMaxUnits : wsum;
    // envelope (Eq. 8): the exponentials in parallel, then the running
    // max(e_t, e^(-1/16) u_{t-1}) in order by one thread
    float m = -INFINITY;
    for (int t = tid; t < wlen; t += kSelThreads) m = fmaxf(m, r[wa + t]);
    const float rmax = block_max(m, s_best);
    for (int t = tid; t < wlen; t += kSelThreads) e[t] = expf(r[wa + t] - rmax);
    __syncthreads();
    if (tid == 0) {
      // batches of 16: the loads issued together, the recurrence in registers
      const float c = 0.939413062813475786f;   // e^(-1/16) rounded to float32
      float prev = 0.f;
      for (int base = 0; base < wlen; base += 16) {
        float x[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) x[j] = base + j < wlen ? e[base + j] : 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          prev = fmaxf(x[j], c * prev);
          x[j] = prev;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (base + j < wlen) e[base + j] = x[j];
      }
    }
    __syncthreads();
    // every window sum, left to right from its start
    for (int a = tid; a <= wlen - w; a += kSelThreads) {
      float acc = 0.f;
      for (int i = 0; i < w; ++i) acc += e[a + i];
      sums[a] = acc;
    }
    __syncthreads();
    // earliest maximiser: per-thread best over a strided subset, then a
    // reduction that keeps the lower start on equal sums
    float bs = -INFINITY;
    int bi = 0x7fffffff;
    for (int a = tid; a <= wlen - w; a += kSelThreads)
      if (sums[a] > bs) { bs = sums[a]; bi = a; }
    const int best = block_argmax_first(bs, bi, s_best, scan);
    if (tid == 0) s_ws = best;
    __syncthreads();
  }
  const int ws = (wu >= 0) ? s_ws : 0;
  // chosen ranges in position order -> T
  int total = 0;
  if (U <= kSelThreads) {
    // offsets of every unit's range, then each output slot finds its unit
    int len = 0, st = 0;
    if (tid < U) {
      const int a = ustart[tid];
      const int n = ((tid + 1 < U) ? ustart[tid + 1] : S) - a;
      if (rank[tid] < k) { len = n; st = a; }
      else if (tid == wu) { len = w; st = a + ws; }
    }
    const int incl = block_scan_incl(len, scan, &total);
    s_incl[tid] = incl;
    s_st[tid] = st - (incl - len);   // position of slot i in this unit: s_st + i
    __syncthreads();
    if (total > cap) {
      if (tid == 0) s_bad = 1;
    } else {
      for (int i = tid; i < total; i += kSelThreads) {
        int lo = 0, hi = U - 1;   // first unit with incl > i
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (s_incl[mid] > i) hi = mid; else lo = mid + 1;
        }
        T[i] = pos0 + s_st[lo] + i;
      }
    }
  } else {
    carry = 0;
    for (int base = 0; base < U; base += kSelThreads) {
      const int u = base + tid;
      int len = 0, st = 0;
      if (u < U) {
        const int a = ustart[u];
        const int n = ((u + 1 < U) ? ustart[u + 1] : S) - a;
        if (rank[u] < k) { len = n; st = a; }
        else if (u == wu) { len = w; st = a + ws; }
      }
      int chunk;
      const int incl = block_scan_incl(len, scan, &chunk) + carry;
      const int off = incl - len;
      if (off + len > cap) atomicOr(&s_bad, 1);
      else
        for (int j = 0; j < len; ++j) T[off + j] = pos0 + st + j;
      carry += chunk;
    }
    total = carry;
  }
  __syncthreads();
  if (s_bad || total != budget) {
    if (tid == 0) { counts[0] = total; counts[1] = 0; counts[2] = KVR_ERR_CAPACITY; }
    return;
  }
  __threadfence_block();
  __syncthreads();
  // runs: maximal stretches of consecutive positions.  First pass: each run
  // start records its position and its index in T (in run_len for now).
  carry = 0;
  for (int base = 0; base < total; base += kSelThreads) {
    const int i = base + tid;
    const int is_start = (i < total && (i == 0 || T[i] != T[i - 1] + 1)) ? 1 : 0;
    int chunk;
    const int incl = block_scan_incl(is_start, scan, &chunk) + carry;
    if (is_start) {
      run_start[incl - 1] = T[i];
      run_len[incl - 1] = i;
    }
    carry += chunk;
  }
  const int R = carry;
  __threadfence_block();
  __syncthreads();
  // second pass: length = next run's index - this one's (read, sync, write)
  for (int base = 0; base < R; base += kSelThreads) {
    const int j = base + tid;
    int len = 0;
    if (j < R) len = ((j + 1 < R) ? run_len[j + 1] : total) - run_len[j];
    __syncthreads();
    if (j < R) run_len[j] = len;
    __syncthreads();
  }
  if (tid == 0) { counts[0] = total; counts[1] = R; counts[2] = KVR_OK; }
}

}  // namespace

hipError_t launch_sur_scores(kvr_dtype dt, const void* E, int vocab, int hidden,
                             const int32_t* sid, int S, const int32_t* qid, int Q, float* r,
                             hipStream_t stream) {
  if (S == 0) return hipSuccess;
  if (dt == KVR_F32) {
    hipLaunchKernelGGL(k_sur_scores_f32, dim3(S), dim3(kScoreThreads), 0, stream,
                       static_cast<const float*>(E), vocab, hidden, sid, qid, Q, r);
    return hipGetLastError();
  }
  const bf16_t* e = static_cast<const bf16_t*>(E);
  if (hidden % kStatChunk == 0 && Q <= 128) {
    const dim3 grid((S + kStatTokens - 1) / kStatTokens), block(kStatThreads);
    switch ((Q + 15) / 16) {
      case 1: hipLaunchKernelGGL(k_sur_scores_stat<1>, grid, block, 0, stream, e, vocab, hidden, sid, S, qid, Q, r); break;
      case 2: hipLaunchKernelGGL(k_sur_scores_stat<2>, grid, block, 0, stream, e, vocab, hidden, sid, S, qid, Q, r); break;
      case 3: hipLaunchKernelGGL(k_sur_scores_stat<3>, grid, block, 0, stream, e, vocab, hidden, sid, S, qid, Q, r); break;
      case 4: hipLaunchKernelGGL(k_sur_scores_stat<4>, grid, block, 0, stream, e, vocab, hidden, sid, S, qid, Q, r); break;
      case 5: case 6: hipLaunchKernelGGL(k_sur_scores_stat<6>, grid, block, 0, stream, e, vocab, hidden, sid, S, qid, Q, r); break;
      default: hipLaunchKernelGGL(k_sur_scores_stat<8>, grid, block, 0, stream, e, vocab, hidden, sid, S, qid, Q, r); break;
    }
    return hipGetLastError();
  }
  const dim3 grid((S + 31) / 32);
  switch ((Q + 31) / 32) {
    case 1: hipLaunchKernelGGL(k_sur_scores_mfma<1>, grid, dim3(kScoreThreads), 0, stream, e, vocab, hidden, sid, S, qid, Q, r); break;
    case 2: hipLaunchKernelGGL(k_sur_scores_mfma<2>, grid, dim3(kScoreThreads), 0, stream, e, vocab, hidden, sid, S, qid, Q, r); break;
    case 3: case 4: hipLaunchKernelGGL(k_sur_scores_mfma<4>, grid, dim3(kScoreThreads), 0, stream, e, vocab, hidden, sid, S, qid, Q, r); break;
    default: hipLaunchKernelGGL(k_sur_scores_mfma<8>, grid, dim3(kScoreThreads), 0, stream, e, vocab, hidden, sid, S, qid, Q, r); break;
  }
  return hipGetLastError();
}

hipError_t launch_sur_select(const float* r, int S, const int32_t* ustart, int U,
                             float* uscore, int budget, int pos0, float* ws, int32_t* T,
                             int32_t* run_start, int32_t* run_len, int32_t* counts, int cap,
                             hipStream_t stream) {
  hipLaunchKernelGGL(k_sur_unit_scores, dim3((U + kUnitWaves - 1) / kUnitWaves),
                     dim3(64 * kUnitWaves), 0, stream, r, S, ustart, U, uscore);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_sur_select, dim3(1), dim3(kSelThreads), 0, stream, r, S, ustart, U,
                     uscore, budget, pos0, ws, ws + S, T, run_start, run_len, counts, cap);
  return hipGetLastError();
}

}  // namespace kvr
