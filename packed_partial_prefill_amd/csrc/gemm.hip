// Dense projections of the packed rows: QKV, O, gate/up (+SwiGLU) and down.
// C = A * W^T with A [M, K] (packed activations) and W [N, K] (PyTorch
// Linear layout); both operands are K-contiguous.
//
// bf16 storage runs on the MFMA kernel below; float32 storage runs on an
// LDS-tiled float32 FMA kernel (no reduced-precision matrix modes).
#include <cmath>

#include "common.h"
#include "kvr_internal.h"

namespace kvr {

namespace {

constexpr int kTile = 64, kKStep = 32, kThreads = 256;

template <typename T>
__device__ __forceinline__ const T* seg_row(const WeightSegs& W, int n, int K) {
  int j = 0;
  if (W.nseg > 1 && n >= W.n_begin[1]) j = 1;
  if (W.nseg > 2 && n >= W.n_begin[2]) j = 2;
  return static_cast<const T*>(W.w[j]) + static_cast<size_t>(n - W.n_begin[j]) * K;
}

// MODE 0: part[split][M][N] = partial product over this split's K range.
// MODE 1: out[M][N] = SiLU(A Wg^T) * (A Wu^T) (W.w[0] = Wg, W.w[1] = Wu, full K).
template <typename T, int MODE>
__global__ __launch_bounds__(kThreads) void k_gemm_fma(const T* __restrict__ A, WeightSegs W,
                                                       int M, int N, int K, int k_per_split,
                                                       float* __restrict__ part,
                                                       T* __restrict__ out) {
  __shared__ float As[kKStep][kTile + 1];
  __shared__ float Bs[kKStep][kTile + 1];
  __shared__ float Us[MODE == 1 ? kKStep : 1][kTile + 1];
  const int tid = threadIdx.x;
  const int bm = blockIdx.y * kTile, bn = blockIdx.x * kTile;
  const int k0 = blockIdx.z * k_per_split, k1 = min(K, k0 + k_per_split);
  const int tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  float acu[MODE == 1 ? 4 : 1][4] = {};

  for (int kb = k0; kb < k1; kb += kKStep) {
    for (int idx = tid; idx < kTile * kKStep; idx += kThreads) {
      const int row = idx / kKStep, kk = idx - row * kKStep;
      const int m = bm + row, n = bn + row, k = kb + kk;
      As[kk][row] = (m < M && k < k1) ? Elem<T>::load(A, static_cast<size_t>(m) * K + k) : 0.f;
      if (MODE == 0) {
        Bs[kk][row] = (n < N && k < k1) ? Elem<T>::load(seg_row<T>(W, n, K), k) : 0.f;
      } else {
        const size_t off = static_cast<size_t>(n) * K + k;
        const bool ok = n < N && k < k1;
        Bs[kk][row] = ok ? Elem<T>::load(static_cast<const T*>(W.w[0]), off) : 0.f;
        Us[MODE == 1 ? kk : 0][row] = ok ? Elem<T>::load(static_cast<const T*>(W.w[1]), off) : 0.f;
      }
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < kKStep; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
      if (MODE == 1) {
        float u[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) u[j] = Us[MODE == 1 ? kk : 0][tx * 4 + j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acu[MODE == 1 ? i : 0][j] = fmaf(a[i], u[j], acu[MODE == 1 ? i : 0][j]);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = bm + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = bn + tx * 4 + j;
      if (n >= N) continue;
      if (MODE == 0) {
        part[(static_cast<size_t>(blockIdx.z) * M + m) * N + n] = acc[i][j];
      } else {
        const float g = acc[i][j];
        const float sg = g / (1.f + expf(-g));
        Elem<T>::store(out, static_cast<size_t>(m) * N + n, sg * acu[MODE == 1 ? i : 0][j]);
      }
    }
  }
}


// ---------------------------------------------------------------------------
// bf16 MFMA kernel (gfx950 v_mfma_f32_32x32x16_bf16), float32 accumulation.
//
// A workgroup computes a BM (rows of A) x BN (rows of W) tile with WM x WN
// waves; each wave owns TM x TN blocks of 32 x 32.  K advances 32 at a time
// through NS LDS stages that are filled straight from global memory by
// global_load_lds_dwordx4 (no register staging), NS - 1 stages ahead of the
// MFMAs; the barrier that recycles a stage sits in the middle of each step,
// after the first half of its MFMAs is issued, so the matrix core stays busy
// while the waves synchronise.  A stage holds the tile's BM x 32 slice of A
// and BN x 32 slice of W as 64-byte rows of four 16-byte chunks; chunk c of
// row r sits at c ^ ((r >> 2) & 3).  Of the XOR patterns on the row bits,
// this one (like bits 3-4) measures no LDS bank conflicts for the MFMA
// operand reads on gfx950 (rocprofv3 SQ_LDS_BANK_CONFLICT); patterns on bits
// 0-1 or 1-3 measure 2- to 4-way conflicts.  The stage buffers are separate LDS
// objects picked at compile time, which lets the compiler keep the newer
// stages in flight while one is consumed.  MFMA operand layout (32x32x16):
// lane l supplies row/column l%32 and k = 8*(l/32) .. +7 of the 16-wide K
// slice; accumulator t of lane l is D[8*(t/4) + 4*(l/32) + t%4][l%32].
//
// The fused gate/up tile for large M (TileLP) fetches W in 128-byte row
// pieces instead: each DMA piece covers 8 rows x 128 bytes, the two K steps
// of a "pair", into a ring of 3 pair slots (the A stages keep 64-byte
// pieces).  With every CU streaming from L2, 128-byte pieces move about 1.5x
// the bytes per clock of 64-byte ones (a 64-byte piece costs the L2 -> L1
// path a whole line); the pair ring also gives W a step more of lead.
// Measured 4% faster for gate/up at the 7B layer (8% at the 1.5B layer's
// 128 x 128 tile, 6% at M = 64); slower for the split-K projections, which
// keep 64-byte pieces.
//
// Tile shapes: 256 x 256 (8 waves) for large M; 128 x 128 (4 waves, two
// workgroups per CU) and 64 x 128 (2 waves, three per CU, deeper pipeline)
// when M is small and the weights, not the matrix core, set the pace: there
// a launch needs many workgroups, each with several stages of weights in
// flight, to keep HBM busy.
//
// Workgroups are numbered along M fastest, then N panel, then K split, and
// block b is mapped so that each XCD (b % 8) takes one contiguous run of that
// order: the M tiles sharing a weight panel then run together on one XCD and
// the panel is fetched from HBM into that XCD's L2 once.
// ---------------------------------------------------------------------------
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int KB = 32;

template <int BM_, int BN_, int WM_, int WN_, int NS_, int OCC_, bool WP_ = false>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, NS = NS_;
  static constexpr int occupancy = OCC_;               // workgroups per CU it is sized for
  // WP: W arrives in 128-byte row pieces that cover a pair of K steps, in a
  // ring of NWP pair slots after the NS A stages (A keeps 64-byte pieces)
  static constexpr bool WP = WP_;
  static constexpr int NWP = 3;
  static constexpr int TM = BM / (32 * WM), TN = BN / (32 * WN);
  static constexpr int waves = WM * WN, threads = 64 * waves;
  static constexpr int waves_per_simd = (OCC_ * waves + 3) / 4;
  static constexpr int LA = BM / 16 / waves;           // 1 KB DMA slices per wave per stage (A)
  static constexpr int LW = BN / 16 / waves;           // ... (W)
  static constexpr int LS = LA + LW;
  static constexpr int LWP = BN / 8 / waves;          // 1 KB DMA pieces per wave per W pair
  static constexpr int ABytes = BM * KB * 2, WBytes = BN * KB * 2, WPBytes = 2 * WBytes;
  static_assert(TM * 32 * WM == BM && TN * 32 * WN == BN, "wave blocks tile the workgroup");
  static_assert(LA * 16 * waves == BM && LW * 16 * waves == BN, "whole DMA slices per wave");
  static_assert(TN % 2 == 0, "gate and up blocks pair up in the fused SwiGLU epilogue");
  static_assert(NS >= 3 && NS <= 6 && (NS - 2) * LS < 64, "pipeline depth and vmcnt range");
  static_assert(!WP || (NS == 4 && LWP * 8 * waves == BN && 2 * LA + LWP < 64),
                "the pair schedule (prologue and vmcnt counts) is laid out for 4 A stages; "
                "whole pieces; vmcnt range");
  // one dynamic LDS buffer: the NS A stages, then the NS W stages, so that a
  // fragment address is a lane register plus a compile-time offset
  static constexpr int aOff(int s) { return s * ABytes; }
  static constexpr int wOff(int s) { return NS * ABytes + s * WBytes; }
  static constexpr int wpOff(int p) { return NS * ABytes + p * WPBytes; }
  static constexpr int smem = WP ? NS * ABytes + NWP * WPBytes : NS * (ABytes + WBytes);
  static_assert(smem * OCC_ <= 160 * 1024, "LDS per CU");
  static_assert((NS - 1) * ABytes < 65536 && (NS - 1) * WBytes < 65536, "ds offset field");
};

// The tile shapes the library launches.
using TileL = Tile<256, 256, 4, 2, 4, 1>;
using TileLP = Tile<256, 256, 4, 2, 4, 1, true>;    // W pairs: fused gate/up, K a multiple of 64
using TileM = Tile<128, 128, 2, 2, 4, 2>;
using TileMP = Tile<128, 128, 2, 2, 4, 2, true>;    // W pairs: fused gate/up
using TileS = Tile<64, 128, 1, 2, 6, 2>;
using TileSP = Tile<64, 128, 1, 2, 4, 2, true>;     // W pairs: fused gate/up
// Fused gate/up for 128 < M <= 256: every row of A in one tile, so each
// weight panel is staged in LDS once (two 128-row tiles each stage it, and
// a CU holding two of them takes in twice the bytes).
using TileT = Tile<256, 128, 4, 2, 4, 1>;
using TileTP = Tile<256, 128, 4, 2, 4, 1, true>;

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * (KB * 2) + ((chunk ^ ((row >> 2) & 3)) << 4);
}
// 128-byte rows (W pairs): chunk c of row r at c ^ ((r >> 1) & 7), so that
// the 16 lanes of one ds_read_b128 quarter, one chunk of 16 consecutive
// rows, fall in 16 distinct 16-byte groups of the 256-byte bank row
__device__ __forceinline__ int swz2(int row, int chunk) {
  return row * (KB * 4) + ((chunk ^ ((row >> 1) & 7)) << 4);
}

#define KVR_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define KVR_GLB(p) ((const __attribute__((address_space(1))) void*)(p))

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] and
// vmcnt[5:4] at bits 15:14, expcnt[6:4] = 7, lgkmcnt[11:8] = 15).
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0xF70);
}

template <class C>
struct GemmThread {
  static constexpr int NW = C::WP ? C::LWP : C::LW;
  const bf16_t* asrc[C::LA];   // this lane's global source (A), at the split's first k
  const bf16_t* wsrc[NW];      // ... (W)
  int adst[C::LA], wdst[NW];   // wave-uniform LDS byte offset of each 1 KB slice
  // fragment LDS addresses in stage (pair slot) 0, per K half (for W pairs
  // those of the pair's first step: the second step's chunk differs in bit
  // 2, which is address bit 6 in a 128-byte row, the pair slots starting
  // on 128-byte boundaries of an LDS buffer at address 0 -- the kernel has
  // no static LDS)
  uint32_t la[C::TM][2], lw[C::TN][2];
  uint8_t* smem;
};

// stage S of step kb / KB: A and (without W pairs) W
template <class C, int S>
__device__ __forceinline__ void issue_stage(const GemmThread<C>& g, int kb) {
#pragma unroll
  for (int j = 0; j < C::LA; ++j)
    __builtin_amdgcn_global_load_lds(KVR_GLB(g.asrc[j] + kb), KVR_LDS(g.smem + C::aOff(S) + g.adst[j]),
                                     16, 0, 0);
  if constexpr (!C::WP) {
#pragma unroll
    for (int j = 0; j < C::LW; ++j)
      __builtin_amdgcn_global_load_lds(KVR_GLB(g.wsrc[j] + kb), KVR_LDS(g.smem + C::wOff(S) + g.wdst[j]),
                                       16, 0, 0);
  }
}

// W pair `pair` (steps 2 pair, 2 pair + 1; clamped to the last pair: a
// refill past the end is never read) into pair slot pair % NWP
template <class C>
__device__ __forceinline__ void issue_wpair(const GemmThread<C>& g, int pair, int nsteps) {
  const int p = min(pair, nsteps / 2 - 1);
  uint8_t* d = g.smem + C::wpOff(0) + (pair % C::NWP) * C::WPBytes;
#pragma unroll
  for (int j = 0; j < C::LWP; ++j)
    __builtin_amdgcn_global_load_lds(KVR_GLB(g.wsrc[j] + p * 2 * KB), KVR_LDS(d + g.wdst[j]), 16, 0, 0);
}

// LDS byte offset of step i's W pair slot
template <class C>
__device__ __forceinline__ uint32_t wpair_off(int i) {
  return C::WP ? static_cast<uint32_t>(((i >> 1) % C::NWP) * C::WPBytes) : 0u;
}

// Operand fragments of one 16-wide K half of a stage.
template <class C>
struct Frags {
  bf16x8_t a[C::TM], w[C::TN];
};

// Reads of the main loop are inline assembly (the compiler's lgkmcnt
// tracking across the stage pipeline waits for every outstanding LDS read
// before the first product); a step waits for the older half with
// lds_wait_n<TM + TN> while the newer half's reads stay in flight.
template <class C, int S, int KS>
__device__ __forceinline__ void load_frags(const GemmThread<C>& g, Frags<C>& f, uint32_t woff) {
#pragma unroll
  for (int mb = 0; mb < C::TM; ++mb)
    f.a[mb] = __builtin_bit_cast(bf16x8_t, ds_read_b128<S * C::ABytes>(g.la[mb][KS]));
#pragma unroll
  for (int nb = 0; nb < C::TN; ++nb) {
    if constexpr (C::WP)
      f.w[nb] = __builtin_bit_cast(bf16x8_t, ds_read_b128((g.lw[nb][KS] ^ ((S % 2) * 64u)) + woff));
    else
      f.w[nb] = __builtin_bit_cast(bf16x8_t, ds_read_b128<S * C::WBytes>(g.lw[nb][KS]));
  }
}

// the fragments read before the last TM + TN reads have landed
template <class C>
__device__ __forceinline__ void frags_ready(Frags<C>& f) {
  lds_wait_n<C::TM + C::TN>();
#pragma unroll
  for (int mb = 0; mb < C::TM; ++mb) reg_fence(f.a[mb]);
#pragma unroll
  for (int nb = 0; nb < C::TN; ++nb) reg_fence(f.w[nb]);
}

template <class C>
__device__ __forceinline__ void mma(const Frags<C>& f, f32x16_t (&acc)[C::TM][C::TN]) {
#pragma unroll
  for (int mb = 0; mb < C::TM; ++mb)
#pragma unroll
    for (int nb = 0; nb < C::TN; ++nb)
      acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[mb], f.w[nb], acc[mb][nb], 0, 0, 0);
}

// Barrier between the stage waits and the stage reads/refills; the empty asm
// statements keep the compiler from moving LDS reads or DMA across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One K step on stage S, software-pipelined over the two 16-wide halves:
// f0 arrives holding half 0 of stage S (read during the previous step).
// Half 1's reads are issued, then half 0 multiplies while they land; then
// wait until the next stage's DMA has landed (NS - 3 newer stages may stay
// in flight) and barrier (every wave is past the previous stage), refill the
// previous stage's buffers with the step NS - 1 ahead (clamped to the last
// step: a refill past the end is never read), read half 0 of the next stage
// into f0, and multiply half 1 while those land.
// With W pairs, step i also refills, when i is even, the pair slot of the
// pair just finished with the pair two ahead (steps i + 4, i + 5).  The
// issue order is then A(i + 3) [, W pair (i / 2 + 2)] per step, and at
// every step's wait exactly LA + LWP instructions were issued after the
// last one it needs (A(i + 1); the W pair of step i + 1 came earlier).
template <class C, int S>
__device__ __forceinline__ void k_step(const GemmThread<C>& g, int i,
                                       int nsteps, f32x16_t (&acc)[C::TM][C::TN], Frags<C>& f0,
                                       Frags<C>& f1) {
  load_frags<C, S, 1>(g, f1, wpair_off<C>(i));
  frags_ready<C>(f0);
  mma<C>(f0, acc);
  if constexpr (C::WP) wait_vmcnt<C::LA + C::LWP>();
  else wait_vmcnt<(C::NS - 3) * C::LS>();
  stage_barrier();
  issue_stage<C, (S + C::NS - 1) % C::NS>(g, min(i + C::NS - 1, nsteps - 1) * KB);
  if constexpr (C::WP && S % 2 == 0) issue_wpair<C>(g, i / 2 + 2, nsteps);
  load_frags<C, (S + 1) % C::NS, 0>(g, f0, wpair_off<C>(i + 1));   // unused after the last step (in bounds)
  frags_ready<C>(f1);
  mma<C>(f1, acc);
}

// NS consecutive steps starting on stage S = 0.
template <class C, int S>
__device__ __forceinline__ void k_round(const GemmThread<C>& g, int i,
                                        int nsteps, f32x16_t (&acc)[C::TM][C::TN], Frags<C>& f0,
                                        Frags<C>& f1) {
  k_step<C, S>(g, i + S, nsteps, acc, f0, f1);
  if constexpr (S + 1 < C::NS) k_round<C, S + 1>(g, i, nsteps, acc, f0, f1);
}

// The last nsteps - i (< NS) steps.
template <class C, int S>
__device__ __forceinline__ void k_tail(const GemmThread<C>& g, int i,
                                       int nsteps, f32x16_t (&acc)[C::TM][C::TN], Frags<C>& f0,
                                       Frags<C>& f1) {
  if (i + S < nsteps) {
    k_step<C, S>(g, i + S, nsteps, acc, f0, f1);
    if constexpr (S + 2 < C::NS) k_tail<C, S + 1>(g, i, nsteps, acc, f0, f1);
  }
}

template <class C, int S>
__device__ __forceinline__ void k_prologue(const GemmThread<C>& g, int nsteps) {
  issue_stage<C, S>(g, min(S, nsteps - 1) * KB);
  if constexpr (S + 2 < C::NS) k_prologue<C, S + 1>(g, nsteps);
}

// MODE 0: part[split][M][N] = A * W^T over this split's K range (W segmented).
// MODE 1: W.w[0] = W_gate, W.w[1] = W_up; the tile holds BN/2 gate rows and the
//         same BN/2 up rows; out[M][N] = bf16(SiLU(gate) * up), full K.  A wave's
//         first TN/2 column blocks are gate columns, the last TN/2 the matching
//         up columns, so both factors of an output meet in one lane.
template <int MODE, class C>
__global__ __launch_bounds__(C::threads, C::waves_per_simd) void k_gemm_mfma(
    const bf16_t* __restrict__ A, WeightSegs W, int M, int N, int K, int k_per_split,
    int tiles_m, int tiles_n, int splits, float* __restrict__ part, bf16_t* __restrict__ out) {
  constexpr int TM = C::TM, TN = C::TN, BM = C::BM, BN = C::BN;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  // XCD-aware order: t = ((split * tiles_n) + n) * tiles_m + m
  const int total = tiles_m * tiles_n * splits;
  const int t = xcd_linear(blockIdx.x, total);
  const int tm = t % tiles_m, tn = (t / tiles_m) % tiles_n, split = t / (tiles_m * tiles_n);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int m0 = tm * BM;
  const int n0 = tn * (MODE == 1 ? BN / 2 : BN);
  const int k0 = split * k_per_split;
  const int k1 = min(K, k0 + k_per_split);
  const int nsteps = k1 > k0 ? (k1 - k0) / KB : 0;

  GemmThread<C> g;
#pragma unroll
  for (int j = 0; j < C::LA; ++j) {
    const int row0 = (wave * C::LA + j) * 16;
    const int row = row0 + (lane >> 2);                      // tile row this lane fetches
    const int chunk = (lane & 3) ^ ((row >> 2) & 3);   // logical chunk of its slot
    g.adst[j] = row0 * (KB * 2);
    const int m = min(m0 + row, M - 1);
    g.asrc[j] = A + static_cast<size_t>(m) * K + k0 + chunk * 8;
  }
#pragma unroll
  for (int j = 0; j < GemmThread<C>::NW; ++j) {
    // 64-byte pieces: 16 rows of 4 chunks; W pairs: 8 rows of 8 chunks
    const int rows = C::WP ? 8 : 16, lpr = 64 / rows;
    const int row0 = (wave * GemmThread<C>::NW + j) * rows;
    const int row = row0 + lane / lpr;
    const int chunk = C::WP ? (lane & 7) ^ ((row >> 1) & 7) : (lane & 3) ^ ((row >> 2) & 3);
    g.wdst[j] = row0 * lpr * 16;
    const bf16_t* wr;
    if (MODE == 0) {
      const int n = min(n0 + row, N - 1);
      int sj = 0;
      if (W.nseg > 1 && n >= W.n_begin[1]) sj = 1;
      if (W.nseg > 2 && n >= W.n_begin[2]) sj = 2;
      wr = static_cast<const bf16_t*>(W.w[sj]) + static_cast<size_t>(n - W.n_begin[sj]) * K;
    } else {
      const int n = min(n0 + row % (BN / 2), N - 1);
      wr = static_cast<const bf16_t*>(W.w[row / (BN / 2)]) + static_cast<size_t>(n) * K;
    }
    g.wsrc[j] = wr + k0 + chunk * 8;
  }
  g.smem = smem;
  const int khalf = lane >> 5;
#pragma unroll
  for (int mb = 0; mb < TM; ++mb) {
    const int arow = (wm * TM + mb) * 32 + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) g.la[mb][ks] = lds_addr(smem) + C::aOff(0) + swz(arow, ks * 2 + khalf);
  }
#pragma unroll
  for (int nb = 0; nb < TN; ++nb) {
    const int wrow = MODE == 0 ? (wn * TN + nb) * 32 + (lane & 31)
                               : (nb < TN / 2 ? 0 : BN / 2) + (wn * (TN / 2) + nb % (TN / 2)) * 32 + (lane & 31);
    if constexpr (C::WP) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) g.lw[nb][ks] = lds_addr(smem) + C::wpOff(0) + swz2(wrow, ks * 2 + khalf);
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) g.lw[nb][ks] = lds_addr(smem) + C::wOff(0) + swz(wrow, ks * 2 + khalf);
    }
  }

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int mb = 0; mb < TM; ++mb)
#pragma unroll
    for (int nb = 0; nb < TN; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mb][nb][e] = 0.f;

  if (nsteps > 0) {
    if constexpr (C::WP) {
      // A0, W pair 0, A1, A2, W pair 1: step 0 needs the first two
      issue_stage<C, 0>(g, 0);
      issue_wpair<C>(g, 0, nsteps);
      issue_stage<C, 1>(g, min(1, nsteps - 1) * KB);
      issue_stage<C, 2>(g, min(2, nsteps - 1) * KB);
      issue_wpair<C>(g, 1, nsteps);
      wait_vmcnt<2 * C::LA + C::LWP>();
    } else {
      k_prologue<C, 0>(g, nsteps);              // stages 0 .. NS-2
      wait_vmcnt<(C::NS - 2) * C::LS>();        // stage 0 landed; the rest may be in flight
    }
    stage_barrier();
    Frags<C> f0, f1;
    load_frags<C, 0, 0>(g, f0, 0);
    int i = 0;
    for (; i + C::NS <= nsteps; i += C::NS) k_round<C, 0>(g, i, nsteps, acc, f0, f1);
    k_tail<C, 0>(g, i, nsteps, acc, f0, f1);
    wait_vmcnt<0>();
    lds_wait();   // the unused reads after the last step
  }

  // epilogue
  if constexpr (MODE == 0) {
    // float32 partials, staged through LDS one band of TM * 32 rows (one
    // wave row) at a time so that they leave in 16-byte row chunks
    constexpr int RB = TM * 32;                // rows per band
    constexpr int RS = BN * 4 + 16;            // LDS row stride in bytes (padded)
    constexpr int CH = BN / 4;                 // 16-byte chunks per row
    static_assert(RB * RS <= C::smem, "band fits the stage buffers");
    float* pbase = part + static_cast<size_t>(split) * M * N;
#pragma unroll 1
    for (int band = 0; band < C::WM; ++band) {
      stage_barrier();   // the previous band (or the last stage) has been read
      if (wm == band) {
#pragma unroll
        for (int mb = 0; mb < TM; ++mb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int rl = mb * 32 + 8 * (e >> 2) + 4 * khalf + (e & 3);
#pragma unroll
            for (int nb = 0; nb < TN; ++nb) {
              const int cl = (wn * TN + nb) * 32 + (lane & 31);
              *reinterpret_cast<float*>(smem + rl * RS + cl * 4) = acc[mb][nb][e];
            }
          }
      }
      __syncthreads();
      for (int i = tid; i < RB * CH; i += C::threads) {
        const int rl = i / CH, ch = i - rl * CH;
        const int m = m0 + band * RB + rl, n = n0 + ch * 4;
        if (m >= M || n >= N) continue;
        const uint8_t* src = smem + rl * RS + ch * 16;
        float* dst = pbase + static_cast<size_t>(m) * N + n;
        if (n + 4 <= N && (N & 3) == 0) {
          *reinterpret_cast<float4*>(dst) = *reinterpret_cast<const float4*>(src);
        } else {
          for (int k = 0; k < 4 && n + k < N; ++k) dst[k] = reinterpret_cast<const float*>(src)[k];
        }
      }
    }
  } else {
    // SiLU(gate) * up in bf16, staged through LDS (free once every wave is
    // past its last stage read) so that the tile leaves in 16-byte row
    // chunks rather than 2-byte stores.  SiLU uses the hardware exp2 and
    // reciprocal (each within an ulp or two of float32; the result is
    // rounded to bf16).
    constexpr int OC = BN / 2;                 // output columns of the tile
    constexpr int RS = OC * 2 + 16;            // LDS row stride in bytes (padded)
    static_assert(BM * RS <= C::smem, "output tile fits the stage buffers");
    stage_barrier();
#pragma unroll
    for (int mb = 0; mb < TM; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rl = (wm * TM + mb) * 32 + 8 * (e >> 2) + 4 * khalf + (e & 3);
#pragma unroll
        for (int nb = 0; nb < TN / 2; ++nb) {
          const int cl = (wn * (TN / 2) + nb) * 32 + (lane & 31);
          const float gt = acc[mb][nb][e], up = acc[mb][nb + TN / 2][e];
          const float sg = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-gt * 1.4426950408889634f));
          *reinterpret_cast<bf16_t*>(smem + rl * RS + cl * 2) = f32_to_bf16(gt * sg * up);
        }
      }
    __syncthreads();
    constexpr int CH = OC / 8;                 // 16-byte chunks per output row
    for (int i = tid; i < BM * CH; i += C::threads) {
      const int rl = i / CH, ch = i - rl * CH;
      const int m = m0 + rl, n = n0 + ch * 8;
      if (m >= M || n >= N) continue;
      const uint8_t* src = smem + rl * RS + ch * 16;
      bf16_t* dst = out + static_cast<size_t>(m) * N + n;
      if (n + 8 <= N && (N & 7) == 0) {
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
      } else {
        for (int k = 0; k < 8 && n + k < N; ++k) dst[k] = reinterpret_cast<const bf16_t*>(src)[k];
      }
    }
  }
}

// out[m][n] = SiLU(sum_s part[s][m][n]) * sum_s part[s][m][N + n] (part rows
// hold the gate columns, then the up columns), stored in bf16.
constexpr int kRedThreads = 256;
__global__ __launch_bounds__(kRedThreads) void k_swiglu_reduce(const float* __restrict__ part,
                                                               int splits, int M, int N,
                                                               bf16_t* __restrict__ out) {
  const size_t n4 = static_cast<size_t>(N) >> 2;
  const size_t idx = static_cast<size_t>(blockIdx.x) * kRedThreads + threadIdx.x;
  if (idx >= static_cast<size_t>(M) * n4) return;
  const size_t m = idx / n4, j = idx - m * n4;
  const size_t stride4 = static_cast<size_t>(M) * 2 * n4;
  const float4* g4 = reinterpret_cast<const float4*>(part) + m * 2 * n4 + j;
  float4 g = g4[0], u = g4[n4];
  // unrolled so that several partials' loads are in flight together
#pragma unroll 8
  for (int s = 1; s < splits; ++s) {
    const float4 a = g4[s * stride4], c = g4[s * stride4 + n4];
    g.x += a.x; g.y += a.y; g.z += a.z; g.w += a.w;
    u.x += c.x; u.y += c.y; u.z += c.z; u.w += c.w;
  }
  uint2 p;
  p.x = static_cast<uint32_t>(f32_to_bf16(g.x / (1.f + expf(-g.x)) * u.x)) |
        (static_cast<uint32_t>(f32_to_bf16(g.y / (1.f + expf(-g.y)) * u.y)) << 16);
  p.y = static_cast<uint32_t>(f32_to_bf16(g.z / (1.f + expf(-g.z)) * u.z)) |
        (static_cast<uint32_t>(f32_to_bf16(g.w / (1.f + expf(-g.w)) * u.w)) << 16);
  reinterpret_cast<uint2*>(out)[idx] = p;
}

template <int MODE, class C>
void launch_mfma(const bf16_t* A, const WeightSegs& W, int M, int N, int K, int splits,
                 float* part, bf16_t* out, hipStream_t stream) {
  constexpr int G = C::WP ? 2 * KB : KB;   // K granule of a split (whole W pairs)
  const int kps = ((K / splits + G - 1) / G) * G;
  const int tm = (M + C::BM - 1) / C::BM;
  const int tn = MODE == 1 ? (N + C::BN / 2 - 1) / (C::BN / 2) : (N + C::BN - 1) / C::BN;
  static bool attr = false;
  if (!attr) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_mfma<MODE, C>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, C::smem) != hipSuccess)
      return;   // the launch below then reports the error
    attr = true;
  }
  hipLaunchKernelGGL((k_gemm_mfma<MODE, C>), dim3(tm * tn * splits), dim3(C::threads), C::smem,
                     stream, A, W, M, N, K, kps, tm, tn, splits, part, out);
}

// The fused gate/up takes the W-pair form CP of a tile when K allows it
// (measured 4-8% faster); the split-K projections keep C (slower with pairs).
template <int MODE, class CP, class C>
void launch_tile(const bf16_t* A, const WeightSegs& W, int M, int N, int K, int splits, float* part,
                 bf16_t* out, hipStream_t stream) {
  if constexpr (MODE == 1) {
    if (K % (2 * KB) == 0) {
      launch_mfma<MODE, CP>(A, W, M, N, K, splits, part, out, stream);
      return;
    }
  }
  launch_mfma<MODE, C>(A, W, M, N, K, splits, part, out, stream);
}

template <int MODE>
void launch_variant(int variant, const bf16_t* A, const WeightSegs& W, int M, int N, int K,
                    int splits, float* part, bf16_t* out, hipStream_t stream) {
  switch (variant) {
    case 0: launch_tile<MODE, TileLP, TileL>(A, W, M, N, K, splits, part, out, stream); break;
    case 1: launch_tile<MODE, TileMP, TileM>(A, W, M, N, K, splits, part, out, stream); break;
    case 3:
      if constexpr (MODE == 1) {
        launch_tile<MODE, TileTP, TileT>(A, W, M, N, K, splits, part, out, stream);
        break;
      }
      [[fallthrough]];
    default: launch_tile<MODE, TileSP, TileS>(A, W, M, N, K, splits, part, out, stream); break;
  }
}

struct VariantGeom { int bm, bn, occupancy; };
constexpr VariantGeom kGeom[4] = {{TileL::BM, TileL::BN, TileL::occupancy},
                                  {TileM::BM, TileM::BN, TileM::occupancy},
                                  {TileS::BM, TileS::BN, TileS::occupancy},
                                  {TileT::BM, TileT::BN, TileT::occupancy}};

}  // namespace

// Launch plan for C[M, N] = A[M, K] W[N, K]^T.
//
// Large M (> 512): 256 x 256 tiles; the K split is the smallest that
// minimises the critical path, rounds of 256 resident workgroups times K
// steps per workgroup (the launch is MFMA-bound).
// Small M: the launch streams weights (HBM-bound) and what matters is having
// enough workgroups in flight: 128 x 128 tiles up to M = 512, 64 x 128 up to
// M = 128, and the K split that divides the K steps evenly and brings the
// launch closest to one workgroup per CU (measured on the Qwen2.5-1.5B and
// Qwen3-8B projection shapes: fewer leave CUs idle, more add float32 partial
// traffic and a second round).
// swiglu: the gate/up pair (W = [Wg; Wu], 2N columns).  The SwiGLU is fused
// into the epilogue when the unsplit launch has enough workgroups; otherwise
// gate and up are computed as split-K partials and reduced by a row kernel.
// float32 storage uses the FMA kernel and never splits.
GemmPlan gemm_plan_for(kvr_dtype dt, int M, int N, int K, bool swiglu) {
  if (dt != KVR_BF16) return GemmPlan{0, 1, swiglu};
  const int cols = swiglu ? 2 * N : N;
  const int ksteps = K / KB;
  if (M > 512) {
    if (swiglu) return GemmPlan{0, 1, true};
    const long tiles = static_cast<long>((M + TileL::BM - 1) / TileL::BM) * ((cols + TileL::BN - 1) / TileL::BN);
    int best = 1;
    long best_cost = -1;
    for (int s = 1; s <= 8; ++s) {
      const long kps = (ksteps + s - 1) / s;
      if (kps < 2 && s > 1) break;
      const long cost = ((tiles * s + 255) / 256) * kps;
      if (best_cost < 0 || cost < best_cost) { best_cost = cost; best = s; }
    }
    return GemmPlan{0, best, false};
  }
  const int variant = M <= 128 ? 2 : 1;
  const VariantGeom vg = kGeom[variant];
  const long tiles_m = (M + vg.bm - 1) / vg.bm;
  constexpr long kTarget = 256;
  // fused gate/up with all rows in one 256 x 128 tile (one workgroup per CU)
  if (swiglu && M > 128 && M <= 256 && (N + kGeom[3].bn / 2 - 1) / (kGeom[3].bn / 2) >= kTarget / 2)
    return GemmPlan{3, 1, true};
  if (swiglu && tiles_m * ((N + vg.bn / 2 - 1) / (vg.bn / 2)) >= kTarget / 2)
    return GemmPlan{variant, 1, true};
  const long tiles = tiles_m * ((cols + vg.bn - 1) / vg.bn);
  int best = 1;
  double best_dist = 1e30;
  for (int s = 1; s <= 16; ++s) {
    if (ksteps / s < 4) break;
    if (ksteps % s != 0) continue;
    const double dist = std::fabs(std::log(static_cast<double>(tiles * s) / kTarget));
    if (dist < best_dist - 1e-9) { best_dist = dist; best = s; }
  }
  return GemmPlan{variant, best, false};
}

hipError_t launch_gemm_partial(kvr_dtype dt, const void* A, const WeightSegs& W, int M, int N,
                               int K, const GemmPlan& plan, float* part, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (dt == KVR_BF16) {
    launch_variant<0>(plan.variant, static_cast<const bf16_t*>(A), W, M, N, K, plan.splits, part,
                      nullptr, stream);
  } else {
    const int kps = ((K / plan.splits + 63) / 64) * 64;
    dim3 grid((N + kTile - 1) / kTile, (M + kTile - 1) / kTile, plan.splits);
    hipLaunchKernelGGL((k_gemm_fma<float, 0>), grid, dim3(kThreads), 0, stream,
                       static_cast<const float*>(A), W, M, N, K, kps, part, nullptr);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_swiglu(kvr_dtype dt, const void* A, const void* Wg, const void* Wu, int M,
                              int N, int K, const GemmPlan& plan, float* part, void* out,
                              hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (dt == KVR_BF16) {
    const bf16_t* a = static_cast<const bf16_t*>(A);
    if (plan.fused) {
      WeightSegs W{{Wg, Wu, nullptr}, {0, N, N, N}, 2};
      launch_variant<1>(plan.variant, a, W, M, N, K, 1, nullptr, static_cast<bf16_t*>(out), stream);
    } else {
      WeightSegs W{{Wg, Wu, nullptr}, {0, N, 2 * N, 2 * N}, 2};
      launch_variant<0>(plan.variant, a, W, M, 2 * N, K, plan.splits, part, nullptr, stream);
      const size_t n = static_cast<size_t>(M) * (N / 4);
      hipLaunchKernelGGL(k_swiglu_reduce, dim3(static_cast<unsigned>((n + kRedThreads - 1) / kRedThreads)),
                         dim3(kRedThreads), 0, stream, part, plan.splits, M, N,
                         static_cast<bf16_t*>(out));
    }
  } else {
    WeightSegs W{{Wg, Wu, nullptr}, {0, N, N, N}, 2};
    dim3 grid((N + kTile - 1) / kTile, (M + kTile - 1) / kTile, 1);
    hipLaunchKernelGGL((k_gemm_fma<float, 1>), grid, dim3(kThreads), 0, stream,
                       static_cast<const float*>(A), W, M, N, K, K, nullptr,
                       static_cast<float*>(out));
  }
  return hipGetLastError();
}

}  // namespace kvr
