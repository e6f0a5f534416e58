// Dense projections of the packed rows: QKV, O, gate/up (+SwiGLU) and down.
// C = A * W^T with A [M, K] (packed activations) and W [N, K] (PyTorch
// Linear layout); both operands are K-contiguous.
//
// bf16 storage runs on the MFMA kernel below; float32 storage runs on an
// LDS-tiled float32 FMA kernel (no reduced-precision matrix modes).
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
// Workgroup tile 256 (M) x 256 (N), 8 waves; wave w owns rows (w/2)*64 .. +64
// and a 128-column slice (2 x 4 blocks of 32x32).  K advances 32 at a time
// through four LDS stages that are filled straight from global memory by
// global_load_lds_dwordx4 (no register staging), three stages ahead of the
// MFMAs; the barrier that recycles a stage sits in the middle of each step,
// after the first half of its MFMAs is issued, so the matrix core stays busy
// while the waves synchronise.  Each stage holds a 256 x 32 tile of A and of W as 64-byte rows of
// four 16-byte chunks; chunk c of row r sits at c ^ (((r >> 1) ^ (r >> 3)) & 3),
// so any 8 consecutive rows read by an MFMA operand load fall in distinct
// 16-byte slots of 128 bytes and any 16 in distinct slots of 256 bytes (no
// bank conflicts whether the LDS serves 8 or 16 lanes per pass).
// The stage buffers are separate LDS objects picked at compile time, which
// lets the compiler keep the three newer stages in flight while a stage is
// consumed.  MFMA operand layout (32x32x16): lane l supplies row/column l%32
// and k = 8*(l/32) .. +7 of the 16-wide K slice; accumulator t of lane l is
// D[8*(t/4) + 4*(l/32) + t%4][l%32].
//
// Workgroups are numbered along M fastest, then N panel, then K split, and
// block b is mapped so that each XCD (b % 8) takes one contiguous run of that
// order: the M tiles sharing a weight panel then run together on one XCD and
// the panel is fetched from HBM into that XCD's L2 once.
// ---------------------------------------------------------------------------
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int MB = 256, NB = 256, KB = 32, kStages = 4;
constexpr int kTileBytes = MB * KB * 2;   // 16 KB: one 256 x 32 bf16 tile
constexpr int kXcds = 8;

__shared__ __attribute__((aligned(16))) uint8_t g_a0[kTileBytes];
__shared__ __attribute__((aligned(16))) uint8_t g_a1[kTileBytes];
__shared__ __attribute__((aligned(16))) uint8_t g_a2[kTileBytes];
__shared__ __attribute__((aligned(16))) uint8_t g_a3[kTileBytes];
__shared__ __attribute__((aligned(16))) uint8_t g_w0[kTileBytes];
__shared__ __attribute__((aligned(16))) uint8_t g_w1[kTileBytes];
__shared__ __attribute__((aligned(16))) uint8_t g_w2[kTileBytes];
__shared__ __attribute__((aligned(16))) uint8_t g_w3[kTileBytes];

template <int S> __device__ __forceinline__ uint8_t* a_stage() {
  if constexpr (S == 0) return g_a0; else if constexpr (S == 1) return g_a1;
  else if constexpr (S == 2) return g_a2; else return g_a3;
}
template <int S> __device__ __forceinline__ uint8_t* w_stage() {
  if constexpr (S == 0) return g_w0; else if constexpr (S == 1) return g_w1;
  else if constexpr (S == 2) return g_w2; else return g_w3;
}

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * (KB * 2) + ((chunk ^ (((row >> 1) ^ (row >> 3)) & 3)) << 4);
}

#define KVR_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define KVR_GLB(p) ((const __attribute__((address_space(1))) void*)(p))

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] and
// vmcnt[5:4] at bits 15:14, expcnt[6:4] = 7, lgkmcnt[11:8] = 15).
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0xF70);
}

// Wave arrangement: WM x WN waves, each owning TM x TN blocks of 32 x 32.
template <int WM, int WN, int TM, int TN>
struct Cfg {
  static_assert(WM * TM * 32 == MB && WN * TN * 32 == NB, "256 x 256 workgroup tile");
  static constexpr int waves = WM * WN;
  static constexpr int threads = 64 * waves;
  static constexpr int loads = (MB / 16) / waves;   // 1 KB DMA slices per wave per operand
};

template <class C>
struct GemmThread {
  const bf16_t* asrc[C::loads];   // this lane's global source (A), at the split's first k
  const bf16_t* wsrc[C::loads];   // ... (W)
  int dst[C::loads];              // wave-uniform LDS byte offset of each 1 KB slice
  int arow[4], wrow[4];
  int khalf;
};

template <class C, int S>
__device__ __forceinline__ void issue_stage(const GemmThread<C>& g, int kb) {
#pragma unroll
  for (int j = 0; j < C::loads; ++j) {
    __builtin_amdgcn_global_load_lds(KVR_GLB(g.asrc[j] + kb), KVR_LDS(a_stage<S>() + g.dst[j]), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(KVR_GLB(g.wsrc[j] + kb), KVR_LDS(w_stage<S>() + g.dst[j]), 16, 0, 0);
  }
}

template <class C, int TM, int TN, int S>
__device__ __forceinline__ void mma_half(const GemmThread<C>& g, int ks, f32x16_t (&acc)[TM][TN]) {
  const uint8_t* a = a_stage<S>();
  const uint8_t* w = w_stage<S>();
  const int chunk = ks * 2 + g.khalf;
  bf16x8_t fa[TM], fw[TN];
#pragma unroll
  for (int mb = 0; mb < TM; ++mb) fa[mb] = *reinterpret_cast<const bf16x8_t*>(a + swz(g.arow[mb], chunk));
#pragma unroll
  for (int nb = 0; nb < TN; ++nb) fw[nb] = *reinterpret_cast<const bf16x8_t*>(w + swz(g.wrow[nb], chunk));
#pragma unroll
  for (int mb = 0; mb < TM; ++mb)
#pragma unroll
    for (int nb = 0; nb < TN; ++nb)
      acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mb], fw[nb], acc[mb][nb], 0, 0, 0);
}

// One K step on stage S (its data was certified by the previous barrier):
// the first 16-wide half is read and its MFMAs issued; then, with those in
// flight, wait until the next stage's DMA has landed (one newer stage may
// stay in flight), barrier (every wave is past the previous stage), refill
// the previous stage's buffers with the step three ahead (clamped to the last
// step: a refill past the end is never read), and run the second half.
template <class C, int TM, int TN, int S>
__device__ __forceinline__ void k_step(const GemmThread<C>& g, int i, int nsteps,
                                       f32x16_t (&acc)[TM][TN]) {
  mma_half<C, TM, TN, S>(g, 0, acc);
  wait_vmcnt<2 * C::loads>();
  __builtin_amdgcn_s_barrier();
  issue_stage<C, (S + 3) % kStages>(g, min(i + 3, nsteps - 1) * KB);
  mma_half<C, TM, TN, S>(g, 1, acc);
}

// MODE 0: part[split][M][N] = A * W^T over this split's K range (W segmented).
// MODE 1: W.w[0] = W_gate, W.w[1] = W_up; the tile holds 128 gate rows and the
//         same 128 up rows; out[M][N] = bf16(SiLU(gate) * up), full K.  A wave's
//         first TN/2 column blocks are gate columns, the last TN/2 the matching
//         up columns, so both factors of an output meet in one lane.
template <int MODE, int WM, int WN, int TM, int TN>
__global__ __launch_bounds__(64 * WM * WN, 1) void k_gemm_mfma(
    const bf16_t* __restrict__ A, WeightSegs W, int M, int N, int K, int k_per_split,
    int tiles_m, int tiles_n, int splits, float* __restrict__ part, bf16_t* __restrict__ out) {
  using C = Cfg<WM, WN, TM, TN>;
  // XCD-aware order: t = ((split * tiles_n) + n) * tiles_m + m
  const int total = tiles_m * tiles_n * splits;
  const int b = blockIdx.x, xcd = b % kXcds, q = total / kXcds, rem = total % kXcds;
  const int t = xcd * q + min(xcd, rem) + b / kXcds;
  const int tm = t % tiles_m, tn = (t / tiles_m) % tiles_n, split = t / (tiles_m * tiles_n);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int m0 = tm * MB;
  const int n0 = tn * (MODE == 1 ? NB / 2 : NB);
  const int k0 = split * k_per_split;
  const int k1 = min(K, k0 + k_per_split);
  const int nsteps = k1 > k0 ? (k1 - k0) / KB : 0;

  GemmThread<C> g;
#pragma unroll
  for (int j = 0; j < C::loads; ++j) {
    const int row0 = (wave * C::loads + j) * 16;
    const int row = row0 + (lane >> 2);                      // tile row this lane fetches
    const int chunk = (lane & 3) ^ (((row >> 1) ^ (row >> 3)) & 3);   // logical chunk of its slot
    g.dst[j] = row0 * (KB * 2);
    const int m = min(m0 + row, M - 1);
    g.asrc[j] = A + static_cast<size_t>(m) * K + k0 + chunk * 8;
    const bf16_t* wr;
    if (MODE == 0) {
      const int n = min(n0 + row, N - 1);
      int sj = 0;
      if (W.nseg > 1 && n >= W.n_begin[1]) sj = 1;
      if (W.nseg > 2 && n >= W.n_begin[2]) sj = 2;
      wr = static_cast<const bf16_t*>(W.w[sj]) + static_cast<size_t>(n - W.n_begin[sj]) * K;
    } else {
      const int n = min(n0 + (row & 127), N - 1);
      wr = static_cast<const bf16_t*>(W.w[row >> 7]) + static_cast<size_t>(n) * K;
    }
    g.wsrc[j] = wr + k0 + chunk * 8;
  }
#pragma unroll
  for (int mb = 0; mb < TM; ++mb) g.arow[mb] = (wm * TM + mb) * 32 + (lane & 31);
#pragma unroll
  for (int nb = 0; nb < TN; ++nb) {
    if (MODE == 0) g.wrow[nb] = (wn * TN + nb) * 32 + (lane & 31);
    else g.wrow[nb] = (nb < TN / 2 ? 0 : NB / 2) + (wn * (TN / 2) + nb % (TN / 2)) * 32 + (lane & 31);
  }
  g.khalf = lane >> 5;

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int mb = 0; mb < TM; ++mb)
#pragma unroll
    for (int nb = 0; nb < TN; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mb][nb][e] = 0.f;

  if (nsteps > 0) {
    issue_stage<C, 0>(g, 0);
    issue_stage<C, 1>(g, min(1, nsteps - 1) * KB);
    issue_stage<C, 2>(g, min(2, nsteps - 1) * KB);
    wait_vmcnt<4 * C::loads>();       // stage 0 landed; stages 1 and 2 may be in flight
    __builtin_amdgcn_s_barrier();
    int i = 0;
    for (; i + 4 <= nsteps; i += 4) {
      k_step<C, TM, TN, 0>(g, i, nsteps, acc);
      k_step<C, TM, TN, 1>(g, i + 1, nsteps, acc);
      k_step<C, TM, TN, 2>(g, i + 2, nsteps, acc);
      k_step<C, TM, TN, 3>(g, i + 3, nsteps, acc);
    }
    if (i < nsteps) k_step<C, TM, TN, 0>(g, i, nsteps, acc);
    if (i + 1 < nsteps) k_step<C, TM, TN, 1>(g, i + 1, nsteps, acc);
    if (i + 2 < nsteps) k_step<C, TM, TN, 2>(g, i + 2, nsteps, acc);
    wait_vmcnt<0>();
  }

  // epilogue
  const int khalf = g.khalf;
#pragma unroll
  for (int mb = 0; mb < TM; ++mb) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = m0 + (wm * TM + mb) * 32 + 8 * (e >> 2) + 4 * khalf + (e & 3);
      if (m >= M) continue;
      if (MODE == 0) {
        float* crow = part + (static_cast<size_t>(split) * M + m) * N;
#pragma unroll
        for (int nb = 0; nb < TN; ++nb) {
          const int n = n0 + (wn * TN + nb) * 32 + (lane & 31);
          if (n < N) crow[n] = acc[mb][nb][e];
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < TN / 2; ++nb) {
          const int n = n0 + (wn * (TN / 2) + nb) * 32 + (lane & 31);
          if (n < N) {
            const float gt = acc[mb][nb][e], up = acc[mb][nb + TN / 2][e];
            out[static_cast<size_t>(m) * N + n] = f32_to_bf16(gt / (1.f + expf(-gt)) * up);
          }
        }
      }
    }
  }
}

// Wave arrangement used by the library.
#ifndef KVR_GEMM_WAVES_M
#define KVR_GEMM_WAVES_M 4
#endif
constexpr int kWM = KVR_GEMM_WAVES_M, kWN = 2, kTM = 8 / kWM, kTN = 4;
constexpr int MT = 64 * kWM * kWN;

}  // namespace

// Split-K factor for the partial-output GEMMs: the smallest split that
// minimises the critical path (waves of 256 workgroups, one per CU, times the
// K steps per workgroup).  float32 storage does not split.
int gemm_splits_for(kvr_dtype dt, int M, int N, int K) {
  if (dt != KVR_BF16) return 1;
  const long tiles = static_cast<long>((M + MB - 1) / MB) * ((N + NB - 1) / NB);
  int best = 1;
  long best_cost = -1;
  for (int s = 1; s <= 8; ++s) {
    const long kps = ((K / s + KB - 1) / KB) * KB;
    if (kps < 2 * KB && s > 1) break;
    const long cost = ((tiles * s + 255) / 256) * kps;
    if (best_cost < 0 || cost < best_cost) { best_cost = cost; best = s; }
  }
  return best;
}

hipError_t launch_gemm_partial(kvr_dtype dt, const void* A, const WeightSegs& W, int M, int N,
                               int K, int splits, float* part, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (dt == KVR_BF16) {
    const int kps = ((K / splits + KB - 1) / KB) * KB;
    const int tm = (M + MB - 1) / MB, tn = (N + NB - 1) / NB;
    hipLaunchKernelGGL((k_gemm_mfma<0, kWM, kWN, kTM, kTN>), dim3(tm * tn * splits), dim3(MT), 0, stream,
                       static_cast<const bf16_t*>(A), W, M, N, K, kps, tm, tn, splits, part,
                       nullptr);
  } else {
    const int kps = ((K / splits + 63) / 64) * 64;
    dim3 grid((N + kTile - 1) / kTile, (M + kTile - 1) / kTile, splits);
    hipLaunchKernelGGL((k_gemm_fma<float, 0>), grid, dim3(kThreads), 0, stream,
                       static_cast<const float*>(A), W, M, N, K, kps, part, nullptr);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_swiglu(kvr_dtype dt, const void* A, const void* Wg, const void* Wu, int M,
                              int N, int K, void* out, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  WeightSegs W{{Wg, Wu, nullptr}, {0, N, N, N}, 2};
  if (dt == KVR_BF16) {
    const int tm = (M + MB - 1) / MB, tn = (N + NB / 2 - 1) / (NB / 2);
    hipLaunchKernelGGL((k_gemm_mfma<1, kWM, kWN, kTM, kTN>), dim3(tm * tn), dim3(MT), 0, stream,
                       static_cast<const bf16_t*>(A), W, M, N, K, K, tm, tn, 1, nullptr,
                       static_cast<bf16_t*>(out));
  } else {
    dim3 grid((N + kTile - 1) / kTile, (M + kTile - 1) / kTile, 1);
    hipLaunchKernelGGL((k_gemm_fma<float, 1>), grid, dim3(kThreads), 0, stream,
                       static_cast<const float*>(A), W, M, N, K, K, nullptr,
                       static_cast<float*>(out));
  }
  return hipGetLastError();
}

}  // namespace kvr
