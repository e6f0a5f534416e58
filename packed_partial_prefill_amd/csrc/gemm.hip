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
// Workgroup tile 256 (M) x 256 (N) x 64 (K), 8 waves; wave w owns rows
// (w/2)*64 .. +64 and a 128-column slice.  A (activations) and W tiles are
// staged in LDS, double-buffered, as rows of eight 16-byte chunks whose
// chunk index is XOR-swizzled with (row & 7) so that the 32 rows read by one
// MFMA operand load hit distinct banks.  MFMA operand layout (32x32x16):
// lane l supplies row/column l%32 and k = 8*(l/32) .. +7 of the 16-wide
// K slice; accumulator t of lane l is D[8*(t/4) + 4*(l/32) + t%4][l%32].
// ---------------------------------------------------------------------------
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

constexpr int MB = 256, NB = 256, KB = 64, MT = 512;
constexpr int kTileBytes = MB * KB * 2;              // one 256 x 64 bf16 tile
constexpr int kLdsBytes = 2 * 2 * kTileBytes;        // A and W, double-buffered

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * (KB * 2) + (((chunk ^ (row & 7))) << 4);
}

// MODE 0: part[split][M][N] = A * W^T over this split's K range (W segmented).
// MODE 1: W.w[0] = W_gate, W.w[1] = W_up; the tile holds 128 gate rows and the
//         same 128 up rows; out[M][N] = bf16(SiLU(gate) * up), full K.
template <int MODE>
__global__ __launch_bounds__(MT, 1) void k_gemm_mfma(const bf16_t* __restrict__ A, WeightSegs W,
                                                     int M, int N, int K, int k_per_split,
                                                     float* __restrict__ part,
                                                     bf16_t* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * MB;
  const int n0 = blockIdx.x * (MODE == 1 ? NB / 2 : NB);
  const int k0 = blockIdx.z * k_per_split;
  const int k1 = min(K, k0 + k_per_split);

  // global source rows of the 4 + 4 chunks this thread stages per K step
  const u32x4_t* asrc[4];
  const u32x4_t* wsrc[4];
  int lofs[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int v = tid + i * MT;
    const int row = v >> 3, chunk = v & 7;
    lofs[i] = swz(row, chunk);
    const int m = min(m0 + row, M - 1);
    asrc[i] = reinterpret_cast<const u32x4_t*>(A + static_cast<size_t>(m) * K + chunk * 8);
    const bf16_t* wrow;
    if (MODE == 0) {
      const int n = min(n0 + row, N - 1);
      int j = 0;
      if (W.nseg > 1 && n >= W.n_begin[1]) j = 1;
      if (W.nseg > 2 && n >= W.n_begin[2]) j = 2;
      wrow = static_cast<const bf16_t*>(W.w[j]) + static_cast<size_t>(n - W.n_begin[j]) * K;
    } else {
      const int n = min(n0 + (row & 127), N - 1);
      wrow = static_cast<const bf16_t*>(W.w[row >> 7]) + static_cast<size_t>(n) * K;
    }
    wsrc[i] = reinterpret_cast<const u32x4_t*>(wrow + chunk * 8);
  }

  u32x4_t ra[4], rw[4];
  auto gload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = asrc[i][kb >> 3];
      rw[i] = wsrc[i][kb >> 3];
    }
  };
  auto lstore = [&](int buf) {
    uint8_t* a = lds + buf * 2 * kTileBytes;
    uint8_t* w = a + kTileBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4_t*>(a + lofs[i]) = ra[i];
      *reinterpret_cast<u32x4_t*>(w + lofs[i]) = rw[i];
    }
  };

  // LDS rows this lane reads as MFMA operands
  int arow[2], wrow_l[4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) arow[mb] = wm * 64 + mb * 32 + (lane & 31);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    if (MODE == 0) wrow_l[nb] = wn * 128 + nb * 32 + (lane & 31);
    else wrow_l[nb] = (nb < 2 ? 0 : 128) + wn * 64 + (nb & 1) * 32 + (lane & 31);
  }
  const int khalf = lane >> 5;

  f32x16_t acc[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int t = 0; t < 16; ++t) acc[mb][nb][t] = 0.f;

  if (k0 < k1) {
    gload(k0);
    lstore(0);
  }
  __syncthreads();
  int cur = 0;
  for (int kb = k0; kb < k1; kb += KB) {
    const bool more = kb + KB < k1;
    if (more) gload(kb + KB);
    const uint8_t* a = lds + cur * 2 * kTileBytes;
    const uint8_t* w = a + kTileBytes;
#pragma unroll
    for (int ks = 0; ks < KB / 16; ++ks) {
      const int chunk = ks * 2 + khalf;
      bf16x8_t fa[2], fw[4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        fa[mb] = *reinterpret_cast<const bf16x8_t*>(a + swz(arow[mb], chunk));
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        fw[nb] = *reinterpret_cast<const bf16x8_t*>(w + swz(wrow_l[nb], chunk));
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mb], fw[nb], acc[mb][nb], 0, 0, 0);
    }
    if (more) lstore(cur ^ 1);
    __syncthreads();
    cur ^= 1;
  }

  // epilogue
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int m = m0 + wm * 64 + mb * 32 + 8 * (t >> 2) + 4 * khalf + (t & 3);
      if (m >= M) continue;
      if (MODE == 0) {
        float* crow = part + (static_cast<size_t>(blockIdx.z) * M + m) * N;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int n = n0 + wn * 128 + nb * 32 + (lane & 31);
          if (n < N) crow[n] = acc[mb][nb][t];
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int n = n0 + wn * 64 + nb * 32 + (lane & 31);
          if (n < N) {
            const float g = acc[mb][nb][t], u = acc[mb][nb + 2][t];
            out[static_cast<size_t>(m) * N + n] = f32_to_bf16(g / (1.f + expf(-g)) * u);
          }
        }
      }
    }
  }
}

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

namespace {
bool g_lds_attr_set = false;
hipError_t set_lds_attr() {
  if (g_lds_attr_set) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_mfma<0>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_mfma<1>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (e == hipSuccess) g_lds_attr_set = true;
  return e;
}
}  // namespace

hipError_t launch_gemm_partial(kvr_dtype dt, const void* A, const WeightSegs& W, int M, int N,
                               int K, int splits, float* part, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int kps = ((K / splits + 63) / 64) * 64;
  if (dt == KVR_BF16) {
    hipError_t e = set_lds_attr();
    if (e != hipSuccess) return e;
    dim3 grid((N + NB - 1) / NB, (M + MB - 1) / MB, splits);
    hipLaunchKernelGGL((k_gemm_mfma<0>), grid, dim3(MT), kLdsBytes, stream,
                       static_cast<const bf16_t*>(A), W, M, N, K, kps, part, nullptr);
  } else {
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
    hipError_t e = set_lds_attr();
    if (e != hipSuccess) return e;
    dim3 grid((N + NB / 2 - 1) / (NB / 2), (M + MB - 1) / MB, 1);
    hipLaunchKernelGGL((k_gemm_mfma<1>), grid, dim3(MT), kLdsBytes, stream,
                       static_cast<const bf16_t*>(A), W, M, N, K, K, nullptr,
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
