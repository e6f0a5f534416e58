// Dense projections of the packed rows: QKV, O, gate/up (+SwiGLU) and down.
// C = A * W^T with A [M, K] (packed activations) and W [N, K] (PyTorch
// Linear layout); both operands are K-contiguous.
//
// This file holds the portable float32-FMA tiled kernel, used for float32
// storage and as the fallback shape path.
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

}  // namespace

int gemm_splits_for(kvr_dtype, int, int, int) { return 1; }

hipError_t launch_gemm_partial(kvr_dtype dt, const void* A, const WeightSegs& W, int M, int N,
                               int K, int splits, float* part, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int kps = ((K / splits + 63) / 64) * 64;
  dim3 grid((N + kTile - 1) / kTile, (M + kTile - 1) / kTile, splits);
  if (dt == KVR_BF16)
    hipLaunchKernelGGL((k_gemm_fma<bf16_t, 0>), grid, dim3(kThreads), 0, stream,
                       static_cast<const bf16_t*>(A), W, M, N, K, kps, part, nullptr);
  else
    hipLaunchKernelGGL((k_gemm_fma<float, 0>), grid, dim3(kThreads), 0, stream,
                       static_cast<const float*>(A), W, M, N, K, kps, part, nullptr);
  return hipGetLastError();
}

hipError_t launch_gemm_swiglu(kvr_dtype dt, const void* A, const void* Wg, const void* Wu, int M,
                              int N, int K, void* out, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  WeightSegs W{{Wg, Wu, nullptr}, {0, N, N, N}, 2};
  dim3 grid((N + kTile - 1) / kTile, (M + kTile - 1) / kTile, 1);
  if (dt == KVR_BF16)
    hipLaunchKernelGGL((k_gemm_fma<bf16_t, 1>), grid, dim3(kThreads), 0, stream,
                       static_cast<const bf16_t*>(A), W, M, N, K, K, nullptr,
                       static_cast<bf16_t*>(out));
  else
    hipLaunchKernelGGL((k_gemm_fma<float, 1>), grid, dim3(kThreads), 0, stream,
                       static_cast<const float*>(A), W, M, N, K, K, nullptr,
                       static_cast<float*>(out));
  return hipGetLastError();
}

}  // namespace kvr
