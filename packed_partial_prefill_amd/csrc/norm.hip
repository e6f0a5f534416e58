// Row kernels on the packed residual stream: the one-time gather of the
// selected rows (the compact B-row hidden buffer of "Budgeted KV-Cache
// Repair", section 13.2), split-K partial sums added to the residual, and
// RMSNorm producing the next GEMM's operand.
#include "common.h"
#include "kvr_internal.h"

namespace kvr {

namespace {

constexpr int kRowThreads = 256;
constexpr int kMaxPerThread = 32;  // hidden <= 8192

template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_gather_norm(
    const float* __restrict__ x_in, const int32_t* __restrict__ gather_T, float* x_res,
    const float* __restrict__ gamma, float eps, T* __restrict__ n_out, int hidden) {
  __shared__ float red[16];
  const int r = blockIdx.x;
  const size_t src = gather_T ? static_cast<size_t>(gather_T[r]) : static_cast<size_t>(r);
  const float* xr = x_in + src * hidden;
  float v[kMaxPerThread];
  float ss = 0.f;
  int c = 0;
  for (int j = threadIdx.x; j < hidden; j += kRowThreads, ++c) {
    v[c] = xr[j];
    ss += v[c] * v[c];
  }
  const float tot = block_sum(ss, red);  // all reads of x_in precede any write
  const float rs = rsqrtf(tot / hidden + eps);
  float* xo = x_res + static_cast<size_t>(r) * hidden;
  T* no = n_out + static_cast<size_t>(r) * hidden;
  c = 0;
  for (int j = threadIdx.x; j < hidden; j += kRowThreads, ++c) {
    xo[j] = v[c];
    Elem<T>::store(no, j, v[c] * rs * gamma[j]);
  }
}

template <typename T>
__global__ __launch_bounds__(kRowThreads) void k_residual_norm(
    float* __restrict__ x_res, const float* __restrict__ part, int splits, size_t split_stride,
    const float* __restrict__ gamma, float eps, T* __restrict__ n_out, int hidden) {
  __shared__ float red[16];
  const int r = blockIdx.x;
  float* xr = x_res + static_cast<size_t>(r) * hidden;
  const float* pr = part + static_cast<size_t>(r) * hidden;
  float v[kMaxPerThread];
  float ss = 0.f;
  int c = 0;
  for (int j = threadIdx.x; j < hidden; j += kRowThreads, ++c) {
    float a = 0.f;
    for (int s = 0; s < splits; ++s) a += pr[s * split_stride + j];
    v[c] = xr[j] + a;
    xr[j] = v[c];
    ss += v[c] * v[c];
  }
  if (gamma == nullptr) return;
  const float tot = block_sum(ss, red);
  const float rs = rsqrtf(tot / hidden + eps);
  T* no = n_out + static_cast<size_t>(r) * hidden;
  c = 0;
  for (int j = threadIdx.x; j < hidden; j += kRowThreads, ++c) Elem<T>::store(no, j, v[c] * rs * gamma[j]);
}

}  // namespace

hipError_t launch_gather_norm(kvr_dtype dt, const float* x_in, const int32_t* gather_T,
                              float* x_res, const float* gamma, float eps, void* n_out, int B,
                              int hidden, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  if (dt == KVR_BF16)
    hipLaunchKernelGGL(k_gather_norm<bf16_t>, dim3(B), dim3(kRowThreads), 0, stream, x_in,
                       gather_T, x_res, gamma, eps, static_cast<bf16_t*>(n_out), hidden);
  else
    hipLaunchKernelGGL(k_gather_norm<float>, dim3(B), dim3(kRowThreads), 0, stream, x_in,
                       gather_T, x_res, gamma, eps, static_cast<float*>(n_out), hidden);
  return hipGetLastError();
}

hipError_t launch_residual_norm(kvr_dtype dt, float* x_res, const float* part, int splits,
                                size_t split_stride, const float* gamma, float eps, void* n_out,
                                int B, int hidden, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  if (dt == KVR_BF16)
    hipLaunchKernelGGL(k_residual_norm<bf16_t>, dim3(B), dim3(kRowThreads), 0, stream, x_res,
                       part, splits, split_stride, gamma, eps, static_cast<bf16_t*>(n_out),
                       hidden);
  else
    hipLaunchKernelGGL(k_residual_norm<float>, dim3(B), dim3(kRowThreads), 0, stream, x_res,
                       part, splits, split_stride, gamma, eps, static_cast<float*>(n_out),
                       hidden);
  return hipGetLastError();
}

}  // namespace kvr
