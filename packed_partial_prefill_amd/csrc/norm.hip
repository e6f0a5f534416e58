// Row kernels on the packed residual stream: the one-time gather of the
// selected rows (the compact B-row hidden buffer of "Budgeted KV-Cache
// Repair", section 13.2), split-K partial sums added to the residual, and
// RMSNorm producing the next GEMM's operand.  One workgroup per row; every
// thread owns float4 chunks of the row (hidden is a multiple of 64).
#include "common.h"
#include "kvr_internal.h"
#include "tables.h"

namespace kvr {

namespace {

constexpr int kRowThreads = 256;
constexpr int kMaxChunks = 8;  // float4 chunks per thread: hidden <= 8192

template <typename T>
__device__ __forceinline__ void store4(T* row, int j4, float4 v);
template <>
__device__ __forceinline__ void store4<float>(float* row, int j4, float4 v) {
  reinterpret_cast<float4*>(row)[j4] = v;
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* row, int j4, float4 v) {
  uint2 p;
  p.x = static_cast<uint32_t>(f32_to_bf16(v.x)) | (static_cast<uint32_t>(f32_to_bf16(v.y)) << 16);
  p.y = static_cast<uint32_t>(f32_to_bf16(v.z)) | (static_cast<uint32_t>(f32_to_bf16(v.w)) << 16);
  reinterpret_cast<uint2*>(row)[j4] = p;
}

__device__ __forceinline__ float4 scale4(float4 v, float s, float4 g) {
  return make_float4(v.x * s * g.x, v.y * s * g.y, v.z * s * g.z, v.w * s * g.w);
}

// x_res[r] = x_in[gather_T[r]] (or x_in[r]); n_out[r] = RMSNorm(x_res[r]) * gamma.
// NC = float4 chunks per thread; chunks past the row's end load its last
// chunk (discarded) so that every load is unconditional and all of them,
// gamma's included, are in flight together.  Workgroups past the B rows
// build the call's tables (LayerTables), one entry per thread; they run
// beside the row workgroups, so the tables need no launch of their own.
template <typename T, int NC>
__global__ __launch_bounds__(kRowThreads) __attribute__((amdgpu_waves_per_eu(1, 4))) void k_gather_norm(
    const float* __restrict__ x_in, const int32_t* __restrict__ gather_T, float* x_res,
    const float* __restrict__ gamma, float eps, T* __restrict__ n_out, int hidden, int B,
    LayerTables tabs) {
  __shared__ float red[16];
  const int r = blockIdx.x;
  if (r >= B) {
    table_entry(tabs, (r - B) * kRowThreads + static_cast<int>(threadIdx.x));
    return;
  }
  const int h4 = hidden >> 2;
  const size_t src = gather_T ? static_cast<size_t>(gather_T[r]) : static_cast<size_t>(r);
  const float4* xr = reinterpret_cast<const float4*>(x_in + src * hidden);
  const float4* g4 = reinterpret_cast<const float4*>(gamma);
  int jc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) jc[c] = min(static_cast<int>(threadIdx.x) + c * kRowThreads, h4 - 1);
  float4 v[NC], g[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) v[c] = xr[jc[c]];
#pragma unroll
  for (int c = 0; c < NC; ++c) g[c] = g4[jc[c]];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const float q = v[c].x * v[c].x + v[c].y * v[c].y + v[c].z * v[c].z + v[c].w * v[c].w;
    ss += static_cast<int>(threadIdx.x) + c * kRowThreads < h4 ? q : 0.f;
  }
  const float tot = block_sum(ss, red);  // all reads of x_in precede any write
  const float rs = rsqrtf(tot / hidden + eps);
  float4* xo = reinterpret_cast<float4*>(x_res + static_cast<size_t>(r) * hidden);
  T* no = n_out + static_cast<size_t>(r) * hidden;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int j4 = threadIdx.x + c * kRowThreads;
    if (j4 < h4) {
      xo[j4] = v[c];
      store4<T>(no, j4, scale4(v[c], rs, g[c]));
    }
  }
}

// x_res[r] += sum_s part[s][r]; when gamma is given, n_out[r] = RMSNorm(x_res[r]) * gamma.
// NC = float4 chunks per thread, ceil(hidden / 4 / kRowThreads).
// (at most 4 waves per SIMD: room for every chunk's loads in flight; the
// default occupancy target made the scheduler reuse one register set and
// wait for each load)
template <typename T, int NC>
__global__ __launch_bounds__(kRowThreads) __attribute__((amdgpu_waves_per_eu(1, 4))) void k_residual_norm(
    float* __restrict__ x_res, const float* __restrict__ part, int splits, size_t split_stride,
    const float* __restrict__ gamma, float eps, T* __restrict__ n_out, int hidden) {
  __shared__ float red[16];
  const int r = blockIdx.x;
  const int h4 = hidden >> 2;
  float4* xr = reinterpret_cast<float4*>(x_res + static_cast<size_t>(r) * hidden);
  const float4* pr = reinterpret_cast<const float4*>(part + static_cast<size_t>(r) * hidden);
  const size_t ps4 = split_stride >> 2;
  // Chunks past the row's end read its last chunk (discarded), so that the
  // loads need no branch and every chunk's loads (residual, then the
  // partials in split order) can be in flight together.
  int jc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) jc[c] = min(static_cast<int>(threadIdx.x) + c * kRowThreads, h4 - 1);
  float4 v[NC];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) v[c] = xr[jc[c]];
#pragma unroll 4
  for (int s = 0; s < splits; ++s) {
    float4 p[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) p[c] = pr[s * ps4 + jc[c]];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      v[c].x += p[c].x; v[c].y += p[c].y; v[c].z += p[c].z; v[c].w += p[c].w;
    }
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int j4 = threadIdx.x + c * kRowThreads;
    if (j4 < h4) {
      const float4 a = v[c];
      xr[j4] = a;
      ss += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
    }
  }
  if (gamma == nullptr) return;
  const float tot = block_sum(ss, red);
  const float rs = rsqrtf(tot / hidden + eps);
  T* no = n_out + static_cast<size_t>(r) * hidden;
  const float4* g4 = reinterpret_cast<const float4*>(gamma);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int j4 = threadIdx.x + c * kRowThreads;
    if (j4 < h4) store4<T>(no, j4, scale4(v[c], rs, g4[j4]));
  }
}

template <typename T, int NC>
void launch_residual_norm_t(float* x_res, const float* part, int splits, size_t split_stride,
                            const float* gamma, float eps, T* n_out, int B, int hidden,
                            hipStream_t stream) {
  if constexpr (NC < kMaxChunks) {
    if (hidden > 4 * kRowThreads * NC) {
      launch_residual_norm_t<T, NC + 1>(x_res, part, splits, split_stride, gamma, eps, n_out, B,
                                        hidden, stream);
      return;
    }
  }
  hipLaunchKernelGGL((k_residual_norm<T, NC>), dim3(B), dim3(kRowThreads), 0, stream, x_res, part,
                     splits, split_stride, gamma, eps, n_out, hidden);
}

template <typename T, int NC>
void launch_gather_norm_t(const float* x_in, const int32_t* gather_T, float* x_res,
                          const float* gamma, float eps, T* n_out, int B, int hidden,
                          const LayerTables& tabs, hipStream_t stream) {
  if constexpr (NC < kMaxChunks) {
    if (hidden > 4 * kRowThreads * NC) {
      launch_gather_norm_t<T, NC + 1>(x_in, gather_T, x_res, gamma, eps, n_out, B, hidden, tabs,
                                      stream);
      return;
    }
  }
  const int table_groups = (tabs.entries() + kRowThreads - 1) / kRowThreads;
  hipLaunchKernelGGL((k_gather_norm<T, NC>), dim3(B + table_groups), dim3(kRowThreads), 0, stream,
                     x_in, gather_T, x_res, gamma, eps, n_out, hidden, B, tabs);
}

}  // namespace

hipError_t launch_gather_norm(kvr_dtype dt, const float* x_in, const int32_t* gather_T,
                              float* x_res, const float* gamma, float eps, void* n_out, int B,
                              int hidden, const LayerTables* tabs, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  const LayerTables none{nullptr, nullptr, 0, 1, 0, nullptr, nullptr, 0, 0.0, nullptr};
  const LayerTables& t = tabs ? *tabs : none;
  if (dt == KVR_BF16)
    launch_gather_norm_t<bf16_t, 1>(x_in, gather_T, x_res, gamma, eps, static_cast<bf16_t*>(n_out),
                                    B, hidden, t, stream);
  else
    launch_gather_norm_t<float, 1>(x_in, gather_T, x_res, gamma, eps, static_cast<float*>(n_out),
                                   B, hidden, t, stream);
  return hipGetLastError();
}

hipError_t launch_residual_norm(kvr_dtype dt, float* x_res, const float* part, int splits,
                                size_t split_stride, const float* gamma, float eps, void* n_out,
                                int B, int hidden, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  if (dt == KVR_BF16)
    launch_residual_norm_t<bf16_t, 1>(x_res, part, splits, split_stride, gamma, eps,
                                      static_cast<bf16_t*>(n_out), B, hidden, stream);
  else
    launch_residual_norm_t<float, 1>(x_res, part, splits, split_stride, gamma, eps,
                                     static_cast<float*>(n_out), B, hidden, stream);
  return hipGetLastError();
}

}  // namespace kvr
