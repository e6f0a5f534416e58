// Fused RoPE + K/V write-back for the packed rows.
//
// For row r at position u = T[r]: the QKV projection's split-K partials are
// summed (plus optional biases), q and k are rotated at u (rotate-half
// pairing (i, i+d/2), angle u * theta^(-2i/d), from the per-call float64
// table), q is stored for attention (times the attention kernel's score
// factor, folded in here), and the fresh k, v overwrite cache row
// u before attention runs ("Budgeted KV-Cache Repair", section 13.2, Eq. 21);
// the position's metadata becomes global with the sink bit cleared
// (cross-attention reuse page, 6.4: write-back sets type <- global).
#include "common.h"
#include "kvr_internal.h"
#include "tables.h"

namespace kvr {

namespace {

constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ void put4(T* p, float4 v);
template <>
__device__ __forceinline__ void put4<float>(float* p, float4 v) {
  *reinterpret_cast<float4*>(p) = v;
}
template <>
__device__ __forceinline__ void put4<bf16_t>(bf16_t* p, float4 v) {
  uint2 w;
  w.x = static_cast<uint32_t>(f32_to_bf16(v.x)) | (static_cast<uint32_t>(f32_to_bf16(v.y)) << 16);
  w.y = static_cast<uint32_t>(f32_to_bf16(v.z)) | (static_cast<uint32_t>(f32_to_bf16(v.w)) << 16);
  *reinterpret_cast<uint2*>(p) = w;
}

__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// Sum of the split-K partials of 4 consecutive columns starting at c (in
// split order; unrolled by 4 so that those loads are in flight together).
__device__ __forceinline__ float4 cols4(const float* pr, int splits, size_t split_stride, int c) {
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int s = 0; s < splits; ++s)
    a = add4(a, *reinterpret_cast<const float4*>(pr + s * split_stride + c));
  return a;
}

// The same for the columns c and c + half of a rotated pair, in one loop.
__device__ __forceinline__ void cols4x2(const float* pr, int splits, size_t split_stride, int c,
                                        int half, float4& a, float4& b) {
  a = make_float4(0.f, 0.f, 0.f, 0.f);
  b = a;
#pragma unroll 4
  for (int s = 0; s < splits; ++s) {
    const float4 pa = *reinterpret_cast<const float4*>(pr + s * split_stride + c);
    const float4 pb = *reinterpret_cast<const float4*>(pr + s * split_stride + c + half);
    a = add4(a, pa);
    b = add4(b, pb);
  }
}

// Rotate 4 consecutive pairs (i .. i+3, i+half .. i+half+3) of one head.
template <typename T>
__device__ __forceinline__ void rotate4(const float* pr, int splits, size_t split_stride,
                                        const float* bias, int c0, int half,
                                        const float2* tr, float scale, T* dst) {
  float4 a, b;
  cols4x2(pr, splits, split_stride, c0, half, a, b);
  if (bias) {
    a = add4(a, *reinterpret_cast<const float4*>(bias + c0));
    b = add4(b, *reinterpret_cast<const float4*>(bias + c0 + half));
  }
  const float4 t01 = *reinterpret_cast<const float4*>(tr);       // (cos, sin) of pairs i, i+1
  const float4 t23 = *reinterpret_cast<const float4*>(tr + 2);   // pairs i+2, i+3
  const float c[4] = {t01.x, t01.z, t23.x, t23.z}, sn[4] = {t01.y, t01.w, t23.y, t23.w};
  const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
  float lo[4], hi[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    lo[j] = (av[j] * c[j] - bv[j] * sn[j]) * scale;
    hi[j] = (bv[j] * c[j] + av[j] * sn[j]) * scale;
  }
  put4<T>(dst, make_float4(lo[0], lo[1], lo[2], lo[3]));
  put4<T>(dst + half, make_float4(hi[0], hi[1], hi[2], hi[3]));
}

// (at most 4 waves per SIMD, so that the scheduler keeps the partial loads of
// an item in flight together rather than reusing one register set)
template <typename T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 4))) void k_rope_writeback(
    const float* __restrict__ part, int splits, size_t split_stride, const float* __restrict__ bq,
    const float* __restrict__ bk, const float* __restrict__ bv, const float2* __restrict__ tab,
    const int32_t* __restrict__ Tpos, int B, Shape sh, float q_scale, T* __restrict__ q_out,
    T* __restrict__ kc, T* __restrict__ vc, uint8_t* __restrict__ flags) {
  // One thread per item of a row: 4 rotated pairs of a query head, 4 rotated
  // pairs of a key head, or 4 value columns (every load of the launch is
  // then in flight at once; a workgroup per row looped over its items).
  const int d = sh.d, half = d >> 1, q4 = half >> 2, ncols = sh.qkv_cols();
  const int n_q = sh.hq * q4, n_k = sh.hkv * q4, n_v = sh.hkv * (d >> 2);
  const int per_row = n_q + n_k + n_v;
  const size_t t = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (t >= static_cast<size_t>(B) * per_row) return;
  const int r = static_cast<int>(t / per_row);
  int idx = static_cast<int>(t - static_cast<size_t>(r) * per_row);
  const int u = Tpos[r];
  const float* pr = part + static_cast<size_t>(r) * ncols;
  const float2* tr = tab + static_cast<size_t>(r) * half;
  if (idx < n_q) {   // query heads (times the attention kernel's score factor)
    const int h = idx / q4, i = (idx - h * q4) * 4;
    rotate4<T>(pr, splits, split_stride, bq, h * d + i, half, tr + i, q_scale,
               q_out + (static_cast<size_t>(r) * sh.hq + h) * d + i);
    return;
  }
  idx -= n_q;
  if (idx < n_k) {   // key heads: rotated, written to cache row u
    const int g = idx / q4, i = (idx - g * q4) * 4;
    rotate4<T>(pr + sh.hq * d, splits, split_stride, bk, g * d + i, half, tr + i, 1.f,
               kc + (static_cast<size_t>(u) * sh.hkv + g) * d + i);
    if (idx == 0)
      flags[u] = static_cast<uint8_t>(flags[u] & ~(KVR_FLAG_LOCAL | KVR_FLAG_SINK));
    return;
  }
  idx -= n_k;        // values: copied to cache row u
  const int vbase = (sh.hq + sh.hkv) * d;
  float4 a = cols4(pr, splits, split_stride, vbase + idx * 4);
  if (bv) a = add4(a, *reinterpret_cast<const float4*>(bv + idx * 4));
  put4<T>(vc + static_cast<size_t>(u) * sh.hkv * d + idx * 4, a);
}

// Queries handed in from outside the repair (inference mode): scaled by the
// attention kernel's score factor and stored in the cache's dtype.  The
// workgroups past the queries' build the attention plan of the query
// positions ("Budgeted KV-Cache Repair", section 13.2, Eq. 23-24), so that
// it takes no launch of its own.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_prep_queries(
    const float4* __restrict__ q, size_t n4, float scale, T* __restrict__ out, unsigned qblocks,
    const int32_t* __restrict__ pos, int B, int group, int n_tiles, int32_t* __restrict__ n_full,
    int32_t* __restrict__ n_total) {
  if (blockIdx.x >= qblocks) {
    const int t = static_cast<int>(blockIdx.x - qblocks) * kThreads + threadIdx.x;
    if (t < n_tiles) plan_entry(pos, B, group, t, n_full, n_total);
    return;
  }
  const size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= n4) return;
  const float4 v = q[i];
  put4<T>(out + 4 * i, make_float4(v.x * scale, v.y * scale, v.z * scale, v.w * scale));
}

}  // namespace

hipError_t launch_prep_queries(kvr_dtype dt, const float* q, size_t n, float scale, void* q_out,
                               const int32_t* pos, int B, int group, int32_t* n_full,
                               int32_t* n_total, hipStream_t stream) {
  const size_t n4 = n / 4;
  const int n_tiles = plan_tiles(B, group);
  const unsigned qblocks = static_cast<unsigned>((n4 + kThreads - 1) / kThreads);
  const dim3 grid(qblocks + static_cast<unsigned>((n_tiles + kThreads - 1) / kThreads));
  if (grid.x == 0) return hipSuccess;
  if (dt == KVR_BF16)
    hipLaunchKernelGGL(k_prep_queries<bf16_t>, grid, dim3(kThreads), 0, stream,
                       reinterpret_cast<const float4*>(q), n4, scale, static_cast<bf16_t*>(q_out),
                       qblocks, pos, B, group, n_tiles, n_full, n_total);
  else
    hipLaunchKernelGGL(k_prep_queries<float>, grid, dim3(kThreads), 0, stream,
                       reinterpret_cast<const float4*>(q), n4, scale, static_cast<float*>(q_out),
                       qblocks, pos, B, group, n_tiles, n_full, n_total);
  return hipGetLastError();
}

hipError_t launch_rope_writeback(kvr_dtype dt, const float* qkv_part, int splits,
                                 size_t split_stride, const float* bq, const float* bk,
                                 const float* bv, const float2* tab, const int32_t* T, int B,
                                 const Shape& sh, float q_scale, void* q_out, void* k_cache,
                                 void* v_cache, uint8_t* flags, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  const int q4 = sh.d / 8;
  const size_t items = static_cast<size_t>(B) * ((sh.hq + sh.hkv) * q4 + sh.hkv * (sh.d / 4));
  const dim3 grid(static_cast<unsigned>((items + kThreads - 1) / kThreads));
  if (dt == KVR_BF16)
    hipLaunchKernelGGL(k_rope_writeback<bf16_t>, grid, dim3(kThreads), 0, stream, qkv_part,
                       splits, split_stride, bq, bk, bv, tab, T, B, sh, q_scale,
                       static_cast<bf16_t*>(q_out), static_cast<bf16_t*>(k_cache),
                       static_cast<bf16_t*>(v_cache), flags);
  else
    hipLaunchKernelGGL(k_rope_writeback<float>, grid, dim3(kThreads), 0, stream, qkv_part,
                       splits, split_stride, bq, bk, bv, tab, T, B, sh, q_scale,
                       static_cast<float*>(q_out), static_cast<float*>(k_cache),
                       static_cast<float*>(v_cache), flags);
  return hipGetLastError();
}

}  // namespace kvr
