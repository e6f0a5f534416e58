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

namespace kvr {

namespace {

constexpr int kThreads = 256;

template <typename T>
__global__ __launch_bounds__(kThreads) void k_rope_writeback(
    const float* __restrict__ part, int splits, size_t split_stride, const float* __restrict__ bq,
    const float* __restrict__ bk, const float* __restrict__ bv, const float2* __restrict__ tab,
    const int32_t* __restrict__ Tpos, Shape sh, float q_scale, T* __restrict__ q_out,
    T* __restrict__ kc,
    T* __restrict__ vc, uint8_t* __restrict__ flags) {
  const int r = blockIdx.x;
  const int u = Tpos[r];
  const int d = sh.d, half = d >> 1, ncols = sh.qkv_cols();
  const float* pr = part + static_cast<size_t>(r) * ncols;
  const float2* tr = tab + static_cast<size_t>(r) * half;
  auto col = [&](int c) {
    float a = 0.f;
    for (int s = 0; s < splits; ++s) a += pr[s * split_stride + c];
    return a;
  };
  // query heads
  for (int idx = threadIdx.x; idx < sh.hq * half; idx += kThreads) {
    const int h = idx / half, i = idx - h * half;
    const int c0 = h * d + i;
    float a = col(c0), b = col(c0 + half);
    if (bq) { a += bq[c0]; b += bq[c0 + half]; }
    const float2 cs = tr[i];
    T* qo = q_out + (static_cast<size_t>(r) * sh.hq + h) * d;
    Elem<T>::store(qo, i, (a * cs.x - b * cs.y) * q_scale);
    Elem<T>::store(qo, i + half, (b * cs.x + a * cs.y) * q_scale);
  }
  // key heads: rotated, written to cache row u
  const int kbase = sh.hq * d;
  for (int idx = threadIdx.x; idx < sh.hkv * half; idx += kThreads) {
    const int g = idx / half, i = idx - g * half;
    const int c0 = g * d + i;
    float a = col(kbase + c0), b = col(kbase + c0 + half);
    if (bk) { a += bk[c0]; b += bk[c0 + half]; }
    const float2 cs = tr[i];
    T* ko = kc + (static_cast<size_t>(u) * sh.hkv + g) * d;
    Elem<T>::store(ko, i, a * cs.x - b * cs.y);
    Elem<T>::store(ko, i + half, b * cs.x + a * cs.y);
  }
  // values: copied to cache row u
  const int vbase = (sh.hq + sh.hkv) * d;
  for (int idx = threadIdx.x; idx < sh.hkv * d; idx += kThreads) {
    float a = col(vbase + idx);
    if (bv) a += bv[idx];
    Elem<T>::store(vc + static_cast<size_t>(u) * sh.hkv * d, idx, a);
  }
  if (threadIdx.x == 0) flags[u] = static_cast<uint8_t>(flags[u] & ~(KVR_FLAG_LOCAL | KVR_FLAG_SINK));
}

}  // namespace

hipError_t launch_rope_writeback(kvr_dtype dt, const float* qkv_part, int splits,
                                 size_t split_stride, const float* bq, const float* bk,
                                 const float* bv, const float2* tab, const int32_t* T, int B,
                                 const Shape& sh, float q_scale, void* q_out, void* k_cache,
                                 void* v_cache, uint8_t* flags, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  if (dt == KVR_BF16)
    hipLaunchKernelGGL(k_rope_writeback<bf16_t>, dim3(B), dim3(kThreads), 0, stream, qkv_part,
                       splits, split_stride, bq, bk, bv, tab, T, sh, q_scale, static_cast<bf16_t*>(q_out),
                       static_cast<bf16_t*>(k_cache), static_cast<bf16_t*>(v_cache), flags);
  else
    hipLaunchKernelGGL(k_rope_writeback<float>, dim3(B), dim3(kThreads), 0, stream, qkv_part,
                       splits, split_stride, bq, bk, bv, tab, T, sh, q_scale, static_cast<float*>(q_out),
                       static_cast<float*>(k_cache), static_cast<float*>(v_cache), flags);
  return hipGetLastError();
}

}  // namespace kvr
