// Packed causal attention over the mixed cache with the metadata bias.
//
// Query row r (position u = T[r]), head h reads KV head g = h / (Hq/Hkv)
// over keys j = 0..u inclusive ("Budgeted KV-Cache Repair", section 13.2,
// Eq. 22) with logits <q, k_j>/sqrt(d) + alpha*[local_j] + beta*[sink_j]
// (cross-attention reuse page, 6.4) and an online softmax.
//
// This file holds the VALU kernel used for float32 storage: one wave per
// (row, head); each 64-key step scores one key per lane, then accumulates
// P*V with every lane owning d/64 output columns.
#include "common.h"
#include "kvr_internal.h"

namespace kvr {

namespace {

template <typename T>
__global__ __launch_bounds__(64) void k_attn_rowwise(const T* __restrict__ q,
                                                     const T* __restrict__ kc,
                                                     const T* __restrict__ vc,
                                                     const uint8_t* __restrict__ flags,
                                                     const int32_t* __restrict__ Tpos, Shape sh,
                                                     float alpha, float beta, T* __restrict__ o) {
  __shared__ float qs[128];
  __shared__ float ps[64];
  const int r = blockIdx.x / sh.hq, h = blockIdx.x - r * sh.hq;
  const int g = h / sh.group;
  const int u = Tpos[r];
  const int d = sh.d, lane = threadIdx.x;
  const int per = d >> 6;  // 1 or 2 output columns per lane
  const T* qr = q + (static_cast<size_t>(r) * sh.hq + h) * d;
  for (int c = lane; c < d; c += 64) qs[c] = Elem<T>::load(qr, c);
  __syncthreads();
  const float scale = rsqrtf(static_cast<float>(d));
  const size_t kv_stride = static_cast<size_t>(sh.hkv) * d;
  float m = -INFINITY, l = 0.f, acc[2] = {0.f, 0.f};
  for (int j0 = 0; j0 <= u; j0 += 64) {
    const int j = j0 + lane;
    float s = -INFINITY;
    if (j <= u) {
      const T* kr = kc + j * kv_stride + static_cast<size_t>(g) * d;
      float dot = 0.f;
      for (int c = 0; c < d; ++c) dot = fmaf(qs[c], Elem<T>::load(kr, c), dot);
      const uint8_t f = flags[j];
      s = dot * scale + ((f & KVR_FLAG_LOCAL) ? alpha : 0.f) + ((f & KVR_FLAG_SINK) ? beta : 0.f);
    }
    const float mn = fmaxf(m, wave_max(s));
    const float p = (j <= u) ? expf(s - mn) : 0.f;
    const float corr = expf(m - mn);
    l = l * corr + wave_sum(p);
    ps[lane] = p;
    __syncthreads();
    acc[0] *= corr;
    acc[1] *= corr;
    const int nk = min(64, u + 1 - j0);
    for (int jj = 0; jj < nk; ++jj) {
      const float pj = ps[jj];
      const T* vr = vc + (j0 + jj) * kv_stride + static_cast<size_t>(g) * d;
      for (int c = 0; c < per; ++c) acc[c] = fmaf(pj, Elem<T>::load(vr, lane * per + c), acc[c]);
    }
    m = mn;
    __syncthreads();
  }
  T* orow = o + (static_cast<size_t>(r) * sh.hq + h) * d;
  const float inv = 1.f / l;
  for (int c = 0; c < per; ++c) Elem<T>::store(orow, lane * per + c, acc[c] * inv);
}

}  // namespace

size_t attention_workspace_bytes(kvr_dtype, int, int, const Shape&) { return 0; }

hipError_t launch_attention(kvr_dtype dt, const void* q, const void* k_cache,
                            const void* v_cache, const uint8_t* flags, const int32_t* T, int B,
                            int n_tokens, const Shape& sh, float alpha, float beta,
                            const int32_t* plan_n_full, const int32_t* plan_n_total, void* ws,
                            void* o_out, hipStream_t stream) {
  (void)n_tokens; (void)plan_n_full; (void)plan_n_total; (void)ws;
  if (B == 0) return hipSuccess;
  dim3 grid(B * sh.hq);
  if (dt == KVR_BF16)
    hipLaunchKernelGGL(k_attn_rowwise<bf16_t>, grid, dim3(64), 0, stream,
                       static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k_cache),
                       static_cast<const bf16_t*>(v_cache), flags, T, sh, alpha, beta,
                       static_cast<bf16_t*>(o_out));
  else
    hipLaunchKernelGGL(k_attn_rowwise<float>, grid, dim3(64), 0, stream,
                       static_cast<const float*>(q), static_cast<const float*>(k_cache),
                       static_cast<const float*>(v_cache), flags, T, sh, alpha, beta,
                       static_cast<float*>(o_out));
  return hipGetLastError();
}

bool attention_needs_merge(kvr_dtype) { return false; }

hipError_t launch_attention_merge(kvr_dtype, int, const Shape&, const int32_t*, void*, void*,
                                  hipStream_t) {
  return hipSuccess;
}

}  // namespace kvr
