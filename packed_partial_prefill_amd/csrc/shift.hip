// Shift: positional correction of the retained suffix after a span is
// deleted ("Budgeted KV-Cache Repair", section 7.1, Eq. 2).  The suffix key
// at old position i moves to i - d and is re-rotated by R_{i-d} R_i^{-1}.
// For rotate-half RoPE that product is the same plane rotation for every i:
// pair (j, j + D/2) turns by the angle -d * theta^(-2j/D).  Values move
// unchanged, rows before the span are copied, metadata moves with its row.
//
// A pure stream over the cache: every byte of the retained rows is read
// once and written once.  One thread owns one 16-byte chunk of the lower
// half of a (row, head) key and the matching chunk of the upper half (the
// two halves of each rotated pair), plus the value chunks at the same
// offsets.  Launches cover up to kMaxLayers layers (grid.y = layer).
#include <cmath>

#include "common.h"
#include "kvr_internal.h"

namespace kvr {

namespace {

constexpr int kThreads = 256;

template <typename T> struct Vec;
template <> struct Vec<bf16_t> { static constexpr int n = 8; };
template <> struct Vec<float> { static constexpr int n = 4; };

__device__ __forceinline__ float to_f(bf16_t x) { return bf16_to_f32(x); }
__device__ __forceinline__ float to_f(float x) { return x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float x) { return f32_to_bf16(x); }
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }

template <typename T>
__global__ __launch_bounds__(kThreads) void k_shift(ShiftLayers L, int n_out, int hkv, int d,
                                                    int del_start, int del_len, double theta) {
  constexpr int VEC = Vec<T>::n;
  __shared__ float2 rot[64];                      // (cos, sin) per pair, d/2 <= 64
  const int half = d >> 1;
  if (threadIdx.x < half) {
    // angle of pair j: -del_len * theta^(-2j/d), evaluated in float64
    const double ang = -static_cast<double>(del_len) *
                       pow(theta, -2.0 * static_cast<double>(threadIdx.x) / static_cast<double>(d));
    double s, c;
    sincos(ang, &s, &c);
    rot[threadIdx.x] = make_float2(static_cast<float>(c), static_cast<float>(s));
  }
  __syncthreads();

  const int per_head = half / VEC;                // pair-chunks per (row, head)
  const size_t work = static_cast<size_t>(n_out) * hkv * per_head;
  const size_t t = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (t >= work) return;
  const int layer = blockIdx.y;
  const size_t rh = t / per_head;                 // (row, head) of the destination
  const int c = static_cast<int>(t - rh * per_head);
  const size_t row = rh / hkv;
  const int head = static_cast<int>(rh - row * hkv);
  const size_t src_row = row < static_cast<size_t>(del_start) ? row : row + del_len;
  const size_t so = (src_row * hkv + head) * d + c * VEC;
  const size_t dof = (row * hkv + head) * d + c * VEC;
  const T* ks = static_cast<const T*>(L.src_k[layer]);
  const T* vs = static_cast<const T*>(L.src_v[layer]);
  T* kd = static_cast<T*>(L.dst_k[layer]);
  T* vd = static_cast<T*>(L.dst_v[layer]);

  const uint4 v_lo = *reinterpret_cast<const uint4*>(vs + so);
  const uint4 v_hi = *reinterpret_cast<const uint4*>(vs + so + half);
  const uint4 k_lo = *reinterpret_cast<const uint4*>(ks + so);
  const uint4 k_hi = *reinterpret_cast<const uint4*>(ks + so + half);
  *reinterpret_cast<uint4*>(vd + dof) = v_lo;
  *reinterpret_cast<uint4*>(vd + dof + half) = v_hi;
  if (row < static_cast<size_t>(del_start)) {     // prefix: copied bit for bit
    *reinterpret_cast<uint4*>(kd + dof) = k_lo;
    *reinterpret_cast<uint4*>(kd + dof + half) = k_hi;
    return;
  }
  const T* a = reinterpret_cast<const T*>(&k_lo);
  const T* b = reinterpret_cast<const T*>(&k_hi);
  uint4 o_lo, o_hi;
  T* x = reinterpret_cast<T*>(&o_lo);
  T* y = reinterpret_cast<T*>(&o_hi);
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    const float2 cs = rot[c * VEC + e];
    const float av = to_f(a[e]), bv = to_f(b[e]);
    x[e] = from_f<T>(av * cs.x - bv * cs.y);
    y[e] = from_f<T>(bv * cs.x + av * cs.y);
  }
  *reinterpret_cast<uint4*>(kd + dof) = o_lo;
  *reinterpret_cast<uint4*>(kd + dof + half) = o_hi;
}

// Metadata: flags (and block ids) move with their rows; `mark` is OR-ed into
// the moved suffix rows.
__global__ __launch_bounds__(kThreads) void k_shift_meta(const uint8_t* __restrict__ f_src,
                                                         uint8_t* __restrict__ f_dst,
                                                         const int32_t* __restrict__ b_src,
                                                         int32_t* __restrict__ b_dst, int n_out,
                                                         int del_start, int del_len,
                                                         uint8_t mark) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= n_out) return;
  const bool moved = i >= del_start;
  const int s = moved ? i + del_len : i;
  if (f_dst) f_dst[i] = static_cast<uint8_t>(f_src[s] | (moved ? mark : 0));
  if (b_dst) b_dst[i] = b_src[s];
}

}  // namespace

hipError_t launch_shift(kvr_dtype dt, const ShiftLayers& L, int n_layers, int n_out,
                        const Shape& sh, int del_start, int del_len, double theta,
                        hipStream_t stream) {
  if (n_out == 0 || n_layers == 0) return hipSuccess;
  const int vec = dt == KVR_BF16 ? 8 : 4;
  const size_t work = static_cast<size_t>(n_out) * sh.hkv * (sh.d / 2 / vec);
  const dim3 grid(static_cast<unsigned>((work + kThreads - 1) / kThreads), n_layers);
  if (dt == KVR_BF16)
    hipLaunchKernelGGL(k_shift<bf16_t>, grid, dim3(kThreads), 0, stream, L, n_out, sh.hkv, sh.d,
                       del_start, del_len, theta);
  else
    hipLaunchKernelGGL(k_shift<float>, grid, dim3(kThreads), 0, stream, L, n_out, sh.hkv, sh.d,
                       del_start, del_len, theta);
  return hipGetLastError();
}

hipError_t launch_shift_meta(const uint8_t* f_src, uint8_t* f_dst, const int32_t* b_src,
                             int32_t* b_dst, int n_out, int del_start, int del_len, uint8_t mark,
                             hipStream_t stream) {
  if (n_out == 0 || (!f_dst && !b_dst)) return hipSuccess;
  hipLaunchKernelGGL(k_shift_meta, dim3((n_out + kThreads - 1) / kThreads), dim3(kThreads), 0,
                     stream, f_src, f_dst, b_src, b_dst, n_out, del_start, del_len, mark);
  return hipGetLastError();
}

}  // namespace kvr
