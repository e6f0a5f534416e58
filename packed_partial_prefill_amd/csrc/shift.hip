// Shift: positional correction of the retained suffix after a span is
// deleted ("Budgeted KV-Cache Repair", section 7.1, Eq. 2).  The suffix key
// at old position i moves to i - d and is re-rotated by R_{i-d} R_i^{-1}.
// For rotate-half RoPE that product is the same plane rotation for every i:
// pair (j, j + D/2) turns by the angle -d * theta^(-2j/D).  Values move
// unchanged, rows before the span are copied, metadata moves with its row.
//
// A pure stream over the cache: every byte of the retained rows is read
// once and written once, with nontemporal accesses (nothing is re-read).
// One thread owns one 16-byte chunk of the lower half of a (row, head) key
// and the matching chunk of the upper half (the two halves of each rotated
// pair); value rows are copied by other threads, one 16-byte chunk each.  Launches cover up to
// kShiftMaxLayers layers (grid.y = layer).  The (cos, sin) of the d/2 angles
// are evaluated once per call on the host in float64 and arrive as a kernel
// argument (each workgroup evaluating them in float64 delayed its loads).
#include <cmath>

#include "common.h"
#include "kvr_internal.h"

namespace kvr {

namespace {

constexpr int kThreads = 256;

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));   // nontemporal access type

// (cos, sin) of the rotation of pair j, j < d/2
struct ShiftRot {
  float2 cs[64];
};

template <typename T> struct Vec;
template <> struct Vec<bf16_t> { static constexpr int n = 8; };
template <> struct Vec<float> { static constexpr int n = 4; };

__device__ __forceinline__ float to_f(bf16_t x) { return bf16_to_f32(x); }
__device__ __forceinline__ float to_f(float x) { return x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float x) { return f32_to_bf16(x); }
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }

template <typename T>
__global__ __launch_bounds__(kThreads) void k_shift(ShiftLayers L, ShiftRot rot, int n_out, int hkv,
                                                    int d, int del_start, int del_len) {
  constexpr int VEC = Vec<T>::n;
  const int half = d >> 1;
  const int per_head = half / VEC;                // pair-chunks per (row, head)
  const size_t work = static_cast<size_t>(n_out) * hkv * per_head;
  // threads [0, work) move and rotate keys (a lower-half chunk and its upper
  // partner each); threads [work, 3 work) copy values, one 16-byte chunk each
  // in row order
  size_t t = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (t >= 3 * work) return;
  const int layer = blockIdx.y;
  auto ld = [](const T* p) { return __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p)); };
  auto st = [](T* p, u32x4v v) { __builtin_nontemporal_store(v, reinterpret_cast<u32x4v*>(p)); };
  if (t >= work) {
    t -= work;
    const size_t row_chunks = static_cast<size_t>(hkv) * d / VEC;
    const size_t row = t / row_chunks;
    const size_t src_row = row < static_cast<size_t>(del_start) ? row : row + del_len;
    const size_t off = (t - row * row_chunks) * VEC;
    st(static_cast<T*>(L.dst_v[layer]) + row * row_chunks * VEC + off,
       ld(static_cast<const T*>(L.src_v[layer]) + src_row * row_chunks * VEC + off));
    return;
  }
  const size_t rh = t / per_head;                 // (row, head) of the destination
  const int c = static_cast<int>(t - rh * per_head);
  const size_t row = rh / hkv;
  const int head = static_cast<int>(rh - row * hkv);
  const size_t src_row = row < static_cast<size_t>(del_start) ? row : row + del_len;
  const size_t so = (src_row * hkv + head) * d + c * VEC;
  const size_t dof = (row * hkv + head) * d + c * VEC;
  const T* src = static_cast<const T*>(L.src_k[layer]);
  T* dst = static_cast<T*>(L.dst_k[layer]);

  const u32x4v lo = ld(src + so), hi = ld(src + so + half);
  if (row < static_cast<size_t>(del_start)) {     // prefix: copied bit for bit
    st(dst + dof, lo);
    st(dst + dof + half, hi);
    return;
  }
  const T* a = reinterpret_cast<const T*>(&lo);
  const T* b = reinterpret_cast<const T*>(&hi);
  u32x4v o_lo, o_hi;
  T* x = reinterpret_cast<T*>(&o_lo);
  T* y = reinterpret_cast<T*>(&o_hi);
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    const float2 cs = rot.cs[c * VEC + e];
    const float av = to_f(a[e]), bv = to_f(b[e]);
    x[e] = from_f<T>(av * cs.x - bv * cs.y);
    y[e] = from_f<T>(bv * cs.x + av * cs.y);
  }
  st(dst + dof, o_lo);
  st(dst + dof + half, o_hi);
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
  const dim3 grid(static_cast<unsigned>((3 * work + kThreads - 1) / kThreads), n_layers);
  // pair j turns by -del_len * theta^(-2j/d), in float64
  ShiftRot rot{};
  for (int j = 0; j < sh.d / 2 && j < 64; ++j) {
    const double ang = -static_cast<double>(del_len) *
                       std::pow(theta, -2.0 * static_cast<double>(j) / static_cast<double>(sh.d));
    rot.cs[j] = make_float2(static_cast<float>(std::cos(ang)), static_cast<float>(std::sin(ang)));
  }
  if (dt == KVR_BF16)
    hipLaunchKernelGGL(k_shift<bf16_t>, grid, dim3(kThreads), 0, stream, L, rot, n_out, sh.hkv,
                       sh.d, del_start, del_len);
  else
    hipLaunchKernelGGL(k_shift<float>, grid, dim3(kThreads), 0, stream, L, rot, n_out, sh.hkv,
                       sh.d, del_start, del_len);
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
