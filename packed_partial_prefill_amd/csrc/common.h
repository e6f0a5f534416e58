// Device helpers shared by the libkvr kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvr {

typedef uint16_t bf16_t;  // bfloat16 bit pattern

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even float32 -> bfloat16 (NaN stays NaN): the language
// conversion, which gfx950 performs with v_cvt_pk_bf16_f32 (no branches).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// Storage traits: float32 or bfloat16 elements, float32 arithmetic.
template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p, size_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  __device__ __forceinline__ static void store(bf16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

// Workgroups are dispatched to the 8 XCDs round-robin by linear id, and each
// XCD has its own L2.  xcd_linear(b, total) maps linear block b to a logical
// index so that XCD b % 8 takes one contiguous run of the logical order
// (a bijection on [0, total)): workgroups that share operands, placed next
// to each other in the logical order, then share one L2.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_linear(int b, int total) {
  const int xcd = b % kXcds, q = total / kXcds, rem = total % kXcds;
  return xcd * q + min(xcd, rem) + b / kXcds;
}

// Combine x with the value of lane ^ 32: v_permlane32_swap exchanges the
// wave's two 32-lane halves in one VALU instruction, leaving each lane its
// own value and its partner's (in either order), where __shfl_xor would take
// an LDS round trip.
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_add(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Sum over a workgroup of up to 1024 threads (multiple of 64).  `red` must
// hold 16 floats of shared memory.  Every thread receives the total.
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

}  // namespace kvr
