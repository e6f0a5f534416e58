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

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

// LDS reads issued as inline assembly, for loops that keep LDS DMA in flight
// into other buffers: the compiler cannot tell such reads from the DMA and
// places a wait for all outstanding DMA (or for all LDS operations) in front
// of its own forms.  The caller waits with lds_wait / lds_wait_n and then
// passes each result through reg_fence.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)(p)));
}
__device__ __forceinline__ void lds_wait() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt not waited for
}
template <int N> __device__ __forceinline__ void lds_wait_n() {
  static_assert(N >= 0 && N < 16, "lgkmcnt");
  __builtin_amdgcn_s_waitcnt(0xC07F | (N << 8));   // at most N LDS operations outstanding
}
// An assembly LDS read's result is valid only after the lgkmcnt wait; the
// compiler must order reg_fence after the wait (both are volatile) and every
// use of the value then depends on it.
template <typename T> __device__ __forceinline__ void reg_fence(T& r) { asm volatile("" : "+v"(r)); }
// ds_read_b128 at LDS byte address addr + OFF
template <int OFF = 0>
__device__ __forceinline__ u32x4_t ds_read_b128(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x4_t r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
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
