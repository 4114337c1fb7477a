// Device-side helpers shared by the retention kernels (gfx950 only). The
// host-visible argument structures they use are declared in kernels.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace ret {

// swish(g) = g * sigmoid(g) = g / (1 + e^-g), the gate's activation: e^-g as
// the hardware exp2 of -g * log2(e), then the hardware reciprocal (about one
// ulp each). For g below about -88, e^-g is +inf, its reciprocal 0 and the
// result -0, the limit; for large g the result is g.
__device__ __forceinline__ float swish(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Round-to-nearest-even conversion (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two values rounded to bf16 in one register, `lo` in the low half (one
// two-source v_cvt_pk_bf16_f32).
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const floatx2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// gamma^e for a (possibly fractional) exponent e >= 0.
__device__ __forceinline__ float decay_pow(float log2g, float e) {
  return exp2f(e * log2g);
}

// Element access for the two supported input types: float and raw bf16 bits.
template <typename T>
struct Elem;

template <>
struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, int64_t i, float x) { p[i] = x; }
};

template <>
struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(uint16_t* p, int64_t i, float x) { p[i] = f32_to_bf16(x); }
};

// Sum over the 64 lanes of a wavefront (every lane receives the total).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

}  // namespace ret

namespace ret {

// Sum over a 256-thread block. `scratch` holds at least 4 floats of LDS.
// Every thread receives the total. Contains barriers: call from all threads.
__device__ __forceinline__ float block_sum_256(float x, float* scratch) {
  x = wave_sum(x);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[wave] = x;
  __syncthreads();
  return scratch[0] + scratch[1] + scratch[2] + scratch[3];
}

}  // namespace ret
