// kla_common.h -- device helpers shared by the KLA kernels (gfx950 / CDNA4).
//
// Element types: the production path stores q/k/v/g/eta/o as bfloat16 and
// computes in fp32; the debug path stores them as fp32.  `Elem<E>` converts
// between the storage type and fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kla {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename E> struct Elem;

template <> struct Elem<bf16> {
  static __device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
  static __device__ __forceinline__ bf16 from_f32(float x) { return (bf16)x; }  // RNE
};

template <> struct Elem<float> {
  static __device__ __forceinline__ float to_f32(float x) { return x; }
  static __device__ __forceinline__ float from_f32(float x) { return x; }
};

// 16-byte global load/store (caller guarantees 16-byte alignment).
__device__ __forceinline__ uint4 ldg16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void stg16(void *p, uint4 v) { *reinterpret_cast<uint4 *>(p) = v; }

// PGDN's preconditioner weight of one key coordinate ("Preconditioned DeltaNet",
// §2.C: the inverse of the accumulated diagonal key moments, squashed in log space
// into [1/band, band]): with the coordinate's accumulator a, the mean accumulator m
// over the coordinates and c = ln(band),
//   p = exp(c tanh(r / c)),  r = ln((m + delta) / (a + delta)),  delta = 1e-30,
// tanh from one exponential, 1 - 2 / (exp(2x) + 1), exact at both saturations.  In
// base 2 (the hardware's exp2 and log2): exp(2 r / c) = 2^(k1 (log2(m + delta) -
// log2(a + delta))) with k1 = 2 / c, and p = 2^(k2 tanh) with k2 = c log2(e); c = 0
// (band 1) gives k1 = k2 = 0 and p = 1.
struct PgdnK {
  float k1, k2;
};
__host__ __device__ inline PgdnK pgdn_k(float c) { return {c == 0.f ? 0.f : 2.f / c, c * 1.4426950408889634f}; }
// log2(m + delta) of a mean accumulator, the form pgdn_precond takes
__device__ __forceinline__ float pgdn_log2_mean(float m) { return __builtin_amdgcn_logf(m + 1e-30f); }
__device__ __forceinline__ float pgdn_precond(float a, float log2_m, PgdnK k) {
  const float e = __builtin_amdgcn_exp2f(k.k1 * (log2_m - __builtin_amdgcn_logf(a + 1e-30f)));
  const float th = 1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f);
  return __builtin_amdgcn_exp2f(k.k2 * th);
}

}  // namespace kla
