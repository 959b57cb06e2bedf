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
// into [1/band, band]): with the coordinate's accumulator a, log_m = ln(m + delta) of
// the mean accumulator over the coordinates and c = ln(band),
//   p = exp(c tanh(r / c)),  r = ln((m + delta) / (a + delta)),  delta = 1e-30,
// tanh from one exponential, 1 - 2 / (exp(2x) + 1), exact at both saturations;
// c = 0 (band 1) gives p = 1.
__device__ __forceinline__ float pgdn_precond_l(float a, float log_m, float c) {
  if (c == 0.f) return 1.f;
  const float r = log_m - __logf(a + 1e-30f);
  const float th = 1.f - 2.f * __builtin_amdgcn_rcpf(__expf(2.f * r / c) + 1.f);
  return __expf(c * th);
}

}  // namespace kla
