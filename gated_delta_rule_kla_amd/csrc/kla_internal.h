// kla_internal.h -- launchers behind the C ABI (not part of the public header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kla {

struct DecodeArgs {
  const void *q, *k, *v, *g, *eta;
  float eps;
  float *state;
  void *o;
  int N, H, dk, dv;
  int dtype;        // kla_dtype_t
  int beta_direct;  // 1: `eta` holds beta itself (gated delta rule); eps unused
};

struct ChunkArgs {
  const void *q, *k, *v, *g, *eta;
  float eps;
  const float *initial_state;
  void *o;
  float *final_state;
  const int32_t *cu_seqlens;  // device, or nullptr
  int num_seqs, B, H, T, dk, dv, chunk;
  int dtype;        // kla_dtype_t
  void *workspace;  // device, chunk_workspace_bytes(*this) bytes
  int beta_direct;  // 1: `eta` holds beta itself (gated delta rule); eps unused
};

// True if a kernel is compiled for this combination.
bool decode_supported(int dtype, int dk, int dv);
bool chunk_supported(int dtype, int dk, int dv, int chunk);

// Bytes of device workspace kla_chunk_fwd needs for these arguments (the
// per-chunk T' and decay vectors handed from the prep kernel to the scan
// kernel).  Arguments are already validated and supported.
size_t chunk_workspace_bytes(const ChunkArgs &a);

// Enqueue the kernel(s).  Arguments are already validated.
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_chunk_fwd(const ChunkArgs &a, hipStream_t stream);

}  // namespace kla
