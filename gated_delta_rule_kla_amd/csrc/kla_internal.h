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

// Upstream gradients in and gradients out of the backward pass (device pointers).
struct ChunkBwdArgs {
  const void *dout;             // dL/do, [B,H,T,dv], dtype
  const float *dfinal_state;    // dL/dS_final, [N,H,dk,dv] fp32, or nullptr (zero)
  void *dq, *dk, *dv;           // dtype, shaped as q, k, v
  float *dg, *deta;             // fp32 [B,H,T]
  float *dinitial_state;        // fp32 [N,H,dk,dv], or nullptr (not written)
};

// PGDN (the preconditioned variant) and its parameters, for the general chunk kernel.
struct GenExtra {
  int pgdn;                  // 1: write keys w_t = p_t (.) k_t (PGDN); 0: w = k
  float band_c;              // ln(band) of the preconditioner's squash (0: p = 1)
  const float *initial_acc;  // [N, H, dk] fp32 accumulator at the start, or nullptr (zeros)
  float *final_acc;          // [N, H, dk] fp32, or nullptr
};

// True if a kernel is compiled for this combination.  chunk_supported covers
// both the pipelined kernels (fast_chunk_supported) and the general kernel.
bool decode_supported(int dtype, int dk, int dv);
bool chunk_supported(int dtype, int dk, int dv, int chunk);
bool fast_chunk_supported(int dtype, int dk, int dv, int chunk);
bool general_supported(int dtype, int dk, int dv, int chunk);
bool pgdn_decode_supported(int dtype, int dk, int dv);

// Bytes of device workspace kla_chunk_fwd needs for these arguments (the
// per-chunk T' and decay vectors handed from the prep kernel to the scan
// kernel).  Arguments are already validated and supported.
size_t chunk_workspace_bytes(const ChunkArgs &a);

// The backward pass supports the forward's shapes; its workspace holds per
// (chunk, head) T, P and vectors plus the chunk-start states and chunk-end
// state gradients (fp32).
bool chunk_bwd_supported(int dtype, int dk, int dv, int chunk);
size_t chunk_bwd_workspace_bytes(const ChunkArgs &a);

// The fixed per-GPU scratch behind kla_chunk_fwd_noalloc: its size, and its
// device address on the current device (looked up on the first call per
// device; no allocation).
size_t static_scratch_bytes();
hipError_t static_scratch(void **ptr);

// Enqueue the kernel(s).  Arguments are already validated.
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_chunk_fwd(const ChunkArgs &a, hipStream_t stream);
hipError_t launch_chunk_bwd(const ChunkArgs &a, const ChunkBwdArgs &b, hipStream_t stream);
// PGDN on the pipelined prep + scan kernels (bf16, chunk 64, dk 64 or 128): its
// device workspace (0 outside those shapes) and launch.  The workspace holds the
// forward's (T'^T images, order), the chunk-start key accumulators and the write keys.
bool pgdn_fast_supported(int dtype, int dk, int dv, int chunk);
size_t pgdn_workspace_bytes(const ChunkArgs &a);
hipError_t launch_pgdn_fast(const ChunkArgs &a, const GenExtra &x, hipStream_t stream);
hipError_t launch_chunk_general(const ChunkArgs &a, const GenExtra &x, hipStream_t stream);
// The forward's prep and scan kernels in states mode: the state at the start of
// every chunk into `states` (the layout of ChunkParams::states in
// kla_chunk.hip; dk * dv elements of the element type per (head, slot)), no
// outputs.  a.workspace is the forward workspace (chunk_workspace_bytes(a)).
// timg (bf16 only, or nullptr): also the packed image of T^T per (head, slot),
// TpLayout<bf16, 64>::PACK bytes each (ChunkParams::timg).  four (bf16, dv % 64 == 0):
// 64-column scan slices; after_prep (bf16, or nullptr): recorded on the stream once the
// prep kernel (and the packed-sequence order) is enqueued, before the scan.
hipError_t launch_chunk_states(const ChunkArgs &a, void *states, hipStream_t stream, void *timg = nullptr,
                               bool four = false, hipEvent_t after_prep = nullptr);
// The reverse scan of the state gradients on the same machinery, after
// launch_chunk_states on the same workspace: dS' of every chunk into dstates
// (the same layout as states), dL/dS_final from dsfin (or zeros), the
// initial-state gradient into ds0 (or not written).
hipError_t launch_chunk_rev(const ChunkArgs &a, const float *dsfin, const void *dout, float *ds0, void *dstates,
                            hipStream_t stream, bool four = false);
// The segment-parallel forward (kla_chunk.hip, kla_seg.hip): each sequence cut into
// segments of L chunks, scanned side by side, then combined and corrected.
// chunk_seg_supported: the shapes it runs (the pipelined kernels').  chunk_seg_count:
// segments for L (cu_host: the host mirror, for packed sequences).  The workspace
// holds kla_chunk_fwd's, then the segment table, the identity tiles' outputs E
// ([B, H, T, dk], element type), the segments' end states and transfer maps and the
// corrections' start states.  chunk_auto_seg_chunks: the library's choice of L for
// kla_chunk_fwd (0: no segments), host-only.
bool chunk_seg_supported(int dtype, int dk, int dv, int chunk);
long long chunk_seg_count(const ChunkArgs &a, const int32_t *cu_host, int L);
size_t chunk_seg_workspace_bytes(const ChunkArgs &a, const int32_t *cu_host, int L);
int chunk_auto_seg_chunks(const ChunkArgs &a, const int32_t *cu_host);
hipError_t launch_chunk_fwd_seg(const ChunkArgs &a, const int32_t *cu_host, int L, hipStream_t stream);

// What the combine and correction kernels of the segmented forward read and write.
struct SegFixParams {
  const int32_t *cu;     // device cu_seqlens or nullptr (dense)
  const int *seg_first;  // [nseq + 1] first segment of each sequence
  int nseq, H, T, C, dk, dv, dtype, seg_chunks;
  int seg_max_chunks;  // chunks of the longest sequence (bounds the correction's runs)
  long long nseg;
  const float *seg_d;  // [nseg, H, dk, dv] end states (first segments: from the initial state)
  const float *seg_m;  // [nseg, H, dk, dk] transfer maps (later segments)
  float *sfin;         // [nseq, H, dk, dv] final states, or nullptr
  void *sfix;          // the later segments' start states (bf16 MFMA groups or fp32 rows)
  const void *eout;    // [B, H, T, dk] the identity tiles' outputs
  void *o;             // [B, H, T, dv] outputs, corrected in place
};
hipError_t launch_seg_table(const SegFixParams &f, int *seg_first, hipStream_t stream);
hipError_t launch_seg_finish(const SegFixParams &f, hipStream_t stream);
bool seg_correct_mfma(int dtype, int dk, int dv);

// True when the backward's two state passes run side by side (64-column slices, both
// within one round of workgroups on `cus` CUs): see kla_chunk.hip.
bool bwd_scans_concurrent(const ChunkArgs &a, int cus);
// a.eta holds the coefficient (beta when a.beta_direct, else eta); acc [N, H, dk] in place
// PGDN's decode step on kla_decode_kernel (the shapes decode_supported lists)
hipError_t launch_decode_pgdn(const DecodeArgs &a, float band_c, float *acc, hipStream_t stream);
hipError_t launch_pgdn_decode(const DecodeArgs &a, float band_c, float *acc, hipStream_t stream);

}  // namespace kla
