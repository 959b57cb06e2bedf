// kla_seg.hip -- the segment-parallel prefill's bookkeeping kernels for gfx950.
//
// A long sequence is a long chain of dependent chunk steps.  The state update of a
// chunk is affine in the state ("Resumen Técnico: Atención Lineal Kaczmarz (KLA)",
// §"Implementación": the chunkwise block solver; with U~ = T'(V - Diag(Gam) K S)):
//
//   S' = M_c S + D_c,   M_c = Gam_C I - K^T Diag(d) T' Diag(Gam) K,   D_c = K^T Diag(d) T' V
//   O  = Diag(Gam) Q S + P U~ = O|_{S=0} + E_c S,   E_c = Diag(Gam) Q - P T' Diag(Gam) K,
//
// so a sequence cut into segments can be scanned segment by segment at the same
// time: each later segment from a zero state (outputs O_loc, end state D), and with
// the identity as the state of dk extra columns and v = 0 (their outputs are
// E = E_c Phi_c with Phi_c the product of the segment's M_c up to chunk c, their end
// state the segment's transfer map M).  The scan kernel does both (kla_chunk.hip,
// ChunkParams::seg_first).  The kernels here finish the job:
//
//   kla_seg_table_kernel    each sequence's first segment (prefix sums)
//   kla_seg_combine_kernel  per (sequence, head, 16 state columns), in segment order:
//                           S = D of the first segment (scanned from the true initial
//                           state); for each later segment s: S is its true start
//                           state (kept for the correction), S <- M_s S + D_s; the
//                           last S is the final state.  fp32 throughout.
//   kla_seg_correct_*       O += E S_start over every later segment's tokens.
//
// This is the context-parallel decomposition of a recurrence into per-segment affine
// maps, applied inside one GPU; it changes the order of the arithmetic only.
#include "kla_common.h"
#include "kla_internal.h"
#include "kla_ops.h"

#include <algorithm>

namespace kla {

// Sequence n of a call: tokens [t0, t1) of batch row b.
__device__ __forceinline__ void seg_seq_range(const int32_t *cu, int n, int T, int &b, int &t0, int &t1) {
  if (cu) {
    b = 0;
    t0 = min(max(cu[n], 0), T);
    t1 = min(max(cu[n + 1], t0), T);
  } else {
    b = n;
    t0 = 0;
    t1 = T;
  }
}

__device__ __forceinline__ int seg_of_seq(const int *seg_first, int nseq, int s) {
  int lo = 0, hi = nseq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seg_first[mid] <= s) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// seg_first[n] = sum over n' < n of max(1, ceil(chunks(n') / L)) for n = 0 .. nseq,
// each value capped at `cap` (the host's count from the cu_seqlens mirror, so that a
// device array that disagrees cannot make the grids read past their ends).  One
// workgroup: each thread sums a run of sequences, then a scan over the threads.
__global__ __launch_bounds__(1024) void kla_seg_table_kernel(const int32_t *cu, int nseq, int T, int C, int L,
                                                             int cap, int *seg_first) {
  __shared__ int part[1024];
  const int t = threadIdx.x;
  const int per = (nseq + 1023) / 1024;
  const int n0 = min(t * per, nseq), n1 = min(n0 + per, nseq);
  auto count = [&](int n) {
    int b, t0, t1;
    seg_seq_range(cu, n, T, b, t0, t1);
    const int nch = (t1 - t0 + C - 1) / C;
    return max(1, (nch + L - 1) / L);
  };
  int sum = 0;
  for (int n = n0; n < n1; ++n) sum += count(n);
  part[t] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = part[t] - sum;
  for (int n = n0; n < n1; ++n) {
    seg_first[n] = min(run, cap);
    run += count(n);
  }
  if (t == 1023) seg_first[nseq] = min(part[1023], cap);
}

// ---- combine -----------------------------------------------------------------------
// One workgroup of min(1024, 16 dk) threads per (sequence, head, 16 state columns).
// Thread t owns column t & 15 and rows (t >> 4) + (NT / 16) j of that slice.  The current S and the
// segment's M are staged in LDS (M rows padded by four floats: the 16-byte stores
// stay aligned and the rows a wave reads fall on distinct banks).
//   GRP: the start states go to the correction as bf16 MFMA groups -- group (column
//   tile, q) of segment s, head h at ((s H + h) dv/16 + tile) dk/32 + q, 64 lanes x
//   16 bytes, lane (i, g) holding S[32 q + 8 g + x][16 tile + i], x < 8; otherwise as
//   fp32 rows, [nseg, H, dk, dv].
template <int DK>
constexpr int combine_threads() { return 16 * DK < 1024 ? 16 * DK : 1024; }

template <int DK, bool GRP>
__global__ __launch_bounds__(combine_threads<DK>()) void kla_seg_combine_kernel(SegFixParams f) {
  constexpr int NT = combine_threads<DK>(), RS = NT / 16, RPT = DK / RS, LDM = DK + 4;
  __shared__ float sS[DK][16];
  __shared__ __attribute__((aligned(16))) float sM[DK * LDM];
  const int t = threadIdx.x;
  const int n = blockIdx.x / f.H, h = blockIdx.x % f.H, ct = blockIdx.y;
  const int s0 = f.seg_first[n], s1 = f.seg_first[n + 1];
  if (s1 <= s0) return;  // (only with a cu_seqlens that disagrees with its mirror)
  const int dv = f.dv, c = t & 15, r0 = t >> 4;
  const size_t col = (size_t)16 * ct + c;
  float S[RPT];
  {
    const float *D = f.seg_d + ((size_t)s0 * f.H + h) * DK * dv + col;
#pragma unroll
    for (int j = 0; j < RPT; ++j) S[j] = D[(size_t)(r0 + RS * j) * dv];
  }
  for (int s = s0 + 1; s < s1; ++s) {
    __syncthreads();  // the previous segment's reads of sS and sM are done
#pragma unroll
    for (int j = 0; j < RPT; ++j) sS[r0 + RS * j][c] = S[j];
    const f32x4 *M = reinterpret_cast<const f32x4 *>(f.seg_m + ((size_t)s * f.H + h) * DK * DK);
#pragma unroll 4
    for (int e = t; e < DK * DK / 4; e += NT) {
      const int row = e / (DK / 4), c4 = e % (DK / 4);
      *reinterpret_cast<f32x4 *>(sM + row * LDM + 4 * c4) = M[e];
    }
    __syncthreads();
    // the true start state of segment s, for the correction of its outputs
    if constexpr (GRP) {
      if (t < 64 * (DK / 32)) {
        const int q = t >> 6, lane = t & 63, i = lane & 15, g = lane >> 4;
        bf16x8 v;
#pragma unroll
        for (int x = 0; x < 8; ++x) v[x] = (bf16)sS[32 * q + 8 * g + x][i];
        const size_t grp = (((size_t)s * f.H + h) * (dv / 16) + ct) * (DK / 32) + q;
        reinterpret_cast<bf16x8 *>(f.sfix)[grp * 64 + lane] = v;
      }
    } else {
      float *F = reinterpret_cast<float *>(f.sfix) + ((size_t)s * f.H + h) * DK * dv + col;
#pragma unroll
      for (int j = 0; j < RPT; ++j) F[(size_t)(r0 + RS * j) * dv] = S[j];
    }
    // S <- M_s S + D_s (four contraction rows at a time: one 16-byte read of each M row)
    const float *D = f.seg_d + ((size_t)s * f.H + h) * DK * dv + col;
#pragma unroll
    for (int j = 0; j < RPT; ++j) S[j] = D[(size_t)(r0 + RS * j) * dv];
#pragma unroll 2
    for (int k = 0; k < DK; k += 4) {
      const float s0 = sS[k][c], s1 = sS[k + 1][c], s2 = sS[k + 2][c], s3 = sS[k + 3][c];
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        const f32x4 m = *reinterpret_cast<const f32x4 *>(sM + (r0 + RS * j) * LDM + k);
        S[j] = fmaf(m[0], s0, S[j]);
        S[j] = fmaf(m[1], s1, S[j]);
        S[j] = fmaf(m[2], s2, S[j]);
        S[j] = fmaf(m[3], s3, S[j]);
      }
    }
  }
  if (f.sfin) {
    float *F = f.sfin + ((size_t)n * f.H + h) * DK * dv + col;
#pragma unroll
    for (int j = 0; j < RPT; ++j) F[(size_t)(r0 + RS * j) * dv] = S[j];
  }
}

// The token range of segment s (later segments only; returns false for a first
// segment or a segment past the table's end) and its batch row.
__device__ __forceinline__ bool seg_tokens(const SegFixParams &f, int s, int &b, int &st0, int &st1) {
  if (s >= f.seg_first[f.nseq]) return false;
  const int n = seg_of_seq(f.seg_first, f.nseq, s);
  const int g = s - f.seg_first[n];
  if (g == 0) return false;
  int t0, t1;
  seg_seq_range(f.cu, n, f.T, b, t0, t1);
  const long long lo = (long long)t0 + (long long)g * f.seg_chunks * f.C;
  st0 = (int)min((long long)t1, lo);
  st1 = (int)min((long long)t1, lo + (long long)f.seg_chunks * f.C);
  return st0 < st1;
}

// ---- correction, bf16 on MFMA --------------------------------------------------------
// One workgroup per (run of kSegRun chunks, later segment, head): grid x is the run, grid
// y the (segment, head) pair (pairs beyond gridDim.y taken in turn), dv / (16 NCTW) waves; wave w owns NCTW column tiles (16 columns each) of o.  Per chunk (64 tokens):
//   1. the chunk's E rows and o rows into LDS, in coalesced 16-byte pieces (consecutive
//      lanes, consecutive bytes of a row: the kernel moves 80 KB per chunk and head at
//      dv = 256 and is bound by HBM; pieces of a few bytes per row per instruction ran it
//      at a third of that);
//   2. per 16 tokens: O^T tile (16 columns x 16 tokens) += S_start^T (16 x dk) E^T
//      (dk x 16 tokens), S_start^T the left operand (the combine kernel's groups, held in
//      registers for the whole run), E rows from LDS the right operand (slot x of lane
//      group g <-> contraction index 32 q + 8 g + x on both sides), the o tile from LDS
//      the accumulator (lane (i, g): token i, columns 4 g .. 4 g + 3), written back there;
//   3. the o rows back to memory in 16-byte pieces.
constexpr int kSegRun = 2;  // chunks per correction workgroup (2: 150 us, 4: 155, 8: 171 on T=65536 dv=256)

template <int DK, int DV>
__global__ __launch_bounds__(64 * (DV == 64 ? 4 : DV / 32)) void kla_seg_correct_mfma_kernel(SegFixParams f) {
  constexpr int NCTW = DV == 64 ? 1 : 2, NW = DV / (16 * NCTW), NT = 64 * NW;
  constexpr int NQ = DK / 32, C = 64;
  constexpr int LDE = DK + 8;       // bf16 E rows in LDS (16 bytes of padding)
  constexpr int LDO = DV + 8;       // bf16 o rows in LDS
  __shared__ __attribute__((aligned(16))) bf16 sE[C * LDE];
  __shared__ __attribute__((aligned(16))) bf16 sO[C * LDO];
  const int tid = threadIdx.x, nt = NT;
  const int lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  constexpr int dv = DV;
  // (segment, head) pairs: blockIdx.y, then every gridDim.y-th (uniform per workgroup)
  for (long long sh = blockIdx.y; sh < f.nseg * f.H; sh += gridDim.y) {
    const int s = (int)(sh / f.H), h = (int)(sh % f.H);
    int b, st0, st1;
    if (!seg_tokens(f, s, b, st0, st1)) continue;
    const long long k0 = (long long)st0 + (long long)blockIdx.x * kSegRun * C;
    if (k0 >= st1) continue;
    const size_t rowbase = ((size_t)b * f.H + h) * (size_t)f.T;
    bf16x8 a[NCTW][NQ];
    {
      const bf16x8 *G = reinterpret_cast<const bf16x8 *>(f.sfix) + ((size_t)s * f.H + h) * (dv / 16) * NQ * 64;
#pragma unroll
      for (int ct = 0; ct < NCTW; ++ct)
#pragma unroll
        for (int q = 0; q < NQ; ++q) a[ct][q] = G[((w * NCTW + ct) * NQ + q) * 64 + lane];
    }
    const int tk0 = (int)k0, tk1 = (int)min((long long)st1, k0 + (long long)kSegRun * C);
    const int nrow = tk1 - tk0;
    // the run's rows of E and o as buffer ranges (rows past its end read as zero)
    const bf16 *E = static_cast<const bf16 *>(f.eout) + (rowbase + (size_t)tk0) * DK;
    bf16 *O = static_cast<bf16 *>(f.o) + (rowbase + (size_t)tk0) * dv;
    const __amdgpu_buffer_rsrc_t re = buffer_rsrc(E, nrow * DK * 2);
    const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(O, nrow * dv * 2);
    constexpr int epr = DK / 8, opr = DV / 8;  // 16-byte pieces per row
    // a chunk's pieces per thread; the next chunk's are loaded into registers while
    // this one is multiplied and stored
    constexpr int NPE = (C * epr + NT - 1) / NT, NPO = (C * opr + NT - 1) / NT;
    uint4 pe[NPE], po[NPO];
    auto load = [&](int tb) {
#pragma unroll
      for (int j = 0; j < NPE; ++j) {
        const int pc = tid + nt * j;
        pe[j] = buffer_ld16(re, ((tb + pc / epr) * DK + 8 * (pc % epr)) * 2);  // past the chunk: past the range
      }
#pragma unroll
      for (int j = 0; j < NPO; ++j) {
        const int pc = tid + nt * j;
        po[j] = buffer_ld16(ro, ((tb + pc / opr) * dv + 8 * (pc % opr)) * 2);
      }
    };
    load(0);
    for (int tb = 0; tb < nrow; tb += C) {
      __syncthreads();  // the previous chunk's o rows have left LDS
#pragma unroll
      for (int j = 0; j < NPE; ++j) {
        const int pc = tid + nt * j;
        if (pc < C * epr) *reinterpret_cast<uint4 *>(sE + (pc / epr) * LDE + 8 * (pc % epr)) = pe[j];
      }
#pragma unroll
      for (int j = 0; j < NPO; ++j) {
        const int pc = tid + nt * j;
        if (pc < C * opr) *reinterpret_cast<uint4 *>(sO + (pc / opr) * LDO + 8 * (pc % opr)) = po[j];
      }
      if (tb + C < nrow) load(tb + C);
      __syncthreads();
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        bf16x8 e[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) e[q] = *reinterpret_cast<const bf16x8 *>(sE + (16 * rb + li) * LDE + 32 * q + 8 * lg);
#pragma unroll
        for (int ct = 0; ct < NCTW; ++ct) {
          bf16 *cell = sO + (16 * rb + li) * LDO + 16 * (w * NCTW + ct) + 4 * lg;
          const bf16x4 v = *reinterpret_cast<const bf16x4 *>(cell);
          f32x4 acc = {(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
#pragma unroll
          for (int q = 0; q < NQ; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ct][q], e[q], acc, 0, 0, 0);
          *reinterpret_cast<bf16x4 *>(cell) = bf16x4{(bf16)acc[0], (bf16)acc[1], (bf16)acc[2], (bf16)acc[3]};
        }
      }
      __syncthreads();
      for (int pc = tid; pc < C * opr; pc += nt) {
        const int r = pc / opr, c8 = pc % opr;
        if (tb + r < nrow)
          *reinterpret_cast<uint4 *>(O + (size_t)(tb + r) * dv + 8 * c8) = *reinterpret_cast<const uint4 *>(sO + r * LDO + 8 * c8);
      }
    }
  }
}

// ---- correction, any element type and width (fp32 arithmetic) --------------------------
// One workgroup of 256 threads per (run of kSegRun chunks, later segment, head), the
// grid as in the MFMA kernel; each thread takes elements (token, column) of the run in
// turn: o += sum_k E[token][k] S[k][col], with S_start as fp32 rows.
template <typename E>
__global__ __launch_bounds__(256) void kla_seg_correct_simple_kernel(SegFixParams f) {
  const int dv = f.dv, dk = f.dk;
  const E *Ee = static_cast<const E *>(f.eout);
  E *O = static_cast<E *>(f.o);
  for (long long sh = blockIdx.y; sh < f.nseg * f.H; sh += gridDim.y) {
    const int s = (int)(sh / f.H), h = (int)(sh % f.H);
    int b, st0, st1;
    if (!seg_tokens(f, s, b, st0, st1)) continue;
    const long long k0 = (long long)st0 + (long long)blockIdx.x * kSegRun * f.C;
    if (k0 >= st1) continue;
    const size_t rowbase = ((size_t)b * f.H + h) * (size_t)f.T;
    const float *S = reinterpret_cast<const float *>(f.sfix) + ((size_t)s * f.H + h) * (size_t)dk * dv;
    const int tk0 = (int)k0, tk1 = (int)min((long long)st1, k0 + (long long)kSegRun * f.C);
    const long long nel = (long long)(tk1 - tk0) * dv;
    for (long long idx = threadIdx.x; idx < nel; idx += 256) {
      const size_t row = rowbase + (size_t)tk0 + (size_t)(idx / dv);
      const int col = (int)(idx % dv);
      float acc = Elem<E>::to_f32(O[row * dv + col]);
      for (int k = 0; k < dk; ++k) acc = fmaf(Elem<E>::to_f32(Ee[row * dk + k]), S[(size_t)k * dv + col], acc);
      O[row * dv + col] = Elem<E>::from_f32(acc);
    }
  }
}

// ---- launchers ----------------------------------------------------------------------------
hipError_t launch_seg_table(const SegFixParams &f, int *seg_first, hipStream_t st) {
  hipLaunchKernelGGL(kla_seg_table_kernel, dim3(1), dim3(1024), 0, st, f.cu, f.nseq, f.T, f.C, f.seg_chunks,
                     (int)f.nseg, seg_first);
  return hipGetLastError();
}

bool seg_correct_mfma(int dtype, int dk, int dv) {
  return dtype == 0 && (dk == 64 || dk == 128) && dv % 64 == 0 && dv >= 64 && dv <= 256;
}

template <int DK, bool GRP>
static hipError_t combine_t(const SegFixParams &f, hipStream_t st) {
  hipLaunchKernelGGL((kla_seg_combine_kernel<DK, GRP>), dim3((unsigned)(f.nseq * f.H), (unsigned)(f.dv / 16)),
                     dim3(combine_threads<DK>()), 0, st, f);
  return hipGetLastError();
}

// two column tiles per wave (one for dv = 64): dv / 32 waves, at most eight
template <int DK>
static hipError_t correct_mfma_t(const SegFixParams &f, dim3 grid, hipStream_t st) {
  switch (f.dv) {
    case 64: hipLaunchKernelGGL((kla_seg_correct_mfma_kernel<DK, 64>), grid, dim3(256), 0, st, f); break;
    case 128: hipLaunchKernelGGL((kla_seg_correct_mfma_kernel<DK, 128>), grid, dim3(256), 0, st, f); break;
    case 192: hipLaunchKernelGGL((kla_seg_correct_mfma_kernel<DK, 192>), grid, dim3(384), 0, st, f); break;
    case 256: hipLaunchKernelGGL((kla_seg_correct_mfma_kernel<DK, 256>), grid, dim3(512), 0, st, f); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_seg_finish(const SegFixParams &f, hipStream_t st) {
  if (f.nseq == 0 || f.H == 0) return hipSuccess;
  const bool mfma = seg_correct_mfma(f.dtype, f.dk, f.dv);
  hipError_t e;
  switch (f.dk) {
    case 16: e = combine_t<16, false>(f, st); break;
    case 32: e = combine_t<32, false>(f, st); break;
    case 64: e = mfma ? combine_t<64, true>(f, st) : combine_t<64, false>(f, st); break;
    case 128: e = mfma ? combine_t<128, true>(f, st) : combine_t<128, false>(f, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  if (f.nseg <= f.nseq) return hipSuccess;  // no later segments: nothing to correct
  // x: runs of kSegRun chunks of the longest segment (consecutive workgroups stream
  // consecutive rows); y: (segment, head) pairs, at most the device's 65,536 (the kernels
  // take the pairs beyond gridDim.y in turn)
  const int runs = (std::min(f.seg_chunks, std::max(f.seg_max_chunks, 1)) + kSegRun - 1) / kSegRun;
  const dim3 grid((unsigned)runs, (unsigned)std::min(f.nseg * f.H, 65535LL));
  if (mfma) return f.dk == 128 ? correct_mfma_t<128>(f, grid, st) : correct_mfma_t<64>(f, grid, st);
  if (f.dtype == 0)
    hipLaunchKernelGGL((kla_seg_correct_simple_kernel<bf16>), grid, dim3(256), 0, st, f);
  else
    hipLaunchKernelGGL((kla_seg_correct_simple_kernel<float>), grid, dim3(256), 0, st, f);
  return hipGetLastError();
}

}  // namespace kla
