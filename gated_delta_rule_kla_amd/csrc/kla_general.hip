// kla_general.hip -- the chunkwise solver for every shape and variant outside the
// two pipelined kernels of kla_chunk.hip, and the preconditioned decode step.
//
// Method: "Resumen Técnico: Atención Lineal Kaczmarz (KLA)" (gist.science/es/paper/2605.08587),
// §"La Regla de Actualización KLA" and §"Implementación" (Gated DeltaNet's block solver with
// B = Diag(beta)); "Preconditioned DeltaNet" (gist.science/es/paper/2604.21100), §2.C (the
// diagonal accumulator A_t = A_{t-1} + k_t (.) k_t and the squashed preconditioner
// P_t = Diag(A_t)^-1 applied to the write key) and §2.D (the gated variant, PGDN, and its
// block-parallel form).
//
// Per chunk of C tokens with start state S (gamma = running sum of g in the chunk,
// Gam = exp(gamma), d_r = exp(gamma_C - gamma_r)), read keys K and write keys W (W = K
// except for PGDN, where w_t = p_t (.) k_t):
//
//   A  = strictly-lower(Diag(beta) K W^T), entry (r, s) weighted by exp(gamma_r - gamma_s)
//   T' = (I + A)^-1 Diag(beta)
//   X  = V - Diag(Gam) K S,   U~ = T' X
//   O  = Diag(Gam) Q S + (Q W^T masked r >= s, weighted exp(gamma_r - gamma_s)) U~
//   S <- Gam_C S + W^T Diag(d) U~
//
// One workgroup (256 threads) owns one (sequence, head, 16 state columns) and walks the
// sequence's chunks in order; every phase below is separated by a workgroup barrier and
// works on fp32 copies of the chunk in LDS (bf16 inputs are widened exactly), so both
// element types compute in fp32 end to end.  It needs no workspace: the S-independent
// work is redone by each column slice, which is what the pipelined kernels avoid; this
// path is for coverage of shapes and variants, not for throughput.
//
// PGDN's accumulator runs through the whole sequence; each workgroup carries it across
// its chunks itself (an in-chunk prefix per key coordinate), and the workgroup of column
// slice 0 writes the final accumulator.  Readings of the preconditioner (the page fixes
// only its ingredients): p_i = exp(c tanh(r_i / c)), c = ln(band), with
// r_i = log((mean_j A_j + delta) / (A_i + delta)), delta = 1e-30; band = 1 gives p = 1.
#include "kla.h"
#include "kla_common.h"
#include "kla_internal.h"
#include "kla_ops.h"

namespace kla {

namespace {

constexpr int kGenThreads = 256;
constexpr int kGenCols = 16;  // state columns per workgroup
constexpr float kPgdnDelta = 1e-30f;

struct GenParams {
  const void *q, *k, *v, *g, *coef;
  float eps;
  int beta_direct;  // 1: coef is beta itself; 0: Kaczmarz gain coef / (k . w + eps)
  float band_c;     // PGDN: ln(band) (0: p = 1)
  const float *s0;
  void *o;
  float *sfin;
  const float *acc0;  // PGDN: [N, H, DK] or nullptr (zeros)
  float *accfin;      // PGDN: [N, H, DK] or nullptr
  const int32_t *cu;
  int H, T, dv, nseq, n_tiles;
};

__device__ __forceinline__ float pgdn_weight(float a, float mean, float c) {
  if (c == 0.f) return 1.f;
  const float r = logf((mean + kPgdnDelta) / (a + kPgdnDelta));
  return expf(c * tanhf(r / c));
}

template <typename E, int C, int DK, bool PG>
struct GenSmem {
  static constexpr int LK = DK + 1;  // K, Q, W rows (odd stride: column reads hit distinct banks)
  static constexpr int LC = C + 1;   // A (then P) and T' rows
  static constexpr int LV = kGenCols + 1;
  static constexpr int K = 0;
  static constexpr int Q = K + C * LK;
  static constexpr int W = Q + C * LK;                        // PGDN only
  static constexpr int AP = W + (PG ? C * LK : 0);            // A, later the decayed scores P
  static constexpr int TT = AP + C * LC;                      // T' = T Diag(beta)
  static constexpr int V = TT + C * LC;                       // V slice, then X in place
  static constexpr int U = V + C * LV;                        // U~
  static constexpr int S = U + C * LV;                        // state slice, DK x 16
  static constexpr int VEC = S + DK * LV;                     // gamma, Gam, d, beta, g, coef, mean
  static constexpr int ACC = VEC + 7 * C;                     // PGDN accumulator, DK
  static constexpr int FLOATS = ACC + DK;
  static_assert(FLOATS * 4 <= 160 * 1024, "LDS budget");
};

// Inclusive prefix sum over one wave's 64 lanes (lanes >= n contribute 0).
__device__ __forceinline__ float wave_prefix(float x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

template <typename E, int C, int DK, bool PG>
__global__ __launch_bounds__(kGenThreads) void kla_chunk_general_kernel(GenParams p) {
  using L = GenSmem<E, C, DK, PG>;
  __shared__ __attribute__((aligned(16))) float sm[L::FLOATS];
  float *sK = sm + L::K, *sQ = sm + L::Q, *sW = PG ? sm + L::W : sm + L::K;
  float *sAP = sm + L::AP, *sT = sm + L::TT, *sV = sm + L::V, *sU = sm + L::U, *sS = sm + L::S;
  float *sGam = sm + L::VEC, *sGm = sGam + C, *sD = sGam + 2 * C, *sBeta = sGam + 3 * C;
  float *sG = sGam + 4 * C, *sCoef = sGam + 5 * C, *sMean = sGam + 6 * C;
  float *sAcc = sm + L::ACC;
  const int tid = threadIdx.x;

  const int grp = blockIdx.x / p.n_tiles, jt = blockIdx.x % p.n_tiles;
  const int n = grp / p.H, h = grp % p.H;
  int b = n, t0 = 0, t1 = p.T;
  if (p.cu) {
    b = 0;
    t0 = min(max(p.cu[n], 0), p.T);
    t1 = min(max(p.cu[n + 1], t0), p.T);
  }
  const int len = t1 - t0;
  const size_t row0 = ((size_t)b * p.H + h) * (size_t)p.T + (size_t)t0;
  const int dv = p.dv, col0 = jt * kGenCols;
  const size_t sbase = ((size_t)n * p.H + h) * DK * (size_t)dv;
  const E *gq = static_cast<const E *>(p.q) + row0 * DK;
  const E *gk = static_cast<const E *>(p.k) + row0 * DK;
  const E *gv = static_cast<const E *>(p.v) + row0 * (size_t)dv;
  const E *gg = static_cast<const E *>(p.g) + row0;
  const E *gc = static_cast<const E *>(p.coef) + row0;
  E *go = static_cast<E *>(p.o) + row0 * (size_t)dv;

  // state slice and accumulator
  for (int e = tid; e < DK * kGenCols; e += kGenThreads) {
    const int i = e / kGenCols, c = e % kGenCols;
    sS[i * L::LV + c] = p.s0 ? p.s0[sbase + (size_t)i * dv + col0 + c] : 0.f;
  }
  if (PG && tid < DK) sAcc[tid] = p.acc0 ? p.acc0[((size_t)n * p.H + h) * DK + tid] : 0.f;
  __syncthreads();

  const int nch = (len + C - 1) / C;
  for (int ch = 0; ch < nch; ++ch) {
    const int r0 = ch * C, nrow = min(C, len - r0);
    // ---- load the chunk: 16-byte pieces, all in flight before any is stored; rows
    // past the chunk's end read as zero through the buffer bounds ------------------
    {
      constexpr int EP = 16 / (int)sizeof(E);                 // elements per piece
      constexpr int PK = C * DK / EP;                         // pieces of K (and of Q)
      constexpr int NPK = (PK + kGenThreads - 1) / kGenThreads;
      constexpr int PPV = kGenCols / EP;                      // pieces per V row slice
      constexpr int PV = C * PPV;
      constexpr int NPV = (PV + kGenThreads - 1) / kGenThreads;
      const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(gk + (size_t)r0 * DK, nrow * DK * (int)sizeof(E));
      const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(gq + (size_t)r0 * DK, nrow * DK * (int)sizeof(E));
      const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(gv + (size_t)r0 * dv, nrow * dv * (int)sizeof(E));
      uint4 kv[NPK], qv[NPK], vv[NPV];
#pragma unroll
      for (int m = 0; m < NPK; ++m) {
        const int pc = min(tid + kGenThreads * m, PK - 1);
        kv[m] = buffer_ld16(rk, pc * 16);
        qv[m] = buffer_ld16(rq, pc * 16);
      }
#pragma unroll
      for (int m = 0; m < NPV; ++m) {
        const int pc = min(tid + kGenThreads * m, PV - 1);
        vv[m] = buffer_ld16(rv, ((pc / PPV) * dv + col0 + (pc % PPV) * EP) * (int)sizeof(E));
      }
#pragma unroll
      for (int m = 0; m < NPK; ++m) {
        const int pc = tid + kGenThreads * m;
        if (PK % kGenThreads == 0 || pc < PK) {
          const int r = pc / (DK / EP), i0 = (pc % (DK / EP)) * EP;
          const E *ke = reinterpret_cast<const E *>(&kv[m]), *qe = reinterpret_cast<const E *>(&qv[m]);
#pragma unroll
          for (int x = 0; x < EP; ++x) {
            sK[r * L::LK + i0 + x] = Elem<E>::to_f32(ke[x]);
            sQ[r * L::LK + i0 + x] = Elem<E>::to_f32(qe[x]);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < NPV; ++m) {
        const int pc = tid + kGenThreads * m;
        if (PV % kGenThreads == 0 || pc < PV) {
          const int r = pc / PPV, c0 = (pc % PPV) * EP;
          const E *ve = reinterpret_cast<const E *>(&vv[m]);
#pragma unroll
          for (int x = 0; x < EP; ++x) sV[r * L::LV + c0 + x] = Elem<E>::to_f32(ve[x]);
        }
      }
    }
    if (tid < C) {
      sG[tid] = tid < nrow ? Elem<E>::to_f32(gg[r0 + tid]) : 0.f;
      sCoef[tid] = tid < nrow ? Elem<E>::to_f32(gc[r0 + tid]) : 0.f;
    }
    __syncthreads();

    // ---- PGDN: accumulator prefix per coordinate, row means, write keys -----------
    if constexpr (PG) {
      if (tid < DK) {
        float a = sAcc[tid];
        for (int r = 0; r < C; ++r) {
          const float x = sK[r * L::LK + tid];
          a = fmaf(x, x, a);
          sW[r * L::LK + tid] = a;  // A_t for row r (includes row r)
        }
        sAcc[tid] = a;
      }
      __syncthreads();
      if (tid < C) {
        float m = 0.f;
        for (int i = 0; i < DK; ++i) m += sW[tid * L::LK + i];
        sMean[tid] = m / (float)DK;
      }
      __syncthreads();
      for (int e = tid; e < C * DK; e += kGenThreads) {
        const int r = e / DK, i = e % DK;
        sW[r * L::LK + i] = pgdn_weight(sW[r * L::LK + i], sMean[r], p.band_c) * sK[r * L::LK + i];
      }
      __syncthreads();
    }

    // ---- gates and beta (wave 0: lane = chunk row) ---------------------------------
    if (tid < 64) {
      const float gam = wave_prefix(tid < C ? sG[tid] : 0.f);
      const float gamC = __shfl(gam, C - 1, 64);
      if (tid < C) {
        sGam[tid] = gam;
        sGm[tid] = expf(gam);
        sD[tid] = expf(gamC - gam);
        float nk = 0.f;
        for (int i = 0; i < DK; ++i) nk = fmaf(sK[tid * L::LK + i], sW[tid * L::LK + i], nk);
        const float c = sCoef[tid];
        sBeta[tid] = tid < nrow ? (p.beta_direct ? c : c / (nk + p.eps)) : 0.f;
      }
    }
    __syncthreads();

    // ---- A = strictly-lower(Diag(beta) K W^T . decay), 4x4 register blocks ---------
    constexpr int NB4 = C / 4;
    for (int blk = tid; blk < NB4 * NB4; blk += kGenThreads) {
      const int bi = blk / NB4, bj = blk % NB4;
      float acc[4][4];
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = 0.f;
      if (bj <= bi) {
        for (int i = 0; i < DK; ++i) {
          float kr[4], ws[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) kr[x] = sK[(4 * bi + x) * L::LK + i];
#pragma unroll
          for (int y = 0; y < 4; ++y) ws[y] = sW[(4 * bj + y) * L::LK + i];
#pragma unroll
          for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int y = 0; y < 4; ++y) acc[x][y] = fmaf(kr[x], ws[y], acc[x][y]);
        }
      }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          const int r = 4 * bi + x, s = 4 * bj + y;
          sAP[r * L::LC + s] = s < r ? sBeta[r] * acc[x][y] * expf(sGam[r] - sGam[s]) : 0.f;
        }
    }
    __syncthreads();

    // ---- T = (I + A)^-1 by forward substitution, one column per thread; T' = T Diag(beta)
    // Thread j keeps column j of T in registers (both loops unrolled, so it is never
    // indexed at run time) and reads the rows of A as broadcasts; four partial sums
    // shorten the dependent chain of each row.  Entries above the diagonal come out
    // as zero because the column's entries above row j are zero.
    if (tid < C) {
      const int j = tid;
      float tc[C];
#pragma unroll
      for (int r = 0; r < C; ++r) {
        float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < r; ++m) s4[m & 3] = fmaf(sAP[r * L::LC + m], tc[m], s4[m & 3]);
        const float sum = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        tc[r] = r < j ? 0.f : (r == j ? 1.f : -sum);
      }
      const float bj = sBeta[j];
#pragma unroll
      for (int r = 0; r < C; ++r) sT[r * L::LC + j] = tc[r] * bj;
    }
    __syncthreads();

    // ---- scores P = (Q W^T) . decay (r >= s) into A's place; X = V - Gam K S; Gam Q S ---
    for (int blk = tid; blk < NB4 * NB4; blk += kGenThreads) {
      const int bi = blk / NB4, bj = blk % NB4;
      float acc[4][4];
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = 0.f;
      if (bj <= bi) {
        for (int i = 0; i < DK; ++i) {
          float qr[4], ws[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) qr[x] = sQ[(4 * bi + x) * L::LK + i];
#pragma unroll
          for (int y = 0; y < 4; ++y) ws[y] = sW[(4 * bj + y) * L::LK + i];
#pragma unroll
          for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int y = 0; y < 4; ++y) acc[x][y] = fmaf(qr[x], ws[y], acc[x][y]);
        }
      }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          const int r = 4 * bi + x, s = 4 * bj + y;
          sAP[r * L::LC + s] = s <= r ? acc[x][y] * expf(sGam[r] - sGam[s]) : 0.f;
        }
    }
    // output rows of this thread: column c = tid % 16, rows tid / 16 + 16 m
    constexpr int RPT = (C * kGenCols + kGenThreads - 1) / kGenThreads;
    float out[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      const int e = tid + kGenThreads * m;
      out[m] = 0.f;
      if (e < C * kGenCols) {
        const int r = e / kGenCols, c = e % kGenCols;
        float ks = 0.f, qs = 0.f;
        for (int i = 0; i < DK; ++i) {
          const float s = sS[i * L::LV + c];
          ks = fmaf(sK[r * L::LK + i], s, ks);
          qs = fmaf(sQ[r * L::LK + i], s, qs);
        }
        sV[r * L::LV + c] -= sGm[r] * ks;  // X
        out[m] = sGm[r] * qs;
      }
    }
    __syncthreads();

    // ---- U~ = T' X -------------------------------------------------------------------
    for (int e = tid; e < C * kGenCols; e += kGenThreads) {
      const int r = e / kGenCols, c = e % kGenCols;
      float u = 0.f;
      for (int s = 0; s <= r; ++s) u = fmaf(sT[r * L::LC + s], sV[s * L::LV + c], u);
      sU[r * L::LV + c] = u;
    }
    __syncthreads();

    // ---- O = Gam Q S + P U~ (written), S <- Gam_C S + W^T Diag(d) U~ -------------------
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      const int e = tid + kGenThreads * m;
      if (e < C * kGenCols) {
        const int r = e / kGenCols, c = e % kGenCols;
        float o = out[m];
        for (int s = 0; s <= r; ++s) o = fmaf(sAP[r * L::LC + s], sU[s * L::LV + c], o);
        if (r < nrow) go[(size_t)(r0 + r) * dv + col0 + c] = Elem<E>::from_f32(o);
      }
    }
    const float gC = sGm[C - 1];
    for (int e = tid; e < DK * kGenCols; e += kGenThreads) {
      const int i = e / kGenCols, c = e % kGenCols;
      float s = gC * sS[i * L::LV + c];
      for (int r = 0; r < C; ++r) s = fmaf(sW[r * L::LK + i] * sD[r], sU[r * L::LV + c], s);
      sS[i * L::LV + c] = s;
    }
    __syncthreads();
  }

  if (p.sfin) {
    for (int e = tid; e < DK * kGenCols; e += kGenThreads) {
      const int i = e / kGenCols, c = e % kGenCols;
      p.sfin[sbase + (size_t)i * dv + col0 + c] = sS[i * L::LV + c];
    }
  }
  if (PG && p.accfin && jt == 0 && tid < DK) p.accfin[((size_t)n * p.H + h) * DK + tid] = sAcc[tid];
}

// ----------------------------------------------------------------------------
// PGDN decode step: one workgroup per (sequence, head), thread j owns state column j
// ----------------------------------------------------------------------------
struct PgdnDecodeParams {
  const void *q, *k, *v, *g, *coef;
  float eps, band_c;
  int beta_direct;
  float *state, *acc;
  void *o;
  int N, H, dv;
};

template <typename E, int DK>
__global__ __launch_bounds__(256) void kla_pgdn_decode_kernel(PgdnDecodeParams p) {
  __shared__ float sk[DK], sq[DK], sw[DK], sred[3][8];
  const int nh = blockIdx.x, tid = threadIdx.x;
  const E *k = static_cast<const E *>(p.k) + (size_t)nh * DK;
  const E *q = static_cast<const E *>(p.q) + (size_t)nh * DK;
  float a = 0.f;
  if (tid < DK) {
    sk[tid] = Elem<E>::to_f32(k[tid]);
    sq[tid] = Elem<E>::to_f32(q[tid]);
    a = p.acc[(size_t)nh * DK + tid] + sk[tid] * sk[tid];
  }
  // mean of the updated accumulator over the DK coordinates
  auto block_sum = [&](float x, int slot) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    if ((tid & 63) == 0) sred[slot][tid >> 6] = x;
    __syncthreads();
    float t = 0.f;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += sred[slot][w];
    return t;
  };
  const float mean = block_sum(a, 0) / (float)DK;
  float wk = 0.f, wq = 0.f;
  if (tid < DK) {
    const float w = pgdn_weight(a, mean, p.band_c) * sk[tid];
    sw[tid] = w;
    wk = w * sk[tid];
    wq = w * sq[tid];
    p.acc[(size_t)nh * DK + tid] = a;
  }
  const float kw = block_sum(wk, 1), qw = block_sum(wq, 2);
  const float alpha = expf(Elem<E>::to_f32(static_cast<const E *>(p.g)[nh]));
  const float c = Elem<E>::to_f32(static_cast<const E *>(p.coef)[nh]);
  const float beta = p.beta_direct ? c : c / (kw + p.eps);
  for (int j = tid; j < p.dv; j += blockDim.x) {
    float *S = p.state + (size_t)nh * DK * p.dv + j;
    float col[DK];
    float yk = 0.f, yq = 0.f;
#pragma unroll
    for (int i = 0; i < DK; ++i) {
      col[i] = S[(size_t)i * p.dv];
      yk = fmaf(col[i], sk[i], yk);
      yq = fmaf(col[i], sq[i], yq);
    }
    const float e = Elem<E>::to_f32(static_cast<const E *>(p.v)[(size_t)nh * p.dv + j]) - alpha * yk;
    // o = S_new^T q = alpha S^T q + beta (w . q) e
    static_cast<E *>(p.o)[(size_t)nh * p.dv + j] = Elem<E>::from_f32(alpha * yq + beta * qw * e);
#pragma unroll
    for (int i = 0; i < DK; ++i) S[(size_t)i * p.dv] = fmaf(alpha, col[i], beta * sw[i] * e);
  }
}

template <typename E, int C, int DK, bool PG>
hipError_t launch_general_t(const ChunkArgs &a, const GenExtra &x, hipStream_t st) {
  GenParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.g = a.g;
  p.coef = a.eta;
  p.eps = a.eps;
  p.beta_direct = a.beta_direct;
  p.band_c = x.band_c;
  p.s0 = a.initial_state;
  p.o = a.o;
  p.sfin = a.final_state;
  p.acc0 = x.initial_acc;
  p.accfin = x.final_acc;
  p.cu = a.cu_seqlens;
  p.H = a.H;
  p.T = a.T;
  p.dv = a.dv;
  p.nseq = a.num_seqs;
  p.n_tiles = a.dv / kGenCols;
  const long long nblk = (long long)a.num_seqs * a.H * p.n_tiles;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL((kla_chunk_general_kernel<E, C, DK, PG>), dim3((unsigned)nblk), dim3(kGenThreads), 0, st, p);
  return hipGetLastError();
}

template <typename E, bool PG>
hipError_t launch_general_dk(const ChunkArgs &a, const GenExtra &x, hipStream_t st) {
  if (a.chunk == 16) {
    switch (a.dk) {
      case 16: return launch_general_t<E, 16, 16, PG>(a, x, st);
      case 32: return launch_general_t<E, 16, 32, PG>(a, x, st);
      case 64: return launch_general_t<E, 16, 64, PG>(a, x, st);
      case 128: return launch_general_t<E, 16, 128, PG>(a, x, st);
    }
  } else if (a.chunk == 64) {
    switch (a.dk) {
      case 16: return launch_general_t<E, 64, 16, PG>(a, x, st);
      case 32: return launch_general_t<E, 64, 32, PG>(a, x, st);
      case 64: return launch_general_t<E, 64, 64, PG>(a, x, st);
      case 128: return launch_general_t<E, 64, 128, PG>(a, x, st);
    }
  }
  return hipErrorInvalidValue;
}

template <typename E, int DK>
hipError_t launch_pgdn_decode_t(const PgdnDecodeParams &p, hipStream_t st) {
  hipLaunchKernelGGL((kla_pgdn_decode_kernel<E, DK>), dim3((unsigned)(p.N * p.H)), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace

bool general_supported(int dtype, int dk, int dv, int chunk) {
  return (dtype == 0 || dtype == 1) && (chunk == 16 || chunk == 64) &&
         (dk == 16 || dk == 32 || dk == 64 || dk == 128) && dv % kGenCols == 0 && dv >= 16 && dv <= 256;
}

hipError_t launch_chunk_general(const ChunkArgs &a, const GenExtra &x, hipStream_t st) {
  if (a.dtype == 0) return x.pgdn ? launch_general_dk<bf16, true>(a, x, st) : launch_general_dk<bf16, false>(a, x, st);
  return x.pgdn ? launch_general_dk<float, true>(a, x, st) : launch_general_dk<float, false>(a, x, st);
}

bool pgdn_decode_supported(int dtype, int dk, int dv) {
  return (dtype == 0 || dtype == 1) && (dk == 16 || dk == 32 || dk == 64 || dk == 128) && dv >= 1 && dv <= 256;
}

hipError_t launch_pgdn_decode(const DecodeArgs &a, float band_c, float *acc, hipStream_t st) {
  // the HBM-tuned decode kernel where it has the shape; this one for the other dv
  if (decode_supported(a.dtype, a.dk, a.dv)) return launch_decode_pgdn(a, band_c, acc, st);
  PgdnDecodeParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.g = a.g;
  p.coef = a.eta;
  p.eps = a.eps;
  p.band_c = band_c;
  p.beta_direct = a.beta_direct;
  p.state = a.state;
  p.acc = acc;
  p.o = a.o;
  p.N = a.N;
  p.H = a.H;
  p.dv = a.dv;
  if ((long long)a.N * a.H == 0) return hipSuccess;
  if (a.dtype == 0) {
    switch (a.dk) {
      case 16: return launch_pgdn_decode_t<bf16, 16>(p, st);
      case 32: return launch_pgdn_decode_t<bf16, 32>(p, st);
      case 64: return launch_pgdn_decode_t<bf16, 64>(p, st);
      case 128: return launch_pgdn_decode_t<bf16, 128>(p, st);
    }
  } else {
    switch (a.dk) {
      case 16: return launch_pgdn_decode_t<float, 16>(p, st);
      case 32: return launch_pgdn_decode_t<float, 32>(p, st);
      case 64: return launch_pgdn_decode_t<float, 64>(p, st);
      case 128: return launch_pgdn_decode_t<float, 128>(p, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace kla
