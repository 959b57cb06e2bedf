// kla_chunk.hip -- chunkwise-parallel KLA prefill for gfx950 (CDNA4).
//
// Method: "Resumen Técnico: Atención Lineal Kaczmarz (KLA)",
// gist.science/es/paper/2605.08587.  §"La Regla de Actualización KLA" gives the
// token update S_t = alpha_t S_{t-1} + beta_t k_t e_t^T with
// beta_t = eta_t / (||k_t||^2 + eps); §"Implementación" says the chunkwise
// block solver of Gated DeltaNet is kept and only B = Diag(beta) changes.
//
// Per chunk of C tokens with start state S (local rows r, s; gamma = running
// sum of the log-decay g inside the chunk, Gam = exp(gamma), d = exp(gamma_C - gamma)):
//
//   A   = strictly-lower(Diag(beta) K K^T weighted by exp(gamma_r - gamma_s))
//   T'  = (I + A)^-1 Diag(beta)                      (S-independent)
//   P   = lower-incl(Q K^T weighted by exp(gamma_r - gamma_s))
//   X   = V - Diag(Gam) K S
//   U~  = T' X                                       (U~_r = beta_r e_r)
//   O   = Diag(Gam) Q S + P U~
//   S  <- Gam_C S + K^T Diag(d) U~
//
// (the reassociated form of W = T Diag(beta Gam) K, U = T Diag(beta) V,
// U~ = U - W S: it keeps the per-column work proportional to the column
// count).  Every exponent used is of a non-positive number; the mask is
// applied before the exponential.
//
// Mapping onto the chip.  One workgroup owns one (sequence, head, slice of
// DVT = 16 NBW state columns) and walks that sequence's chunks in order.  The
// state slice never leaves the chip: it lives in MFMA accumulators of the
// NBW "scan" waves (16 columns each, fp32) for the whole sequence.  Two
// "producer" waves build the S-independent data of chunk c+1 while the scan
// waves consume chunk c (double-buffered LDS, one barrier per chunk):
//   * the K wave: loads K (16-byte loads straight into MFMA operand layout),
//     fuses the ||k||^2 reduction and beta, scans the gates, forms K K^T on
//     MFMA, A, and solves the 64x64 unit-lower-triangular system blockwise:
//     the four 16x16 diagonal blocks by column-parallel forward substitution
//     in fp32 (lane = block x column), the off-diagonal blocks by 16x16x16
//     MFMA products T_ij = -T_ii sum_m A_im T_mj, level by level;
//   * the Q wave: loads Q and V, forms Q K^T on MFMA and the causal score
//     tile P.
// The scan waves run X, U~, O and the state update as MFMA tile products
// (bf16 operands, fp32 accumulation).  Inputs are read from HBM once per
// workgroup; the workgroups of one (sequence, head) are placed on the same
// XCD so their shared K/Q reads hit that XCD's L2.
#include "kla_common.h"
#include "kla_internal.h"

namespace kla {

// ---------------------------------------------------------------------------
// MFMA primitives.  For a 16x16 output tile D (fp32) the conventions are:
//   A operand (row-major M[m][k]):    lane l holds M[l&15][kb + (l>>4)*VPL + x]
//   B operand (stored as Nt[n][k]):   lane l holds Nt[l&15][kb + (l>>4)*VPL + x]
//   D:                                lane l holds D[4*(l>>4) + j][l&15], j < 4
// ---------------------------------------------------------------------------
template <typename E> struct Mfma;

template <> struct Mfma<bf16> {
  static constexpr int KSTEP = 32;
  static constexpr int VPL = 8;
  typedef bf16x8 Op;
  static __device__ __forceinline__ f32x4 mma(Op a, Op b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ Op ld(const bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
  static __device__ __forceinline__ void st(bf16 *p, Op v) { *reinterpret_cast<bf16x8 *>(p) = v; }
  static __device__ __forceinline__ Op ld_strided(const bf16 *p, int stride) {
    Op r;
#pragma unroll
    for (int x = 0; x < 8; ++x) r[x] = p[x * stride];
    return r;
  }
  static __device__ __forceinline__ Op ldg(const bf16 *p) {
    uint4 u = ldg16(p);
    return __builtin_bit_cast(Op, u);
  }
  static __device__ __forceinline__ Op zero() {
    Op r;
#pragma unroll
    for (int x = 0; x < 8; ++x) r[x] = (bf16)0.f;
    return r;
  }
  static __device__ __forceinline__ float sumsq(Op v) {
    float s = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const float f = (float)v[x];
      s = fmaf(f, f, s);
    }
    return s;
  }
};

template <> struct Mfma<float> {
  static constexpr int KSTEP = 4;
  static constexpr int VPL = 1;
  typedef float Op;
  static __device__ __forceinline__ f32x4 mma(Op a, Op b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ Op ld(const float *p) { return *p; }
  static __device__ __forceinline__ void st(float *p, Op v) { *p = v; }
  static __device__ __forceinline__ Op ld_strided(const float *p, int) { return *p; }
  static __device__ __forceinline__ Op ldg(const float *p) { return *p; }
  static __device__ __forceinline__ Op zero() { return 0.f; }
  static __device__ __forceinline__ float sumsq(Op v) { return v * v; }
};

// 16x16x16 product with operands given as 4 fp32 values per lane:
//   a[x] = A[l&15][4(l>>4) + x],  b[x] = B[4(l>>4) + x][l&15]
// The D layout equals this B layout, so products chain in registers.
template <typename E> struct Mm16;

template <> struct Mm16<bf16> {
  static __device__ __forceinline__ f32x4 mma(const float *a, const float *b, f32x4 c) {
    bf16x4 av, bv;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      av[x] = (bf16)a[x];
      bv[x] = (bf16)b[x];
    }
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, c, 0, 0, 0);
  }
};

template <> struct Mm16<float> {
  static __device__ __forceinline__ f32x4 mma(const float *a, const float *b, f32x4 c) {
#pragma unroll
    for (int x = 0; x < 4; ++x) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[x], b[x], c, 0, 0, 0);
    return c;
  }
};

// four consecutive E <-> f32x4
__device__ __forceinline__ void store4(bf16 *p, f32x4 v) {
  bf16x4 b;
#pragma unroll
  for (int x = 0; x < 4; ++x) b[x] = (bf16)v[x];
  *reinterpret_cast<bf16x4 *>(p) = b;
}
__device__ __forceinline__ void store4(float *p, f32x4 v) { *reinterpret_cast<f32x4 *>(p) = v; }
__device__ __forceinline__ f32x4 load4(const bf16 *p) {
  bf16x4 b = *reinterpret_cast<const bf16x4 *>(p);
  f32x4 r;
#pragma unroll
  for (int x = 0; x < 4; ++x) r[x] = (float)b[x];
  return r;
}
__device__ __forceinline__ f32x4 load4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------------------
// LDS plan
// ---------------------------------------------------------------------------
template <typename E, int C, int DK, int NBW>
struct ChunkShape {
  static constexpr int NB = C / 16;           // 16-row blocks per chunk
  static constexpr int DVT = 16 * NBW;        // state columns per workgroup
  static constexpr int NWAVES = NBW + 2;      // scan waves + K wave + Q wave
  static constexpr int NT = 64 * NWAVES;
  static constexpr int PAD = 16 / (int)sizeof(E);
  static constexpr int LDK = DK + PAD;        // pitch of K, Q and S^T rows
  static constexpr int LDC = C + PAD;         // pitch of C-wide rows
  static constexpr int LDD = 20;              // fp32 pitch of 16-wide diagonal blocks
  static constexpr int KSTEPS = DK / Mfma<E>::KSTEP;
  // shared double buffer (elements of E, then floats)
  static constexpr int OFF_K = 0;
  static constexpr int OFF_Q = OFF_K + C * LDK;
  static constexpr int OFF_VT = OFF_Q + C * LDK;
  static constexpr int OFF_TP = OFF_VT + DVT * LDC;
  static constexpr int OFF_P = OFF_TP + C * LDC;
  static constexpr int BUF_E = OFF_P + C * LDC;
  static constexpr int BUF_F = 2 * C;         // Gam[C], d[C]
  static constexpr int BUF_BYTES = BUF_E * (int)sizeof(E) + BUF_F * 4;
  // K wave private
  static constexpr int A_BYTES = C * LDC * (int)sizeof(E);       // A, row-major, E
  static constexpr int ATD_BYTES = NB * 16 * LDD * 4;            // A diagonal blocks, transposed, fp32
  static constexpr int TD_BYTES = NB * 16 * LDD * 4;             // T diagonal blocks, fp32
  // scan wave private: S^T (16 x DK), X^T, U~^T, (dU~)^T (16 x C each)
  static constexpr int SCAN_BYTES = (16 * LDK + 3 * 16 * LDC) * (int)sizeof(E);
  static constexpr int OFF_KW = 2 * BUF_BYTES;
  static constexpr int OFF_SW = OFF_KW + A_BYTES + ATD_BYTES + TD_BYTES;
  static constexpr int BYTES = OFF_SW + NBW * SCAN_BYTES;

  static_assert(C == 16 || C == 64, "chunk");
  static_assert(DK % Mfma<E>::KSTEP == 0 && DK % 16 == 0, "dk");
  static_assert(BUF_BYTES % 16 == 0 && A_BYTES % 16 == 0 && SCAN_BYTES % 16 == 0, "lds align");
  static_assert((16 * LDK * (int)sizeof(E)) % 16 == 0 && (16 * LDC * (int)sizeof(E)) % 16 == 0, "align");
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

struct ChunkParams {
  const void *q, *k, *v, *g, *eta;
  float eps;
  const float *s0;
  void *o;
  float *sfin;
  const int32_t *cu;
  int H, T, dv, n_tiles, remap;
};

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <typename E, int C, int DK, int NBW>
__global__ __launch_bounds__(64 * (NBW + 2)) void kla_chunk_kernel(ChunkParams p) {
  using Sh = ChunkShape<E, C, DK, NBW>;
  using M = Mfma<E>;
  using Op = typename M::Op;
  constexpr int NB = Sh::NB, DVT = Sh::DVT, LDK = Sh::LDK, LDC = Sh::LDC, LDD = Sh::LDD;
  constexpr int KSTEP = M::KSTEP, VPL = M::VPL, KSTEPS = Sh::KSTEPS;
  constexpr int NTRI = NB * (NB + 1) / 2;

  __shared__ __attribute__((aligned(16))) char smem[Sh::BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15;  // row / column inside a 16-wide tile
  const int lg = lane >> 4;  // lane group 0..3

  // ---- which (sequence, head, column slice) this workgroup owns ----------
  int L = blockIdx.x;
  if (p.remap) L = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int jt = L % p.n_tiles;
  const int nh = L / p.n_tiles;
  const int h = nh % p.H;
  const int n = nh / p.H;
  int b = n, t0 = 0, t1 = p.T;
  if (p.cu) {
    b = 0;
    t0 = min(max(p.cu[n], 0), p.T);
    t1 = min(max(p.cu[n + 1], t0), p.T);
  }
  const int len = t1 - t0;
  const int nch = (len + C - 1) / C;
  const size_t row0 = ((size_t)b * p.H + h) * (size_t)p.T + (size_t)t0;
  const E *gq = static_cast<const E *>(p.q);
  const E *gk = static_cast<const E *>(p.k);
  const E *gv = static_cast<const E *>(p.v);
  const E *gg = static_cast<const E *>(p.g);
  const E *geta = static_cast<const E *>(p.eta);
  E *go = static_cast<E *>(p.o);
  const int dv = p.dv;

  auto bufE = [&](int i) { return reinterpret_cast<E *>(smem + i * Sh::BUF_BYTES); };
  auto bufF = [&](int i) {
    return reinterpret_cast<float *>(smem + i * Sh::BUF_BYTES + Sh::BUF_E * (int)sizeof(E));
  };

  // strictly-upper 16x16 blocks of T' and P are zero and never rewritten
  for (int i = threadIdx.x; i < 2 * C * C; i += Sh::NT) {
    const int bi = i / (C * C), rr = (i / C) % C, ss = i % C;
    if ((rr >> 4) < (ss >> 4)) {
      bufE(bi)[Sh::OFF_TP + rr * LDC + ss] = Elem<E>::from_f32(0.f);
      bufE(bi)[Sh::OFF_P + rr * LDC + ss] = Elem<E>::from_f32(0.f);
    }
  }

  // ---- gate scan shared by both producer waves ----------------------------
  // lane r < C: gamma_r (inclusive running sum of g inside the chunk)
  auto gate_scan = [&](int nrow, size_t tok0, float &gv_out) -> float {
    float gl = 0.f;
    if (lane < nrow) gl = Elem<E>::to_f32(gg[tok0 + lane]);
    gv_out = gl;
    float gam = gl;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float t = __shfl_up(gam, off);
      if (lane >= off) gam += t;
    }
    return gam;
  };

  // ======================= K wave: chunk c -> buffer nb ======================
  auto produce_k = [&](int c, int nb) {
    E *sK = bufE(nb) + Sh::OFF_K;
    E *sTp = bufE(nb) + Sh::OFF_TP;
    float *sF = bufF(nb);
    E *sA = reinterpret_cast<E *>(smem + Sh::OFF_KW);
    float *sAtd = reinterpret_cast<float *>(smem + Sh::OFF_KW + Sh::A_BYTES);
    float *sTd = reinterpret_cast<float *>(smem + Sh::OFF_KW + Sh::A_BYTES + Sh::ATD_BYTES);
    const int nrow = min(C, len - c * C);
    const size_t tok0 = row0 + (size_t)c * C;

    // K straight into MFMA operand layout; copy to LDS for the scan waves
    Op kop[NB][KSTEPS];
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      const int r = 16 * rt + li;
#pragma unroll
      for (int kq = 0; kq < KSTEPS; ++kq) {
        const int col = kq * KSTEP + lg * VPL;
        kop[rt][kq] = (r < nrow) ? M::ldg(gk + (tok0 + r) * DK + col) : M::zero();
        M::st(sK + r * LDK + col, kop[rt][kq]);
      }
    }
    // fused ||k_r||^2: lane holds a quarter of row 16rt + li
    float nrm[NB];
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      float s = 0.f;
#pragma unroll
      for (int kq = 0; kq < KSTEPS; ++kq) s += M::sumsq(kop[rt][kq]);
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      nrm[rt] = s;
    }
    float my_nrm = nrm[0];
#pragma unroll
    for (int rt = 1; rt < NB; ++rt)
      if (lg == rt) my_nrm = nrm[rt];
    float gdummy;
    const float gam = gate_scan(nrow, tok0, gdummy);
    float etav = 0.f;
    if (lane < nrow) etav = Elem<E>::to_f32(geta[tok0 + lane]);
    // beta of rows beyond the sequence end is 0 (not 0/0 when eps = 0)
    const float beta = (lane < nrow) ? etav / (my_nrm + p.eps) : 0.f;
    const float gamC = __shfl(gam, C - 1);
    if (lane < C) {
      sF[lane] = __expf(gam);             // Gam_r
      sF[C + lane] = __expf(gamC - gam);  // d_r
    }

    // Gram tiles K K^T (lower, incl. diagonal) and A
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
      for (int st = 0; st <= rt; ++st) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kq = 0; kq < KSTEPS; ++kq) acc = M::mma(kop[rt][kq], kop[st][kq], acc);
        const int s = 16 * st + li;
        const float gs = __shfl(gam, s);
        f32x4 av;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * rt + 4 * lg + j;
          const float gr = __shfl(gam, r);
          const float br = __shfl(beta, r);
          const float dec = (r > s) ? __expf(gr - gs) : 0.f;
          av[j] = (r > s) ? br * acc[j] * dec : 0.f;
        }
        if (st < rt) {
#pragma unroll
          for (int j = 0; j < 4; ++j) sA[(16 * rt + 4 * lg + j) * LDC + s] = Elem<E>::from_f32(av[j]);
        } else {
          // diagonal block, stored transposed: At[s'][r']
          *reinterpret_cast<f32x4 *>(sAtd + rt * 16 * LDD + li * LDD + 4 * lg) = av;
        }
      }
    }

    // diagonal blocks of T = (I + A)^-1: lane = (block lg, column li)
    float x[16];
    if (lg < NB) {
      const float *At = sAtd + lg * 16 * LDD;
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = (r == li) ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < 15; ++s) {
        f32x4 col[4];
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          if (4 * qd + 3 > s) col[qd] = *reinterpret_cast<const f32x4 *>(At + s * LDD + 4 * qd);
#pragma unroll
        for (int r = s + 1; r < 16; ++r) x[r] = fmaf(-col[r >> 2][r & 3], x[s], x[r]);
      }
      float *Td = sTd + lg * 16 * LDD;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        Td[r * LDD + li] = x[r];
        // T' = T Diag(beta): column 16 lg + li scaled by that row's beta (= this lane's)
        sTp[(16 * lg + r) * LDC + 16 * lg + li] = Elem<E>::from_f32(x[r] * beta);
      }
    }

    // off-diagonal blocks, level by level: T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj
    if constexpr (NB > 1) {
      f32x4 Toff[NB][NB];
#pragma unroll
      for (int dist = 1; dist < NB; ++dist) {
#pragma unroll
        for (int i = dist; i < NB; ++i) {
          const int j = i - dist;
          f32x4 y = zero4();
#pragma unroll
          for (int m = j; m < i; ++m) {
            float a[4], bb[4];
            const f32x4 a4 = load4(sA + (16 * i + li) * LDC + 16 * m + 4 * lg);
#pragma unroll
            for (int e = 0; e < 4; ++e) a[e] = a4[e];
            if (m == j) {
#pragma unroll
              for (int e = 0; e < 4; ++e) bb[e] = sTd[j * 16 * LDD + (4 * lg + e) * LDD + li];
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) bb[e] = Toff[m][j][e];
            }
            y = Mm16<E>::mma(a, bb, y);
          }
          float a[4], bb[4];
          const f32x4 t4 = *reinterpret_cast<const f32x4 *>(sTd + i * 16 * LDD + li * LDD + 4 * lg);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a[e] = t4[e];
            bb[e] = y[e];
          }
          const f32x4 t = Mm16<E>::mma(a, bb, zero4());
          Toff[i][j] = -t;
          const float bs = __shfl(beta, 16 * j + li);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sTp[(16 * i + 4 * lg + e) * LDC + 16 * j + li] = Elem<E>::from_f32(-t[e] * bs);
        }
      }
    }
  };

  // ======================= Q wave: chunk c -> buffer nb ======================
  auto produce_q = [&](int c, int nb) {
    E *sQ = bufE(nb) + Sh::OFF_Q;
    E *sVt = bufE(nb) + Sh::OFF_VT;
    E *sP = bufE(nb) + Sh::OFF_P;
    const int nrow = min(C, len - c * C);
    const size_t tok0 = row0 + (size_t)c * C;

    Op qop[NB][KSTEPS], kop[NB][KSTEPS];
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      const int r = 16 * rt + li;
#pragma unroll
      for (int kq = 0; kq < KSTEPS; ++kq) {
        const int col = kq * KSTEP + lg * VPL;
        const bool ok = r < nrow;
        qop[rt][kq] = ok ? M::ldg(gq + (tok0 + r) * DK + col) : M::zero();
        kop[rt][kq] = ok ? M::ldg(gk + (tok0 + r) * DK + col) : M::zero();
        M::st(sQ + r * LDK + col, qop[rt][kq]);
      }
    }
    // V slice [C x DVT] -> V^T in LDS, 16-byte loads
    constexpr int V16 = 16 / (int)sizeof(E);
    constexpr int PPR = DVT / V16;  // 16-byte pieces per row
    const size_t vcol0 = (size_t)jt * DVT;
    for (int pc = lane; pc < C * PPR; pc += 64) {
      const int r = pc / PPR, cq = pc % PPR;
      uint4 u = make_uint4(0u, 0u, 0u, 0u);
      if (r < nrow) u = ldg16(gv + (tok0 + r) * (size_t)dv + vcol0 + cq * V16);
      const E *ve = reinterpret_cast<const E *>(&u);
#pragma unroll
      for (int x = 0; x < V16; ++x) sVt[(cq * V16 + x) * LDC + r] = ve[x];
    }
    float gdummy;
    const float gam = gate_scan(nrow, tok0, gdummy);
    // causal scores P = (Q K^T) weighted by exp(gamma_r - gamma_s), r >= s
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
      for (int st = 0; st <= rt; ++st) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kq = 0; kq < KSTEPS; ++kq) acc = M::mma(qop[rt][kq], kop[st][kq], acc);
        const int s = 16 * st + li;
        const float gs = __shfl(gam, s);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * rt + 4 * lg + j;
          const float gr = __shfl(gam, r);
          const float val = (r >= s) ? acc[j] * __expf(gr - gs) : 0.f;
          sP[r * LDC + s] = Elem<E>::from_f32(val);
        }
      }
    }
  };

  // ======================= scan waves =======================================
  f32x4 accS[DK / 16];
  E *sSt = reinterpret_cast<E *>(smem + Sh::OFF_SW + wave * Sh::SCAN_BYTES);
  E *sXt = sSt + 16 * LDK;
  E *sUt = sXt + 16 * LDC;
  E *sdUt = sUt + 16 * LDC;
  const int col = jt * DVT + 16 * wave + li;  // this lane's state column
  const size_t sbase = (size_t)nh * DK * (size_t)dv;

  auto consume = [&](int c, int cur) {
    const E *sK = bufE(cur) + Sh::OFF_K;
    const E *sQ = bufE(cur) + Sh::OFF_Q;
    const E *sVt = bufE(cur) + Sh::OFF_VT;
    const E *sTp = bufE(cur) + Sh::OFF_TP;
    const E *sP = bufE(cur) + Sh::OFF_P;
    const float *sGam = bufF(cur);
    const float *sD = bufF(cur) + C;

    // K S and Q S
    f32x4 accK[NB], accQ[NB];
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) accK[rt] = accQ[rt] = zero4();
#pragma unroll
    for (int kq = 0; kq < KSTEPS; ++kq) {
      const int kc = kq * KSTEP + lg * VPL;
      const Op bs = M::ld(sSt + li * LDK + kc);
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        accK[rt] = M::mma(M::ld(sK + (16 * rt + li) * LDK + kc), bs, accK[rt]);
        accQ[rt] = M::mma(M::ld(sQ + (16 * rt + li) * LDK + kc), bs, accQ[rt]);
      }
    }
    // X = V - Diag(Gam) K S  (to LDS, transposed);  O starts as Diag(Gam) Q S
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      const int r0 = 16 * rt + 4 * lg;
      const f32x4 gm = *reinterpret_cast<const f32x4 *>(sGam + r0);
      const f32x4 vv = load4(sVt + (16 * wave + li) * LDC + r0);
      f32x4 xv;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xv[j] = vv[j] - gm[j] * accK[rt][j];
        accQ[rt][j] *= gm[j];
      }
      store4(sXt + li * LDC + r0, xv);
    }
    // U~ = T' X   (T' lower triangular: skip zero blocks)
    f32x4 accU[NB];
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      accU[rt] = zero4();
#pragma unroll
      for (int kb = 0; kb < 16 * (rt + 1); kb += KSTEP) {
        const int kc = kb + lg * VPL;
        accU[rt] = M::mma(M::ld(sTp + (16 * rt + li) * LDC + kc), M::ld(sXt + li * LDC + kc), accU[rt]);
      }
    }
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      const int r0 = 16 * rt + 4 * lg;
      const f32x4 dd = *reinterpret_cast<const f32x4 *>(sD + r0);
      store4(sUt + li * LDC + r0, accU[rt]);
      f32x4 du;
#pragma unroll
      for (int j = 0; j < 4; ++j) du[j] = dd[j] * accU[rt][j];
      store4(sdUt + li * LDC + r0, du);
    }
    // O += P U~ ; write the valid rows
    const int nrow = min(C, len - c * C);
    const size_t tok0 = row0 + (size_t)c * C;
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
      for (int kb = 0; kb < 16 * (rt + 1); kb += KSTEP) {
        const int kc = kb + lg * VPL;
        accQ[rt] = M::mma(M::ld(sP + (16 * rt + li) * LDC + kc), M::ld(sUt + li * LDC + kc), accQ[rt]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * rt + 4 * lg + j;
        if (r < nrow) go[(tok0 + r) * (size_t)dv + col] = Elem<E>::from_f32(accQ[rt][j]);
      }
    }
    // S <- Gam_C S + K^T Diag(d) U~
    const float gC = sGam[C - 1];
#pragma unroll
    for (int it = 0; it < DK / 16; ++it) {
#pragma unroll
      for (int j = 0; j < 4; ++j) accS[it][j] *= gC;
#pragma unroll
      for (int kb = 0; kb < C; kb += KSTEP) {
        const int kc = kb + lg * VPL;
        accS[it] = M::mma(M::ld_strided(sK + kc * LDK + 16 * it + li, LDK), M::ld(sdUt + li * LDC + kc), accS[it]);
      }
      store4(sSt + li * LDK + 16 * it + 4 * lg, accS[it]);
    }
  };

  // ---- prologue -----------------------------------------------------------
  if (wave < NBW) {
#pragma unroll
    for (int it = 0; it < DK / 16; ++it) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * it + 4 * lg + j;
        accS[it][j] = p.s0 ? p.s0[sbase + (size_t)r * dv + col] : 0.f;
      }
      store4(sSt + li * LDK + 16 * it + 4 * lg, accS[it]);
    }
  } else if (nch > 0) {
    if (wave == NBW) produce_k(0, 0);
    else produce_q(0, 0);
  }
  __syncthreads();

  // ---- chunk loop: scan chunk c while chunk c+1 is being prepared ----------
  for (int c = 0; c < nch; ++c) {
    const int cur = c & 1;
    if (wave < NBW) {
      consume(c, cur);
    } else if (c + 1 < nch) {
      if (wave == NBW) produce_k(c + 1, cur ^ 1);
      else produce_q(c + 1, cur ^ 1);
    }
    __syncthreads();
  }

  // ---- final state ----------------------------------------------------------
  if (wave < NBW && p.sfin) {
#pragma unroll
    for (int it = 0; it < DK / 16; ++it) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * it + 4 * lg + j;
        p.sfin[sbase + (size_t)r * dv + col] = accS[it][j];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------
template <typename E, int C, int DK, int NBW>
static hipError_t launch_chunk_t(const ChunkArgs &a, hipStream_t st) {
  using Sh = ChunkShape<E, C, DK, NBW>;
  ChunkParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.g = a.g;
  p.eta = a.eta;
  p.eps = a.eps;
  p.s0 = a.initial_state;
  p.o = a.o;
  p.sfin = a.final_state;
  p.cu = a.cu_seqlens;
  p.H = a.H;
  p.T = a.T;
  p.dv = a.dv;
  p.n_tiles = a.dv / Sh::DVT;
  const long long nblk = (long long)a.num_seqs * a.H * p.n_tiles;
  p.remap = (nblk % 8 == 0) ? 1 : 0;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL((kla_chunk_kernel<E, C, DK, NBW>), dim3((unsigned)nblk), dim3(Sh::NT), 0, st, p);
  return hipGetLastError();
}

bool chunk_supported(int dtype, int dk, int dv, int chunk) {
  if (dtype == 0) {
    return chunk == 64 && (dk == 64 || dk == 128) && dv % 16 == 0 && dv >= 16 && dv <= 256;
  }
  if (dtype == 1) {
    if (dv % 16 != 0 || dv < 16 || dv > 256) return false;
    if (chunk == 16) return dk == 16 || dk == 32 || dk == 64 || dk == 128;
    if (chunk == 64) return dk == 16 || dk == 32;
  }
  return false;
}

// Column slice width: 32 columns (2 scan waves) when that still gives at
// least one workgroup per CU, else 16 (more workgroups, more redundant
// S-independent work per column).
static bool use_two_scan_waves(const ChunkArgs &a) {
  return a.dv % 32 == 0 && (long long)a.num_seqs * a.H * (a.dv / 32) >= 256;
}

hipError_t launch_chunk_fwd(const ChunkArgs &a, hipStream_t st) {
  if (a.dtype == 0) {
    const bool two = use_two_scan_waves(a);
    if (a.dk == 128) return two ? launch_chunk_t<bf16, 64, 128, 2>(a, st) : launch_chunk_t<bf16, 64, 128, 1>(a, st);
    if (a.dk == 64) return two ? launch_chunk_t<bf16, 64, 64, 2>(a, st) : launch_chunk_t<bf16, 64, 64, 1>(a, st);
    return hipErrorInvalidValue;
  }
  if (a.chunk == 16) {
    switch (a.dk) {
      case 16: return launch_chunk_t<float, 16, 16, 1>(a, st);
      case 32: return launch_chunk_t<float, 16, 32, 1>(a, st);
      case 64: return launch_chunk_t<float, 16, 64, 1>(a, st);
      case 128: return launch_chunk_t<float, 16, 128, 1>(a, st);
    }
  } else if (a.chunk == 64) {
    switch (a.dk) {
      case 16: return launch_chunk_t<float, 64, 16, 1>(a, st);
      case 32: return launch_chunk_t<float, 64, 32, 1>(a, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace kla
