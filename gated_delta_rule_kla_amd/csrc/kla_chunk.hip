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
// state slice never leaves the chip: it lives in MFMA accumulators of the NBW
// "scan" waves (16 columns each, fp32) for the whole sequence.  Two
// "producer" waves build the S-independent data of chunk c+1 while the scan
// waves consume chunk c (double-buffered LDS, one barrier per chunk):
//   * the K wave: K (16-byte loads straight into MFMA operand layout,
//     prefetched one chunk ahead), the fused ||k||^2 reduction and beta, the
//     gate scan, K K^T on MFMA, A, and the 64x64 unit-lower-triangular solve
//     done blockwise: the four 16x16 diagonal blocks by column-parallel
//     forward substitution in fp32 (lane = block x column), the off-diagonal
//     blocks by 16x16x16 MFMA products T_ij = -T_ii sum_m A_im T_mj;
//   * the Q wave: Q and the V slice, Q K^T on MFMA and the causal tile P.
// The scan waves never round-trip their own data through LDS: every right
// operand (S, X, U~, Diag(d) U~) is fed to the next MFMA straight from the
// accumulator registers, by ordering each instruction's contraction index
// the way the accumulator layout holds it (see Ops below).  The matching left
// operands (K, Q, T', P rows) are stored by the producers with their columns
// permuted into that order, so each is one 16-byte LDS read; K^T and the V
// slice are read from row-major tiles with gfx950's transposing LDS read.
#include "kla_common.h"
#include "kla_internal.h"

namespace kla {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// ---------------------------------------------------------------------------
// Operand machinery.  MFMA conventions (16x16 output tile D, fp32):
//   D: lane l holds D[4(l>>4) + j][l&15], j < 4.
//   A operand: lane l supplies row (l&15) of the left matrix; B operand: lane
//   l supplies column (l&15) of the right matrix; the contraction slots are
//   paired across A and B by (lane group l>>4, slot).
// "Natural" products (producer waves): slot x of lane group g <-> contraction
// index kb + VPL g + x, both operands read row-contiguous.
// "Grouped" products (scan waves): a group of KG contraction rows; slot x of
// lane group g <-> row kb + 16(x>>2) + 4g + (x&3) (bf16: two D tiles per
// group) or kb + 4g + x over four MFMAs (fp32: one D tile per group).  This is
// exactly how a D tile is held, so D tiles are B operands as they stand.
// ---------------------------------------------------------------------------
template <typename E> struct Ops;

template <> struct Ops<bf16> {
  static constexpr int KSTEP = 32, VPL = 8;  // natural: v_mfma_f32_16x16x32_bf16
  static constexpr int KG = 32;               // grouped: rows per group
  typedef bf16x8 Nat;
  typedef bf16x8 Grp;
  static __device__ __forceinline__ f32x4 mma(Nat a, Nat b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma_grp(Grp a, Grp b, f32x4 c) { return mma(a, b, c); }
  static __device__ __forceinline__ Nat ldg(const bf16 *p) { return __builtin_bit_cast(Nat, ldg16(p)); }
  static __device__ __forceinline__ Nat zero() {
    Nat r;
#pragma unroll
    for (int x = 0; x < 8; ++x) r[x] = (bf16)0.f;
    return r;
  }
  static __device__ __forceinline__ float sumsq(Nat v) {
    float s = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) s = fmaf((float)v[x], (float)v[x], s);
    return s;
  }
  // column position inside a row stored in grouped order: inside each block of
  // 32 columns, column 16h + 4g + e is stored at 8g + 4h + e
  static __device__ __forceinline__ int perm(int c) {
    return (c & ~31) | (((c >> 2) & 3) << 3) | (((c >> 4) & 1) << 2) | (c & 3);
  }
  // store a natural operand (columns kq*32 + 8g .. +7 of one row) into a grouped row
  static __device__ __forceinline__ void st_nat(bf16 *row, int kq, int g, Nat v) {
    const int c0 = kq * 32 + 8 * g;
    const bf16x4 lo = {v[0], v[1], v[2], v[3]}, hi = {v[4], v[5], v[6], v[7]};
    *reinterpret_cast<bf16x4 *>(row + perm(c0)) = lo;
    *reinterpret_cast<bf16x4 *>(row + perm(c0 + 4)) = hi;
  }
  // B group from the D tiles of rows kb..kb+31
  static __device__ __forceinline__ Grp b_from_d(const f32x4 *d) {
    Grp r;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      r[x] = (bf16)d[0][x];
      r[4 + x] = (bf16)d[1][x];
    }
    return r;
  }
  // A group of a grouped-stored row
  static __device__ __forceinline__ Grp a_row(const bf16 *row, int kb, int g) {
    return *reinterpret_cast<const bf16x8 *>(row + kb + 8 * g);
  }
  // A group of M^T: rows c16 + (l&15) of M^T, contraction rows kb..kb+31 of M,
  // from M stored row-major (grouped columns) -- two transposing LDS reads
  static __device__ __forceinline__ Grp a_trans(const bf16 *M, int ld, int kb, int c16, int lane) {
    const int g = lane >> 4, x = (lane >> 2) & 3, a = lane & 3;
    const bf16 *p0 = M + (kb + 4 * g + x) * ld + perm(c16 + 4 * a);
    const bf16 *p1 = p0 + 16 * ld;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p0);
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p1);
    return Grp{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  // D-layout tile column: M[r16 + 4g + j][c0 + (l&15)], j < 4, M row-major natural
  static __device__ __forceinline__ f32x4 col4(const bf16 *M, int ld, int r16, int c0, int lane) {
    const int g = lane >> 4, x = (lane >> 2) & 3, a = lane & 3;
    const bf16x4 v =
        __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(M + (r16 + 4 * g + x) * ld + c0 + 4 * a));
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
  }
};

template <> struct Ops<float> {
  static constexpr int KSTEP = 4, VPL = 1;   // natural: v_mfma_f32_16x16x4_f32
  static constexpr int KG = 16;
  typedef float Nat;
  typedef f32x4 Grp;
  static __device__ __forceinline__ f32x4 mma(Nat a, Nat b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma_grp(Grp a, Grp b, f32x4 c) {
#pragma unroll
    for (int x = 0; x < 4; ++x) c = mma(a[x], b[x], c);
    return c;
  }
  static __device__ __forceinline__ Nat ldg(const float *p) { return *p; }
  static __device__ __forceinline__ Nat zero() { return 0.f; }
  static __device__ __forceinline__ float sumsq(Nat v) { return v * v; }
  static __device__ __forceinline__ int perm(int c) { return c; }
  static __device__ __forceinline__ void st_nat(float *row, int kq, int g, Nat v) { row[kq * 4 + g] = v; }
  static __device__ __forceinline__ Grp b_from_d(const f32x4 *d) { return d[0]; }
  static __device__ __forceinline__ Grp a_row(const float *row, int kb, int g) {
    return *reinterpret_cast<const f32x4 *>(row + kb + 4 * g);
  }
  static __device__ __forceinline__ Grp a_trans(const float *M, int ld, int kb, int c16, int lane) {
    const int g = lane >> 4, li = lane & 15;
    Grp r;
#pragma unroll
    for (int x = 0; x < 4; ++x) r[x] = M[(kb + 4 * g + x) * ld + c16 + li];
    return r;
  }
  static __device__ __forceinline__ f32x4 col4(const float *M, int ld, int r16, int c0, int lane) {
    const int g = lane >> 4, li = lane & 15;
    f32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = M[(r16 + 4 * g + j) * ld + c0 + li];
    return r;
  }
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

__device__ __forceinline__ f32x4 load4(const bf16 *p) {
  bf16x4 b = *reinterpret_cast<const bf16x4 *>(p);
  return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
}
__device__ __forceinline__ f32x4 load4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele with DPP
// row shifts inside each 16-lane row, then the row totals via readlane.
template <int CTRL>
__device__ __forceinline__ float dpp_row_shr(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_value(float v, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), src));
}
__device__ __forceinline__ float wave_inclusive_scan(float v) {
  v += dpp_row_shr<0x111>(v);  // row_shr:1
  v += dpp_row_shr<0x112>(v);  // row_shr:2
  v += dpp_row_shr<0x114>(v);  // row_shr:4
  v += dpp_row_shr<0x118>(v);  // row_shr:8
  const float r0 = lane_value(v, 15), r1 = lane_value(v, 31), r2 = lane_value(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  v += (row >= 1 ? r0 : 0.f) + (row >= 2 ? r1 : 0.f) + (row >= 3 ? r2 : 0.f);
  return v;
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS accesses,
// then s_barrier.  Global loads issued before it stay in flight (the chunk
// loop prefetches the next chunk's inputs across it); no wave reads another
// wave's global-memory writes, so no global fence is needed.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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
  static constexpr int LDK = DK + PAD;        // pitch of K and Q rows (grouped columns)
  static constexpr int LDC = C + PAD;         // pitch of T' and P rows (grouped columns) and of A
  static constexpr int LDV = DVT + PAD;       // pitch of V slice rows (natural)
  static constexpr int LDD = 20;              // fp32 pitch of 16-wide diagonal blocks
  static constexpr int KSTEPS = DK / Ops<E>::KSTEP;
  // shared double buffer (elements of E, then floats)
  static constexpr int OFF_K = 0;
  static constexpr int OFF_Q = OFF_K + C * LDK;
  static constexpr int OFF_V = OFF_Q + C * LDK;
  static constexpr int OFF_TP = OFF_V + C * LDV;
  static constexpr int OFF_P = OFF_TP + C * LDC;
  static constexpr int BUF_E = OFF_P + C * LDC;
  static constexpr int BUF_F = 2 * C;         // Gam[C], d[C]
  static constexpr int BUF_BYTES = BUF_E * (int)sizeof(E) + BUF_F * 4;
  // K wave private
  static constexpr int A_BYTES = C * LDC * (int)sizeof(E);       // A, row-major (natural), E
  static constexpr int ATD_BYTES = NB * 16 * LDD * 4;            // A diagonal blocks, transposed, fp32
  static constexpr int TD_BYTES = NB * 16 * LDD * 4;             // T diagonal blocks, fp32
  // producer waves' private per-row vectors: K wave gamma[C], beta[C],
  // norm partials [NB][4][16]; Q wave gamma[C]
  static constexpr int VEC_BYTES = (3 * C + NB * 64) * 4;
  // scan wave private: O^T staging (16 columns x C rows) for row-contiguous stores
  static constexpr int OT_BYTES = 16 * LDC * (int)sizeof(E);
  static constexpr int OFF_KW = 2 * BUF_BYTES;
  static constexpr int OFF_VEC = OFF_KW + A_BYTES + ATD_BYTES + TD_BYTES;
  static constexpr int OFF_OT = OFF_VEC + VEC_BYTES;
  static constexpr int BYTES = OFF_OT + NBW * OT_BYTES;

  static_assert(C == 16 || C == 64, "chunk");
  static_assert(C % Ops<E>::KG == 0 && DK % Ops<E>::KG == 0 && DK % Ops<E>::KSTEP == 0, "dk");
  static_assert(BUF_BYTES % 16 == 0 && A_BYTES % 16 == 0 && VEC_BYTES % 16 == 0 && OT_BYTES % 16 == 0,
                "lds align");
  static_assert((LDK * (int)sizeof(E)) % 16 == 0 && (LDC * (int)sizeof(E)) % 16 == 0 &&
                    (LDV * (int)sizeof(E)) % 16 == 0, "row align");
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
  using O = Ops<E>;
  using Nat = typename O::Nat;
  using Grp = typename O::Grp;
  constexpr int NB = Sh::NB, DVT = Sh::DVT, LDK = Sh::LDK, LDC = Sh::LDC, LDV = Sh::LDV, LDD = Sh::LDD;
  constexpr int KSTEP = O::KSTEP, VPL = O::VPL, KSTEPS = Sh::KSTEPS, KG = O::KG, TPG = KG / 16;

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
      bufE(bi)[Sh::OFF_TP + rr * LDC + O::perm(ss)] = Elem<E>::from_f32(0.f);
      bufE(bi)[Sh::OFF_P + rr * LDC + O::perm(ss)] = Elem<E>::from_f32(0.f);
    }
  }

  // ---- per-row vectors of the producer waves (private LDS) -------------------
  float *sGamK = reinterpret_cast<float *>(smem + Sh::OFF_VEC);
  float *sBetaK = sGamK + C;
  float *sNrmK = sGamK + 2 * C;
  float *sGamQ = sNrmK + NB * 64;

  if (wave < NBW) {
    // ======================= scan wave: 16 state columns =====================
    f32x4 accS[DK / 16];
    const int col0 = jt * DVT + 16 * wave;     // first of this wave's 16 state columns
    const int col = col0 + li;                  // this lane's state column
    E *sOt = reinterpret_cast<E *>(smem + Sh::OFF_OT + wave * Sh::OT_BYTES);
    const size_t sbase = (size_t)nh * DK * (size_t)dv;
#pragma unroll
    for (int it = 0; it < DK / 16; ++it) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * it + 4 * lg + j;
        accS[it][j] = p.s0 ? p.s0[sbase + (size_t)r * dv + col] : 0.f;
      }
    }
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
      const int cur = c & 1;
      const E *sK = bufE(cur) + Sh::OFF_K;
      const E *sQ = bufE(cur) + Sh::OFF_Q;
      const E *sV = bufE(cur) + Sh::OFF_V;
      const E *sTp = bufE(cur) + Sh::OFF_TP;
      const E *sP = bufE(cur) + Sh::OFF_P;
      const float *sGam = bufF(cur);
      const float *sD = bufF(cur) + C;

      // Every S-independent left operand of this chunk is read up front, so the
      // LDS latency overlaps the MFMA chain instead of stalling each step.
      Grp kA[NB][DK / KG], qA[NB][DK / KG];
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
        for (int q = 0; q < DK / KG; ++q) {
          kA[rt][q] = O::a_row(sK + (16 * rt + li) * LDK, q * KG, lg);
          qA[rt][q] = O::a_row(sQ + (16 * rt + li) * LDK, q * KG, lg);
        }
      }
      f32x4 gm[NB], dd[NB], vv[NB];
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        gm[rt] = *reinterpret_cast<const f32x4 *>(sGam + 16 * rt + 4 * lg);
        dd[rt] = *reinterpret_cast<const f32x4 *>(sD + 16 * rt + 4 * lg);
        vv[rt] = O::col4(sV, LDV, 16 * rt, 16 * wave, lane);
      }
      Grp tA[NB][C / KG], pA[NB][C / KG];
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
        for (int q = 0; q * KG < 16 * (rt + 1); ++q) {
          tA[rt][q] = O::a_row(sTp + (16 * rt + li) * LDC, q * KG, lg);
          pA[rt][q] = O::a_row(sP + (16 * rt + li) * LDC, q * KG, lg);
        }
      }
      Grp ktA[DK / 16][C / KG];
#pragma unroll
      for (int it = 0; it < DK / 16; ++it) {
#pragma unroll
        for (int q = 0; q < C / KG; ++q) ktA[it][q] = O::a_trans(sK, LDK, q * KG, 16 * it, lane);
      }
      const float gC = sGam[C - 1];

      // S as right operands, straight from the accumulators
      Grp sb[DK / KG];
#pragma unroll
      for (int q = 0; q < DK / KG; ++q) sb[q] = O::b_from_d(&accS[q * TPG]);
      // K S and Q S
      f32x4 aK[NB], aQ[NB];
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        aK[rt] = aQ[rt] = zero4();
#pragma unroll
        for (int q = 0; q < DK / KG; ++q) {
          aK[rt] = O::mma_grp(kA[rt][q], sb[q], aK[rt]);
          aQ[rt] = O::mma_grp(qA[rt][q], sb[q], aQ[rt]);
        }
      }
      // X = V - Diag(Gam) K S;  O starts as Diag(Gam) Q S
      f32x4 xv[NB];
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        xv[rt] = vv[rt] - gm[rt] * aK[rt];
        aQ[rt] = gm[rt] * aQ[rt];
      }
      Grp xb[C / KG];
#pragma unroll
      for (int q = 0; q < C / KG; ++q) xb[q] = O::b_from_d(&xv[q * TPG]);
      // U~ = T' X   (T' lower triangular: skip the zero groups)
      f32x4 u[NB], du[NB];
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        u[rt] = zero4();
#pragma unroll
        for (int q = 0; q * KG < 16 * (rt + 1); ++q) u[rt] = O::mma_grp(tA[rt][q], xb[q], u[rt]);
        du[rt] = dd[rt] * u[rt];
      }
      Grp ub[C / KG], dub[C / KG];
#pragma unroll
      for (int q = 0; q < C / KG; ++q) {
        ub[q] = O::b_from_d(&u[q * TPG]);
        dub[q] = O::b_from_d(&du[q * TPG]);
      }
      // S <- Gam_C S + K^T Diag(d) U~   (issued before O: it is the chain)
#pragma unroll
      for (int it = 0; it < DK / 16; ++it) {
        accS[it] = gC * accS[it];
#pragma unroll
        for (int q = 0; q < C / KG; ++q) accS[it] = O::mma_grp(ktA[it][q], dub[q], accS[it]);
      }
      // O += P U~ ; write the valid rows
      const int nrow = min(C, len - c * C);
      const size_t tok0 = row0 + (size_t)c * C;
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
        for (int q = 0; q * KG < 16 * (rt + 1); ++q) aQ[rt] = O::mma_grp(pA[rt][q], ub[q], aQ[rt]);
      }
      if constexpr (sizeof(E) == 2) {
        // stage O^T (4 rows of one column per lane = one 8-byte write), read it
        // back transposed (4 columns of one row per lane) and store 8 bytes
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) {
          bf16x4 ob;
#pragma unroll
          for (int j = 0; j < 4; ++j) ob[j] = (bf16)aQ[rt][j];
          *reinterpret_cast<bf16x4 *>(sOt + li * LDC + 16 * rt + 4 * lg) = ob;
        }
        const int x = (lane >> 2) & 3, a = lane & 3;
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) {
          const bf16x4 rowv =
              __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(sOt + (4 * lg + x) * LDC + 16 * rt + 4 * a));
          const int r = 16 * rt + li;
          if (r < nrow) *reinterpret_cast<bf16x4 *>(go + (tok0 + r) * (size_t)dv + col0 + 4 * lg) = rowv;
        }
      } else {
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 16 * rt + 4 * lg + j;
            if (r < nrow) go[(tok0 + r) * (size_t)dv + col] = Elem<E>::from_f32(aQ[rt][j]);
          }
        }
      }
      lds_barrier();
    }
    if (p.sfin) {
#pragma unroll
      for (int it = 0; it < DK / 16; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * it + 4 * lg + j;
          p.sfin[sbase + (size_t)r * dv + col] = accS[it][j];
        }
      }
    }
  } else if (wave == NBW) {
    // ======================= K wave ==========================================
    // The chunk's raw inputs are fetched one chunk ahead into registers: the
    // loads for chunk c+1 are issued at the end of producing chunk c and land
    // while the wave waits at the barrier.  Rows past the sequence end load a
    // clamped (valid) row and are zeroed after arrival.
    Nat kop[NB][KSTEPS];
    E kg_raw = Elem<E>::from_f32(0.f), ke_raw = Elem<E>::from_f32(0.f);
    auto fetch = [&](int c) {
      const int nrow = min(C, len - c * C);
      const size_t tok0 = row0 + (size_t)c * C;
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const int r = min(16 * rt + li, nrow - 1);
#pragma unroll
        for (int kq = 0; kq < KSTEPS; ++kq) kop[rt][kq] = O::ldg(gk + (tok0 + r) * DK + kq * KSTEP + lg * VPL);
      }
      const int lr = min(lane, nrow - 1);
      kg_raw = gg[tok0 + lr];
      ke_raw = geta[tok0 + lr];
    };
    E *sA = reinterpret_cast<E *>(smem + Sh::OFF_KW);
    float *sAtd = reinterpret_cast<float *>(smem + Sh::OFF_KW + Sh::A_BYTES);
    float *sTd = reinterpret_cast<float *>(smem + Sh::OFF_KW + Sh::A_BYTES + Sh::ATD_BYTES);

    auto produce = [&](int c, int nb) {
      E *sK = bufE(nb) + Sh::OFF_K;
      E *sTp = bufE(nb) + Sh::OFF_TP;
      float *sF = bufF(nb);
      const int nrow = min(C, len - c * C);
      // K rows to LDS (grouped columns) for the scan waves
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const int r = 16 * rt + li;
#pragma unroll
        for (int kq = 0; kq < KSTEPS; ++kq) {
          if (r >= nrow) kop[rt][kq] = O::zero();
          O::st_nat(sK + r * LDK, kq, lg, kop[rt][kq]);
        }
      }
      // fused ||k_r||^2: lane holds a quarter of row 16rt + li; the four
      // quarters are summed through LDS by lane r
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        float sq = 0.f;
#pragma unroll
        for (int kq = 0; kq < KSTEPS; ++kq) sq += O::sumsq(kop[rt][kq]);
        sNrmK[(rt * 4 + lg) * 16 + li] = sq;
      }
      const float gam = wave_inclusive_scan((lane < nrow) ? Elem<E>::to_f32(kg_raw) : 0.f);
      float nr = 0.f;
      if (lane < C) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) nr += sNrmK[((lane >> 4) * 4 + q4) * 16 + li];
      }
      // beta of rows beyond the sequence end is 0 (not 0/0 when eps = 0)
      const float beta = (lane < nrow) ? Elem<E>::to_f32(ke_raw) / (nr + p.eps) : 0.f;
      const float gamC = lane_value(gam, C - 1);
      if (lane < C) {
        sGamK[lane] = gam;
        sBetaK[lane] = beta;
        sF[lane] = __expf(gam);             // Gam_r
        sF[C + lane] = __expf(gamC - gam);  // d_r
      }
      // per-lane row (r = 16 rt + 4 lg + j) and column (s = 16 st + li) gate values
      f32x4 gr4[NB], br4[NB];
      float gs1[NB];
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        gr4[rt] = *reinterpret_cast<const f32x4 *>(sGamK + 16 * rt + 4 * lg);
        br4[rt] = *reinterpret_cast<const f32x4 *>(sBetaK + 16 * rt + 4 * lg);
        gs1[rt] = sGamK[16 * rt + li];
      }
      // Gram tiles K K^T (lower, incl. diagonal) and A
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
        for (int st = 0; st <= rt; ++st) {
          f32x4 acc = zero4();
#pragma unroll
          for (int kq = 0; kq < KSTEPS; ++kq) acc = O::mma(kop[rt][kq], kop[st][kq], acc);
          const int s = 16 * st + li;
          f32x4 av;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 16 * rt + 4 * lg + j;
            const float dec = (r > s) ? __expf(gr4[rt][j] - gs1[st]) : 0.f;
            av[j] = (r > s) ? br4[rt][j] * acc[j] * dec : 0.f;
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
      // diagonal blocks of T = (I + A)^-1: lane = (block lg, column li);
      // the block (stored transposed) is read whole before the substitution
      if (lg < NB) {
        float x[16];
        f32x4 at[16][4];
        const float *At = sAtd + lg * 16 * LDD;
#pragma unroll
        for (int s = 0; s < 15; ++s)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd)
            if (4 * qd + 3 > s) at[s][qd] = *reinterpret_cast<const f32x4 *>(At + s * LDD + 4 * qd);
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == li) ? 1.f : 0.f;
#pragma unroll
        for (int s = 0; s < 15; ++s) {
#pragma unroll
          for (int r = s + 1; r < 16; ++r) x[r] = fmaf(-at[s][r >> 2][r & 3], x[s], x[r]);
        }
        float *Td = sTd + lg * 16 * LDD;
        const int pc = O::perm(16 * lg + li);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          Td[r * LDD + li] = x[r];
          // T' = T Diag(beta): column 16 lg + li scaled by that row's beta (= this lane's)
          sTp[(16 * lg + r) * LDC + pc] = Elem<E>::from_f32(x[r] * beta);
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
            const float bs = sBetaK[16 * j + li];
            const int pc = O::perm(16 * j + li);
#pragma unroll
            for (int e = 0; e < 4; ++e) sTp[(16 * i + 4 * lg + e) * LDC + pc] = Elem<E>::from_f32(-t[e] * bs);
          }
        }
      }
      if (c + 1 < nch) fetch(c + 1);
    };

    if (nch > 0) {
      fetch(0);
      produce(0, 0);
    }
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
      if (c + 1 < nch) produce(c + 1, (c + 1) & 1);
      lds_barrier();
    }
  } else {
    // ======================= Q wave ==========================================
    constexpr int V16 = 16 / (int)sizeof(E);  // elements per 16-byte piece
    constexpr int PPR = DVT / V16;            // 16-byte pieces per V row slice
    constexpr int NVP = (C * PPR + 63) / 64;  // V pieces per lane
    Nat qop[NB][KSTEPS], kop[NB][KSTEPS];
    uint4 vreg[NVP];
    E qg_raw = Elem<E>::from_f32(0.f);
    const size_t vcol0 = (size_t)jt * DVT;
    auto fetch = [&](int c) {
      const int nrow = min(C, len - c * C);
      const size_t tok0 = row0 + (size_t)c * C;
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const int r = min(16 * rt + li, nrow - 1);
#pragma unroll
        for (int kq = 0; kq < KSTEPS; ++kq) {
          qop[rt][kq] = O::ldg(gq + (tok0 + r) * DK + kq * KSTEP + lg * VPL);
          kop[rt][kq] = O::ldg(gk + (tok0 + r) * DK + kq * KSTEP + lg * VPL);
        }
      }
#pragma unroll
      for (int i = 0; i < NVP; ++i) {
        const int pc = min(lane + 64 * i, C * PPR - 1);
        const int r = min(pc / PPR, nrow - 1), cq = pc % PPR;
        vreg[i] = ldg16(gv + (tok0 + r) * (size_t)dv + vcol0 + cq * V16);
      }
      qg_raw = gg[tok0 + min(lane, nrow - 1)];
    };

    auto produce = [&](int c, int nb) {
      E *sQ = bufE(nb) + Sh::OFF_Q;
      E *sV = bufE(nb) + Sh::OFF_V;
      E *sP = bufE(nb) + Sh::OFF_P;
      const int nrow = min(C, len - c * C);
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const int r = 16 * rt + li;
#pragma unroll
        for (int kq = 0; kq < KSTEPS; ++kq) {
          if (r >= nrow) {
            qop[rt][kq] = O::zero();
            kop[rt][kq] = O::zero();
          }
          O::st_nat(sQ + r * LDK, kq, lg, qop[rt][kq]);
        }
      }
      // V slice [C x DVT], row-major
#pragma unroll
      for (int i = 0; i < NVP; ++i) {
        const int pc = lane + 64 * i;
        if (pc < C * PPR) {
          const int r = pc / PPR, cq = pc % PPR;
          const uint4 u = (r < nrow) ? vreg[i] : make_uint4(0u, 0u, 0u, 0u);
          *reinterpret_cast<uint4 *>(sV + r * LDV + cq * V16) = u;
        }
      }
      const float gam = wave_inclusive_scan((lane < nrow) ? Elem<E>::to_f32(qg_raw) : 0.f);
      if (lane < C) sGamQ[lane] = gam;
      f32x4 gr4[NB];
      float gs1[NB];
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        gr4[rt] = *reinterpret_cast<const f32x4 *>(sGamQ + 16 * rt + 4 * lg);
        gs1[rt] = sGamQ[16 * rt + li];
      }
      // causal scores P = (Q K^T) weighted by exp(gamma_r - gamma_s), r >= s
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
        for (int st = 0; st <= rt; ++st) {
          f32x4 acc = zero4();
#pragma unroll
          for (int kq = 0; kq < KSTEPS; ++kq) acc = O::mma(qop[rt][kq], kop[st][kq], acc);
          const int s = 16 * st + li;
          const int pc = O::perm(s);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 16 * rt + 4 * lg + j;
            const float val = (r >= s) ? acc[j] * __expf(gr4[rt][j] - gs1[st]) : 0.f;
            sP[r * LDC + pc] = Elem<E>::from_f32(val);
          }
        }
      }
      if (c + 1 < nch) fetch(c + 1);
    };

    if (nch > 0) {
      fetch(0);
      produce(0, 0);
    }
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
      if (c + 1 < nch) produce(c + 1, (c + 1) & 1);
      lds_barrier();
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
