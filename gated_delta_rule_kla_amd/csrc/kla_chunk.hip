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
  // the same group read from a naturally ordered row in global memory
  static __device__ __forceinline__ Grp ldg_grp(const bf16 *row, int kb, int g) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(row + kb + 4 * g);
    const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(row + kb + 16 + 4 * g);
    return Grp{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  static __device__ __forceinline__ Grp zero_grp() { return zero(); }
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
  static __device__ __forceinline__ Grp ldg_grp(const float *row, int kb, int g) {
    return *reinterpret_cast<const f32x4 *>(row + kb + 4 * g);
  }
  static __device__ __forceinline__ Grp zero_grp() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
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
// Roles and LDS plan
// ---------------------------------------------------------------------------
// Waves of a workgroup.  Iteration i (one barrier each, i = -2 .. nch) has
//   CHAIN  scan chunk i        OUTPUT  chunk i-1       PWAVE[2]  P of chunk i
//   TSOLVE T' of chunk i+1     VLOAD   V of chunk i+1  GRAM[2]   chunk i+2
enum Role { CHAIN = 0, OUTPUT = 1, GRAM0 = 2, GRAM1 = 3, TSOLVE = 4, PW0 = 5, PW1 = 6, VLOAD = 7 };
constexpr int kWaves = 8;

// lower-triangular 16x16 tile (rt, st), st <= rt, in row-major order; the two
// Gram waves and the two P waves each take one half of the list
__host__ __device__ constexpr int tile_index(int rt, int st) { return rt * (rt + 1) / 2 + st; }
__host__ __device__ constexpr int tile_part(int NB, int rt, int st) {
  return tile_index(rt, st) < (NB * (NB + 1) / 2 + 1) / 2 ? 0 : 1;
}
__host__ __device__ constexpr bool part_uses_row(int NB, int part, int rt) {
  for (int st = 0; st <= rt; ++st)
    if (tile_part(NB, rt, st) == part) return true;
  return false;
}
// diagonal blocks owned by a Gram wave, in order
__host__ __device__ constexpr int part_diag_count(int NB, int part) {
  int n = 0;
  for (int b = 0; b < NB; ++b) n += (tile_part(NB, b, b) == part);
  return n;
}
__host__ __device__ constexpr int part_diag_block(int NB, int part, int k) {
  for (int b = 0; b < NB; ++b)
    if (tile_part(NB, b, b) == part && k-- == 0) return b;
  return -1;
}

template <typename E, int C, int DK, int NCT>
struct ChunkShape {
  static constexpr int NB = C / 16;            // 16-row blocks per chunk
  static constexpr int DVT = 16 * NCT;         // state columns per workgroup
  static constexpr int NT = 64 * kWaves;
  static constexpr int PAD = 16 / (int)sizeof(E);
  static constexpr int LDK = DK + PAD;         // K rows (grouped columns)
  static constexpr int LDC = C + PAD;          // T' and P rows (grouped columns)
  static constexpr int LDV = DVT + PAD;        // V slice rows (natural)
  static constexpr int LDA = 16 + PAD;         // rows of one 16x16 off-diagonal A block
  static constexpr int LDD = 20;               // fp32 16-wide rows of diagonal blocks
  static constexpr int KG = Ops<E>::KG;
  static constexpr int NOFF = NB * (NB - 1) / 2;
  static constexpr int MAXD = (NB + 1) / 2;    // diagonal blocks per Gram wave
  // sizes in bytes
  static constexpr int K_SLOT = C * LDK * (int)sizeof(E);
  static constexpr int V_SLOT = C * LDV * (int)sizeof(E);
  static constexpr int TP_SLOT = C * LDC * (int)sizeof(E);
  static constexpr int P_SLOT = C * LDC * (int)sizeof(E);
  static constexpr int SU_S = NCT * (DK / KG) * 64 * 16;   // S start groups, 16 B per lane
  static constexpr int SU_U = NCT * (C / KG) * 64 * 16;    // U~ groups
  static constexpr int SU_SLOT = SU_S + SU_U;
  static constexpr int A_SLOT = (NOFF > 0 ? NOFF : 1) * 16 * LDA * (int)sizeof(E);
  static constexpr int TD_SLOT = NB * 16 * LDD * 4;        // T diagonal blocks, transposed, fp32
  static constexpr int VEC_SLOT = 4 * C * 4;               // gamma, Gam, d, beta
  static constexpr int GPRIV = MAXD * 16 * LDD * 4 + NB * 64 * 4 + 2 * C * 4;  // At blocks, norm partials, gamma/beta
  static constexpr int OT_BYTES = (sizeof(E) == 2 ? NCT : 0) * 16 * LDC * (int)sizeof(E);
  // offsets
  static constexpr int OFF_K = 0;
  static constexpr int OFF_V = OFF_K + 3 * K_SLOT;
  static constexpr int OFF_TP = OFF_V + 2 * V_SLOT;
  static constexpr int OFF_P = OFF_TP + 2 * TP_SLOT;
  static constexpr int OFF_SU = OFF_P + 2 * P_SLOT;
  static constexpr int OFF_A = OFF_SU + 2 * SU_SLOT;
  static constexpr int OFF_TD = OFF_A + 2 * A_SLOT;
  static constexpr int OFF_VEC = OFF_TD + 2 * TD_SLOT;
  static constexpr int OFF_GP = OFF_VEC + 4 * VEC_SLOT;
  static constexpr int OFF_OT = OFF_GP + 2 * GPRIV;
  static constexpr int BYTES = OFF_OT + OT_BYTES;

  static_assert(C == 16 || C == 64, "chunk");
  static_assert(C % KG == 0 && DK % KG == 0 && DK % Ops<E>::KSTEP == 0, "dk");
  static_assert(K_SLOT % 16 == 0 && V_SLOT % 16 == 0 && TP_SLOT % 16 == 0 && A_SLOT % 16 == 0 &&
                    GPRIV % 16 == 0 && VEC_SLOT % 16 == 0 && OT_BYTES % 16 == 0, "lds align");
  static_assert((LDK * (int)sizeof(E)) % 16 == 0 && (LDC * (int)sizeof(E)) % 16 == 0 &&
                    (LDV * (int)sizeof(E)) % 16 == 0 && (LDA * (int)sizeof(E)) % 8 == 0, "row align");
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
template <typename E, int C, int DK, int NCT>
__global__ __launch_bounds__(64 * kWaves) void kla_chunk_kernel(ChunkParams p) {
  using Sh = ChunkShape<E, C, DK, NCT>;
  using O = Ops<E>;
  using Nat = typename O::Nat;
  using Grp = typename O::Grp;
  constexpr int NB = Sh::NB, DVT = Sh::DVT, LDK = Sh::LDK, LDC = Sh::LDC, LDV = Sh::LDV;
  constexpr int LDA = Sh::LDA, LDD = Sh::LDD;
  constexpr int KSTEP = O::KSTEP, VPL = O::VPL, KSTEPS = DK / KSTEP, KG = O::KG, TPG = KG / 16;
  constexpr int NQG = DK / KG;  // contraction groups over dk
  constexpr int NCG = C / KG;   // contraction groups over the chunk

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
  auto nrow_of = [&](int c) { return min(C, len - c * C); };
  auto tok0_of = [&](int c) { return row0 + (size_t)c * C; };

  // ---- LDS views -------------------------------------------------------------
  auto sK = [&](int c) { return reinterpret_cast<E *>(smem + Sh::OFF_K + (c % 3) * Sh::K_SLOT); };
  auto sV = [&](int c) { return reinterpret_cast<E *>(smem + Sh::OFF_V + (c & 1) * Sh::V_SLOT); };
  auto sTp = [&](int c) { return reinterpret_cast<E *>(smem + Sh::OFF_TP + (c & 1) * Sh::TP_SLOT); };
  auto sP = [&](int c) { return reinterpret_cast<E *>(smem + Sh::OFF_P + (c & 1) * Sh::P_SLOT); };
  auto sSuS = [&](int c) { return reinterpret_cast<Grp *>(smem + Sh::OFF_SU + (c & 1) * Sh::SU_SLOT); };
  auto sSuU = [&](int c) {
    return reinterpret_cast<Grp *>(smem + Sh::OFF_SU + (c & 1) * Sh::SU_SLOT + Sh::SU_S);
  };
  auto sA = [&](int c) { return reinterpret_cast<E *>(smem + Sh::OFF_A + (c & 1) * Sh::A_SLOT); };
  auto sTd = [&](int c) { return reinterpret_cast<float *>(smem + Sh::OFF_TD + (c & 1) * Sh::TD_SLOT); };
  // per-chunk row vectors: gamma, Gam = exp(gamma), d = exp(gamma_C - gamma), beta
  auto sVec = [&](int c) { return reinterpret_cast<float *>(smem + Sh::OFF_VEC + (c & 3) * Sh::VEC_SLOT); };

  // strictly-upper 16x16 blocks of T' and P are zero and never rewritten
  for (int i = threadIdx.x; i < 2 * C * C; i += Sh::NT) {
    const int bi = i / (C * C), rr = (i / C) % C, ss = i % C;
    if ((rr >> 4) < (ss >> 4)) {
      sTp(bi)[rr * LDC + O::perm(ss)] = Elem<E>::from_f32(0.f);
      sP(bi)[rr * LDC + O::perm(ss)] = Elem<E>::from_f32(0.f);
    }
  }

  if (wave == CHAIN) {
    // =================== chain: the sequential state scan ====================
    // S (DK rows x DVT columns, fp32) lives in the accumulators for the whole
    // sequence: accS[ct][it] is the 16x16 tile (rows 16 it.., columns 16 ct..).
    f32x4 accS[NCT][DK / 16];
    const size_t sbase = (size_t)nh * DK * (size_t)dv;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int col = jt * DVT + 16 * ct + li;
#pragma unroll
      for (int it = 0; it < DK / 16; ++it)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          accS[ct][it][j] = p.s0 ? p.s0[sbase + (size_t)(16 * it + 4 * lg + j) * dv + col] : 0.f;
    }
    __syncthreads();
    for (int i = -2; i <= nch; ++i) {
      if (i >= 0 && i < nch) {
        const int c = i;
        const E *K = sK(c);
        const E *V = sV(c);
        const E *Tp = sTp(c);
        const float *vec = sVec(c);
        Grp *suS = sSuS(c);
        Grp *suU = sSuU(c);
        // S as right operands, straight from the accumulators; also handed to
        // the output wave (it needs the chunk's start state)
        Grp sb[NCT][NQG];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int q = 0; q < NQG; ++q) {
            sb[ct][q] = O::b_from_d(&accS[ct][q * TPG]);
            suS[(ct * NQG + q) * 64 + lane] = sb[ct][q];
          }
        // K S
        f32x4 x[NCT][NB];
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) x[ct][rt] = zero4();
#pragma unroll
          for (int q = 0; q < NQG; ++q) {
            const Grp a = O::a_row(K + (16 * rt + li) * LDK, q * KG, lg);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) x[ct][rt] = O::mma_grp(a, sb[ct][q], x[ct][rt]);
          }
        }
        // X = V - Diag(Gam) K S
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) {
          const f32x4 gm = *reinterpret_cast<const f32x4 *>(vec + C + 16 * rt + 4 * lg);
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) x[ct][rt] = O::col4(V, LDV, 16 * rt, 16 * ct, lane) - gm * x[ct][rt];
        }
        Grp xb[NCT][NCG];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int q = 0; q < NCG; ++q) xb[ct][q] = O::b_from_d(&x[ct][q * TPG]);
        // U~ = T' X   (T' lower triangular: skip the zero groups)
        f32x4 u[NCT][NB];
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) u[ct][rt] = zero4();
#pragma unroll
          for (int q = 0; q * KG < 16 * (rt + 1); ++q) {
            const Grp a = O::a_row(Tp + (16 * rt + li) * LDC, q * KG, lg);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) u[ct][rt] = O::mma_grp(a, xb[ct][q], u[ct][rt]);
          }
        }
        // U~ groups for the output wave; Diag(d) U~ groups for the update
        Grp dub[NCT][NCG];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int q = 0; q < NCG; ++q) {
            suU[(ct * NCG + q) * 64 + lane] = O::b_from_d(&u[ct][q * TPG]);
            f32x4 du[TPG];
#pragma unroll
            for (int tt = 0; tt < TPG; ++tt) {
              const int r16 = 16 * (q * TPG + tt);
              du[tt] = *reinterpret_cast<const f32x4 *>(vec + 2 * C + r16 + 4 * lg) * u[ct][q * TPG + tt];
            }
            dub[ct][q] = O::b_from_d(du);
          }
        // S <- Gam_C S + K^T Diag(d) U~
        const float gC = vec[C + C - 1];
#pragma unroll
        for (int it = 0; it < DK / 16; ++it) {
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) accS[ct][it] = gC * accS[ct][it];
#pragma unroll
          for (int q = 0; q < NCG; ++q) {
            const Grp a = O::a_trans(K, LDK, q * KG, 16 * it, lane);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) accS[ct][it] = O::mma_grp(a, dub[ct][q], accS[ct][it]);
          }
        }
      }
      lds_barrier();
    }
    if (p.sfin) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int col = jt * DVT + 16 * ct + li;
#pragma unroll
        for (int it = 0; it < DK / 16; ++it)
#pragma unroll
          for (int j = 0; j < 4; ++j) p.sfin[sbase + (size_t)(16 * it + 4 * lg + j) * dv + col] = accS[ct][it][j];
      }
    }
  } else if (wave == OUTPUT) {
    // =================== output: O = Diag(Gam) Q S + P U~ =====================
    // Runs one chunk behind the chain; Q comes straight from global memory in
    // grouped column order, fetched one iteration ahead.
    Grp qreg[NB][NQG];
    auto fetch = [&](int c) {
      const int nrow = nrow_of(c);
      const size_t tok0 = tok0_of(c);
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const E *row = gq + (tok0 + min(16 * rt + li, nrow - 1)) * DK;
#pragma unroll
        for (int q = 0; q < NQG; ++q) qreg[rt][q] = O::ldg_grp(row, q * KG, lg);
      }
    };
    E *sOt = reinterpret_cast<E *>(smem + Sh::OFF_OT);
    __syncthreads();
    for (int i = -2; i <= nch; ++i) {
      if (i >= 1 && i <= nch) {
        const int c = i - 1;
        const int nrow = nrow_of(c);
        const size_t tok0 = tok0_of(c);
        const E *Pm = sP(c);
        const Grp *suS = sSuS(c);
        const Grp *suU = sSuU(c);
        const float *vec = sVec(c);
#pragma unroll
        for (int rt = 0; rt < NB; ++rt)
          if (16 * rt + li >= nrow)
#pragma unroll
            for (int q = 0; q < NQG; ++q) qreg[rt][q] = O::zero_grp();
        f32x4 ao[NCT][NB];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          Grp sb[NQG];
#pragma unroll
          for (int q = 0; q < NQG; ++q) sb[q] = suS[(ct * NQG + q) * 64 + lane];
#pragma unroll
          for (int rt = 0; rt < NB; ++rt) {
            ao[ct][rt] = zero4();
#pragma unroll
            for (int q = 0; q < NQG; ++q) ao[ct][rt] = O::mma_grp(qreg[rt][q], sb[q], ao[ct][rt]);
          }
        }
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) {
          const f32x4 gm = *reinterpret_cast<const f32x4 *>(vec + C + 16 * rt + 4 * lg);
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) ao[ct][rt] = gm * ao[ct][rt];
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          Grp ub[NCG];
#pragma unroll
          for (int q = 0; q < NCG; ++q) ub[q] = suU[(ct * NCG + q) * 64 + lane];
#pragma unroll
          for (int rt = 0; rt < NB; ++rt)
#pragma unroll
            for (int q = 0; q * KG < 16 * (rt + 1); ++q)
              ao[ct][rt] = O::mma_grp(O::a_row(Pm + (16 * rt + li) * LDC, q * KG, lg), ub[q], ao[ct][rt]);
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const int col0 = jt * DVT + 16 * ct;
          if constexpr (sizeof(E) == 2) {
            // stage O^T (4 rows of one column = one 8-byte write per lane), read
            // it back transposed (4 columns of one row) and store 8 bytes
            E *st = sOt + ct * 16 * LDC;
#pragma unroll
            for (int rt = 0; rt < NB; ++rt) {
              bf16x4 ob;
#pragma unroll
              for (int j = 0; j < 4; ++j) ob[j] = (bf16)ao[ct][rt][j];
              *reinterpret_cast<bf16x4 *>(st + li * LDC + 16 * rt + 4 * lg) = ob;
            }
            const int x = (lane >> 2) & 3, a = lane & 3;
            bf16x4 rows[NB];
#pragma unroll
            for (int rt = 0; rt < NB; ++rt)
              rows[rt] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(st + (4 * lg + x) * LDC + 16 * rt + 4 * a));
#pragma unroll
            for (int rt = 0; rt < NB; ++rt)
              if (16 * rt + li < nrow)
                *reinterpret_cast<bf16x4 *>(go + (tok0 + 16 * rt + li) * (size_t)dv + col0 + 4 * lg) = rows[rt];
          } else {
#pragma unroll
            for (int rt = 0; rt < NB; ++rt)
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const int r = 16 * rt + 4 * lg + j;
                if (r < nrow) go[(tok0 + r) * (size_t)dv + col0 + li] = Elem<E>::from_f32(ao[ct][rt][j]);
              }
          }
        }
      }
      if (i >= 0 && i < nch) fetch(i);
      lds_barrier();
    }
  } else if (wave == GRAM0 || wave == GRAM1) {
    // =================== Gram waves: chunk i+2 ================================
    const int part = wave - GRAM0;
    Nat kop[NB][KSTEPS];
    E kg_raw = Elem<E>::from_f32(0.f), ke_raw = Elem<E>::from_f32(0.f);
    auto fetch = [&](int c) {
      const int nrow = nrow_of(c);
      const size_t tok0 = tok0_of(c);
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
    char *gp = smem + Sh::OFF_GP + part * Sh::GPRIV;
    float *sAtd = reinterpret_cast<float *>(gp);                       // [MAXD][16][LDD]
    float *sNrm = sAtd + Sh::MAXD * 16 * LDD;                          // [NB][4][16]
    float *sGam = sNrm + NB * 64;                                      // [C]
    float *sBet = sGam + C;                                            // [C]

    auto produce = [&](int c) {
      const int nrow = nrow_of(c);
      E *K = sK(c);
      E *Ablk = sA(c);
      float *Td = sTd(c);
      float *vec = sVec(c);
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const int r = 16 * rt + li;
#pragma unroll
        for (int kq = 0; kq < KSTEPS; ++kq) {
          if (r >= nrow) kop[rt][kq] = O::zero();
          // K rows for the chain and P waves (half the row tiles each)
          if ((rt < (NB + 1) / 2) == (part == 0)) O::st_nat(K + r * LDK, kq, lg, kop[rt][kq]);
        }
      }
      // fused ||k_r||^2: lane holds a quarter of row 16rt + li; lane r sums the
      // four quarters of its row through LDS
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        float sq = 0.f;
#pragma unroll
        for (int kq = 0; kq < KSTEPS; ++kq) sq += O::sumsq(kop[rt][kq]);
        sNrm[(rt * 4 + lg) * 16 + li] = sq;
      }
      const float gam = wave_inclusive_scan((lane < nrow) ? Elem<E>::to_f32(kg_raw) : 0.f);
      float nr = 0.f;
      if (lane < C) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) nr += sNrm[((lane >> 4) * 4 + q4) * 16 + li];
      }
      // beta of rows beyond the sequence end is 0 (not 0/0 when eps = 0)
      const float beta = (lane < nrow) ? Elem<E>::to_f32(ke_raw) / (nr + p.eps) : 0.f;
      const float gamC = lane_value(gam, C - 1);
      if (lane < C) {
        sGam[lane] = gam;
        sBet[lane] = beta;
        if (part == 0) {
          vec[lane] = gam;
          vec[C + lane] = __expf(gam);             // Gam_r
          vec[2 * C + lane] = __expf(gamC - gam);  // d_r
          vec[3 * C + lane] = beta;
        }
      }
      f32x4 gr4[NB], br4[NB];
      float gs1[NB];
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        gr4[rt] = *reinterpret_cast<const f32x4 *>(sGam + 16 * rt + 4 * lg);
        br4[rt] = *reinterpret_cast<const f32x4 *>(sBet + 16 * rt + 4 * lg);
        gs1[rt] = sGam[16 * rt + li];
      }
      // this wave's Gram tiles and A = beta_r (K K^T)_rs exp(gamma_r - gamma_s), r > s
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
        for (int st = 0; st <= rt; ++st) {
          if (tile_part(NB, rt, st) != part) continue;
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
            E *blk = Ablk + (rt * (rt - 1) / 2 + st) * 16 * LDA;
#pragma unroll
            for (int j = 0; j < 4; ++j) blk[(4 * lg + j) * LDA + li] = Elem<E>::from_f32(av[j]);
          } else {
            // own diagonal block, stored transposed: At[s'][r']
            int dl = 0;
#pragma unroll
            for (int kk = 0; kk < Sh::MAXD; ++kk)
              if (part_diag_block(NB, part, kk) == rt) dl = kk;
            *reinterpret_cast<f32x4 *>(sAtd + dl * 16 * LDD + li * LDD + 4 * lg) = av;
          }
        }
      }
      // own diagonal blocks of T = (I + A)^-1 by column-parallel forward
      // substitution in fp32: lane = (local block lg, column li)
      constexpr int ND0 = part_diag_count(NB, 0), ND1 = part_diag_count(NB, 1);
      const int nd = part == 0 ? ND0 : ND1;
      if (lg < nd) {
        int bb = 0;
#pragma unroll
        for (int kk = 0; kk < Sh::MAXD; ++kk)
          if (kk == lg) bb = part_diag_block(NB, part, kk);
        const float *At = sAtd + lg * 16 * LDD;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == li) ? 1.f : 0.f;
#pragma unroll
        for (int s = 0; s < 15; ++s) {
          f32x4 colv[4];
#pragma unroll
          for (int qd = 0; qd < 4; ++qd)
            if (4 * qd + 3 > s) colv[qd] = *reinterpret_cast<const f32x4 *>(At + s * LDD + 4 * qd);
#pragma unroll
          for (int r = s + 1; r < 16; ++r) x[r] = fmaf(-colv[r >> 2][r & 3], x[s], x[r]);
        }
        // T_bb transposed: row li of T^T = column li of T
        float *dst = Td + (bb * 16 + li) * LDD;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          *reinterpret_cast<f32x4 *>(dst + 4 * qd) = f32x4{x[4 * qd], x[4 * qd + 1], x[4 * qd + 2], x[4 * qd + 3]};
      }
    };

    if (nch > 0) fetch(0);
    __syncthreads();
    for (int i = -2; i <= nch; ++i) {
      const int c = i + 2;
      if (c >= 0 && c < nch) {
        produce(c);
        if (c + 1 < nch) fetch(c + 1);
      }
      lds_barrier();
    }
  } else if (wave == TSOLVE) {
    // =================== T' of chunk i+1 ======================================
    // T' = T Diag(beta); diagonal blocks of T come from the Gram waves, the
    // off-diagonal blocks are built level by level: T_ij = -T_ii sum_m A_im T_mj
    auto solve = [&](int c) {
      E *Tp = sTp(c);
      const E *Ablk = sA(c);
      const float *Td = sTd(c);
      const float *beta = sVec(c) + 3 * C;
      // diagonal blocks: lane = (block lg, column li)
      if (lg < NB) {
        const float *src = Td + (lg * 16 + li) * LDD;
        const float bs = beta[16 * lg + li];
        const int pc = O::perm(16 * lg + li);
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const f32x4 t4 = *reinterpret_cast<const f32x4 *>(src + 4 * qd);
#pragma unroll
          for (int e = 0; e < 4; ++e) Tp[(16 * lg + 4 * qd + e) * LDC + pc] = Elem<E>::from_f32(t4[e] * bs);
        }
      }
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
              const f32x4 a4 = load4(Ablk + (i * (i - 1) / 2 + m) * 16 * LDA + li * LDA + 4 * lg);
#pragma unroll
              for (int e = 0; e < 4; ++e) a[e] = a4[e];
              if (m == j) {
                // B operand T_jj[4lg + e][li] = T_jj^T[li][4lg + e]
                const f32x4 t4 = *reinterpret_cast<const f32x4 *>(Td + (j * 16 + li) * LDD + 4 * lg);
#pragma unroll
                for (int e = 0; e < 4; ++e) bb[e] = t4[e];
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) bb[e] = Toff[m][j][e];
              }
              y = Mm16<E>::mma(a, bb, y);
            }
            // A operand T_ii[li][4lg + e] = T_ii^T[4lg + e][li]
            float a[4], bb[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              a[e] = Td[(i * 16 + 4 * lg + e) * LDD + li];
              bb[e] = y[e];
            }
            const f32x4 t = Mm16<E>::mma(a, bb, zero4());
            Toff[i][j] = -t;
            const float bs = beta[16 * j + li];
            const int pc = O::perm(16 * j + li);
#pragma unroll
            for (int e = 0; e < 4; ++e) Tp[(16 * i + 4 * lg + e) * LDC + pc] = Elem<E>::from_f32(-t[e] * bs);
          }
        }
      }
    };
    __syncthreads();
    for (int i = -2; i <= nch; ++i) {
      if (i + 1 >= 0 && i + 1 < nch) solve(i + 1);
      lds_barrier();
    }
  } else if (wave == PW0 || wave == PW1) {
    // =================== P waves: causal scores of chunk i ====================
    const int part = wave - PW0;
    Grp qreg[NB][NQG];
    auto fetch = [&](int c) {
      const int nrow = nrow_of(c);
      const size_t tok0 = tok0_of(c);
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        if (!part_uses_row(NB, part, rt)) continue;
        const E *row = gq + (tok0 + min(16 * rt + li, nrow - 1)) * DK;
#pragma unroll
        for (int q = 0; q < NQG; ++q) qreg[rt][q] = O::ldg_grp(row, q * KG, lg);
      }
    };
    auto produce = [&](int c) {
      const int nrow = nrow_of(c);
      const E *K = sK(c);
      E *Pm = sP(c);
      const float *gamv = sVec(c);
      f32x4 gr4[NB];
      float gs1[NB];
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        gr4[rt] = *reinterpret_cast<const f32x4 *>(gamv + 16 * rt + 4 * lg);
        gs1[rt] = gamv[16 * rt + li];
      }
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        if (!part_uses_row(NB, part, rt)) continue;
        if (16 * rt + li >= nrow)
#pragma unroll
          for (int q = 0; q < NQG; ++q) qreg[rt][q] = O::zero_grp();
#pragma unroll
        for (int st = 0; st <= rt; ++st) {
          if (tile_part(NB, rt, st) != part) continue;
          f32x4 acc = zero4();
#pragma unroll
          for (int q = 0; q < NQG; ++q) acc = O::mma_grp(qreg[rt][q], O::a_row(K + (16 * st + li) * LDK, q * KG, lg), acc);
          const int s = 16 * st + li;
          const int pc = O::perm(s);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 16 * rt + 4 * lg + j;
            const float val = (r >= s) ? acc[j] * __expf(gr4[rt][j] - gs1[st]) : 0.f;
            Pm[r * LDC + pc] = Elem<E>::from_f32(val);
          }
        }
      }
    };
    __syncthreads();
    for (int i = -2; i <= nch; ++i) {
      if (i >= 0 && i < nch) produce(i);
      if (i + 1 >= 0 && i + 1 < nch) fetch(i + 1);
      lds_barrier();
    }
  } else {
    // =================== V loader: V slice of chunk i+1 =======================
    constexpr int V16 = 16 / (int)sizeof(E);  // elements per 16-byte piece
    constexpr int PPR = DVT / V16;            // 16-byte pieces per V row slice
    constexpr int NVP = (C * PPR + 63) / 64;  // pieces per lane
    uint4 vreg[NVP];
    const size_t vcol0 = (size_t)jt * DVT;
    auto fetch = [&](int c) {
      const int nrow = nrow_of(c);
      const size_t tok0 = tok0_of(c);
#pragma unroll
      for (int k = 0; k < NVP; ++k) {
        const int pc = min(lane + 64 * k, C * PPR - 1);
        const int r = min(pc / PPR, nrow - 1), cq = pc % PPR;
        vreg[k] = ldg16(gv + (tok0 + r) * (size_t)dv + vcol0 + cq * V16);
      }
    };
    auto store = [&](int c) {
      const int nrow = nrow_of(c);
      E *V = sV(c);
#pragma unroll
      for (int k = 0; k < NVP; ++k) {
        const int pc = lane + 64 * k;
        if (pc < C * PPR) {
          const int r = pc / PPR, cq = pc % PPR;
          *reinterpret_cast<uint4 *>(V + r * LDV + cq * V16) = (r < nrow) ? vreg[k] : make_uint4(0u, 0u, 0u, 0u);
        }
      }
    };
    if (nch > 0) fetch(0);
    __syncthreads();
    for (int i = -2; i <= nch; ++i) {
      if (i + 1 >= 0 && i + 1 < nch) {
        store(i + 1);
        if (i + 2 < nch) fetch(i + 2);
      }
      lds_barrier();
    }
  }
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------
template <typename E, int C, int DK, int NCT>
static hipError_t launch_chunk_t(const ChunkArgs &a, hipStream_t st) {
  using Sh = ChunkShape<E, C, DK, NCT>;
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
  hipLaunchKernelGGL((kla_chunk_kernel<E, C, DK, NCT>), dim3((unsigned)nblk), dim3(Sh::NT), 0, st, p);
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

// Column slice width: 32 columns (two column tiles per workgroup) when that
// still gives at least one workgroup per CU, else 16 (more workgroups, more
// redundant S-independent work per column).
static bool use_two_column_tiles(const ChunkArgs &a) {
  return a.dv % 32 == 0 && (long long)a.num_seqs * a.H * (a.dv / 32) >= 256;
}

hipError_t launch_chunk_fwd(const ChunkArgs &a, hipStream_t st) {
  if (a.dtype == 0) {
    const bool two = use_two_column_tiles(a);
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
