// kla_ops.h -- the MFMA operand machinery shared by the chunk kernels
// (kla_chunk.hip) and the gradient kernel (kla_bwd.hip) for gfx950 (CDNA4):
// operand and accumulator layouts of the bf16 and fp32 MFMAs, the grouped
// column order of rows kept in LDS, the packed T'^T image of a chunk, and the
// coalesced row, image and value-slice loaders.
#pragma once

#include <type_traits>

#include "kla_common.h"

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
  // sum of squares of the 8 values: bf16 products are exact in fp32
  static __device__ __forceinline__ float sumsq(Nat v) {
    float s = 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const bf16x2 pr = {v[2 * x], v[2 * x + 1]};
      s = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, s, false);
    }
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
  // store one 16-byte piece (natural columns 8m .. 8m+7) into a grouped row
  static __device__ __forceinline__ void st_piece(bf16 *row, int m, uint4 v) {
    st_nat(row, m >> 2, m & 3, __builtin_bit_cast(Nat, v));
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
  static __device__ __forceinline__ void st_piece(float *row, int m, uint4 v) {
    *reinterpret_cast<f32x4 *>(row + 4 * m) = __builtin_bit_cast(f32x4, v);
  }
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
  typedef bf16x4 Op;
  // left operand of a 16x16 block stored transposed (Mt[k][row]): one
  // transposing LDS read gives lane l the entries [l&15][4(l>>4) .. +3]
  static __device__ __forceinline__ Op ld_t(const bf16 *Mt, int ld, int lane) {
    const int g = lane >> 4, x = (lane >> 2) & 3, a = lane & 3;
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(Mt + (4 * g + x) * ld + 4 * a));
  }
  static __device__ __forceinline__ Op cvt(f32x4 v) { return Op{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]}; }
  static __device__ __forceinline__ f32x4 mma(Op a, Op b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
};

template <> struct Mm16<float> {
  typedef f32x4 Op;
  static __device__ __forceinline__ Op ld_t(const float *Mt, int ld, int lane) {
    const int g = lane >> 4, li = lane & 15;
    return Op{Mt[(4 * g) * ld + li], Mt[(4 * g + 1) * ld + li], Mt[(4 * g + 2) * ld + li], Mt[(4 * g + 3) * ld + li]};
  }
  static __device__ __forceinline__ Op cvt(f32x4 v) { return v; }
  static __device__ __forceinline__ f32x4 mma(Op a, Op b, f32x4 c) {
#pragma unroll
    for (int x = 0; x < 4; ++x) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[x], b[x], c, 0, 0, 0);
    return c;
  }
};

// four consecutive elements from fp32
__device__ __forceinline__ void store4(bf16 *p, f32x4 v) {
  *reinterpret_cast<bf16x4 *>(p) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}
__device__ __forceinline__ void store4(float *p, f32x4 v) { *reinterpret_cast<f32x4 *>(p) = v; }

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

// The 16-row blocks of a chunk are split between two waves (two Gram waves in
// the prep kernel, two P waves in the scan kernel): part 0 owns the first and
// the last block, part 1 the ones in between.  A wave handles the
// lower-triangular tiles (rt, st <= rt) of the row blocks rt it owns (5 of the
// 10 tiles each for a 64-token chunk), so the diagonal tiles -- and with them
// ||k_r||^2 and beta_r -- of all its rows are its own.  Chunks of 16 (one
// block) leave part 1 idle.
__host__ __device__ constexpr bool owns_block(int NB, int part, int rt) {
  return (rt == 0 || rt == NB - 1) ? part == 0 : part == 1;
}
template <int NB, int PART>
struct OwnBlocks {  // the blocks a part owns, in order
  static constexpr int N = PART == 0 ? (NB > 1 ? 2 : 1) : NB - 2;
  static __host__ __device__ constexpr int at(int k) { return PART == 0 ? (k == 0 ? 0 : NB - 1) : 1 + k; }
};

template <int NB>
struct AllBlocks {
  static constexpr int N = NB;
  static __host__ __device__ constexpr int at(int k) { return k; }
};

// LDS row padding: 32 bytes.  With 64 four-byte banks, rows 32 bytes apart
// modulo 256 keep the transposing reads (4 rows x 32 bytes per 16 lanes) and
// the 16-byte row reads free of bank conflicts for the row lengths used here
// (measured: 2.9x fewer conflict cycles than 16-byte padding for the K^T reads).
template <typename E>
struct LdsPad {
  static constexpr int V = 32 / (int)sizeof(E);
};

// The per-chunk data the prep kernel hands to the scan kernel.  In LDS: the
// T'^T image (C rows of LDC, grouped columns, zero blocks and pads included),
// then the row vectors gamma, Gam, d (fp32).  In the workspace the image is
// packed: rows s < RW keep all C columns, rows s >= RW only the last C - RW
// (T' U-products never read rows >= 32 at columns < 32: those are zero
// blocks of the upper block triangle of T'^T), then the three vectors.
template <typename E, int C>
struct TpLayout {
  static constexpr int PAD = LdsPad<E>::V;
  static constexpr int LDC = C + PAD;                      // T'^T rows (grouped columns)
  static constexpr int TP_IMG = C * LDC * (int)sizeof(E);  // LDS image
  static constexpr int VEC3 = 3 * C * 4;
  static constexpr int LDS_BYTES = TP_IMG + VEC3;          // one LDS slot
  static constexpr int RW = C > 32 ? 32 : C;
  static constexpr int PACK = (RW * C + (C - RW) * (C - RW)) * (int)sizeof(E);
  static constexpr int BYTES = PACK + VEC3;                // workspace bytes per (chunk, head)
  static constexpr int EPP = 16 / (int)sizeof(E);          // elements per 16-byte piece
  // LDS element offset (in the image) of packed 16-byte piece pc < PACK / 16
  static __device__ __forceinline__ int piece_to_lds(int pc) {
    int e = pc * EPP;
    if constexpr (C > RW) {
      if (e >= RW * C) {
        e -= RW * C;
        return (RW + e / (C - RW)) * LDC + RW + e % (C - RW);
      }
    }
    return (e / C) * LDC + e % C;
  }
  // Compact LDS image: rows >= RW keep only their last C - RW columns (rows of LD2),
  // as in the workspace; the vectors follow it.
  static constexpr int LD2 = C > RW ? (C - RW) + PAD : LDC;
  static constexpr int TP_IMG_C = (RW * LDC + (C - RW) * LD2) * (int)sizeof(E);
  static constexpr int LDS_BYTES_C = TP_IMG_C + VEC3;
  static __device__ __forceinline__ int piece_to_lds_c(int pc) {
    int e = pc * EPP;
    if constexpr (C > RW) {
      if (e >= RW * C) {
        e -= RW * C;
        return RW * LDC + (e / (C - RW)) * LD2 + e % (C - RW);
      }
    }
    return (e / C) * LDC + e % C;
  }
  static_assert(TP_IMG % 16 == 0 && VEC3 % 16 == 0 && PACK % 16 == 0 && TP_IMG_C % 16 == 0, "align");
  static_assert((C - RW) % EPP == 0 && C % EPP == 0, "pieces stay inside a row");
  static_assert((LD2 * (int)sizeof(E)) % 16 == 0, "row align");
};

// Workspace slot of chunk c of sequence n: dense batches use n * ceil(T/C) + c;
// packed sequences use n + floor(t0_n / C) + c, which never collides (each
// sequence's last slot is below the next sequence's first) and stays below
// floor(T/C) + N + 1.
__host__ __device__ inline int slots_per_head(bool varlen, int B, int T, int N, int C) {
  return varlen ? T / C + N + 1 : B * ((T + C - 1) / C);
}

// Raw buffer resource over bytes [0, n) of p: loads at offsets >= n return 0
// (that is how rows past the end of a sequence read as zero rows).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *p, int n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, n, 0x00020000);
}
__device__ __forceinline__ uint4 buffer_ld16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// element i as raw bits (0 past the end of the resource); converted where it
// is used, so that the wait for the load lands there
__device__ __forceinline__ unsigned short buffer_ld_elem(__amdgpu_buffer_rsrc_t r, int i, const bf16 *) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, 2 * i, 0, 0);
}
__device__ __forceinline__ unsigned buffer_ld_elem(__amdgpu_buffer_rsrc_t r, int i, const float *) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, 4 * i, 0, 0);
}
__device__ __forceinline__ float elem_bits_to_f32(unsigned short v) { return Elem<bf16>::to_f32(__builtin_bit_cast(bf16, v)); }
__device__ __forceinline__ float elem_bits_to_f32(unsigned v) { return __builtin_bit_cast(float, v); }

// Coalesced loads of whole K or Q rows of one chunk: lane l takes the 16-byte
// pieces l, l + 64, ... of the listed row blocks, so consecutive lanes read
// consecutive bytes of a row (a wave instruction touches 4 rows of 256 B
// rather than 16 rows; loads that give each lane its own row cost the
// texture-address unit four times more).  The rows then go through LDS into
// the MFMA operand layout, where each lane holds one row.
template <typename E, int DK, class BL>
struct RowLoad {
  static constexpr int RB = DK * (int)sizeof(E);   // bytes per row
  static constexpr int PPR = RB / 16;              // 16-byte pieces per row
  static constexpr int RPJ = 64 / PPR;             // rows per wave instruction
  static constexpr int NPL = BL::N * 16 / RPJ;     // instructions (pieces per lane)
  static_assert(PPR >= 4 && 64 % PPR == 0, "row size");
  uint4 r[NPL > 0 ? NPL : 1];
  // list row of piece j of this lane: RPJ j + lane / PPR; chunk row:
  static __device__ __forceinline__ int chunk_row(int j, int lane) {
    return 16 * BL::at((RPJ * j) >> 4) + ((RPJ * j) & 15) + lane / PPR;
  }
  // chunk rows start at `rows`; rows >= nrow read as zero
  __device__ __forceinline__ void issue(const E *rows, int nrow, int lane) {
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(rows, nrow * RB);
#pragma unroll
    for (int j = 0; j < NPL; ++j) r[j] = buffer_ld16(rs, chunk_row(j, lane) * RB + (lane % PPR) * 16);
  }
  // store the rows in grouped column order; list row lr / chunk row cr goes
  // to row dst_row(lr, cr) of dst
  template <class RowMap>
  __device__ __forceinline__ void put(E *dst, int ld, int lane, RowMap dst_row) const {
#pragma unroll
    for (int j = 0; j < NPL; ++j)
      Ops<E>::st_piece(dst + dst_row(RPJ * j + lane / PPR, chunk_row(j, lane)) * ld, lane % PPR, r[j]);
  }
};

// A chunk's packed T'^T image and gamma, Gam, d from the workspace into the
// LDS slot (image rows at their LDS positions, the vectors after the image).
template <typename E, int C, bool COMPACT = false>
struct ImgCopy {
  using TL = TpLayout<E, C>;
  static constexpr int NI = TL::PACK / 16, NP = TL::BYTES / 16;
  static constexpr int NPL = (NP + 63) / 64;
  u32x4 r[NPL];
  __device__ __forceinline__ void issue(const void *src, int lane) {
#pragma unroll
    for (int j = 0; j < NPL; ++j) r[j] = reinterpret_cast<const u32x4 *>(src)[min(lane + 64 * j, NP - 1)];
  }
  __device__ __forceinline__ void put(E *slot, int lane) const {
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int i = lane + 64 * j;
      if (NP % 64 == 0 || i < NP) {
        char *d = i < NI ? reinterpret_cast<char *>(slot + (COMPACT ? TL::piece_to_lds_c(i) : TL::piece_to_lds(i)))
                         : reinterpret_cast<char *>(slot) + (COMPACT ? TL::TP_IMG_C : TL::TP_IMG) + 16 * (i - NI);
        *reinterpret_cast<u32x4 *>(d) = r[j];
      }
    }
  }
};

// The DVT-column slice of a chunk's V rows (rows past nrow read as zero):
// 16-byte pieces, consecutive lanes along a row.
template <typename E, int C, int DVT>
struct VSliceLoad {
  static constexpr int V16 = 16 / (int)sizeof(E);  // elements per piece
  static constexpr int PPR = DVT / V16;            // pieces per row slice
  static constexpr int NPL = (C * PPR + 63) / 64;  // pieces per lane
  uint4 r[NPL];
  __device__ __forceinline__ void issue(const E *rows, int nrow, int dv, int col0, int lane) {
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(rows, nrow * dv * (int)sizeof(E));
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int pc = min(lane + 64 * j, C * PPR - 1);
      r[j] = buffer_ld16(rs, ((pc / PPR) * dv + col0 + (pc % PPR) * V16) * (int)sizeof(E));
    }
  }
  __device__ __forceinline__ void put(E *V, int ldv, int lane) const {
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int pc = lane + 64 * j;
      if ((C * PPR) % 64 == 0 || pc < C * PPR) *reinterpret_cast<uint4 *>(V + (pc / PPR) * ldv + (pc % PPR) * V16) = r[j];
    }
  }
};

}  // namespace kla
