// kla_bwd.hip -- gradients of the chunkwise KLA forward for gfx950.
//
// "Resumen Técnico: Atención Lineal Kaczmarz (KLA)" (gist.science/es/paper/2605.08587),
// §"Implementación": KLA keeps Gated DeltaNet's parallel chunk training algorithm and
// changes only the diagonal coefficient matrix Diag(beta) inside it.  This file is the
// reverse mode of that chunk algorithm.  Per chunk of C tokens with start state S
// (gamma = running sum of g in the chunk, Gam = exp(gamma), d_r = exp(gamma_C - gamma_r),
// E_rs = exp(gamma_r - gamma_s)):
//
//   forward                                   reverse (dS' = dL/d(chunk-end state))
//   A  = strictly-lower(Diag(b) K K^T . E)     dU  = P^T dO + Diag(d) K dS'
//   T  = (I + A)^-1,  W = T Diag(b)            dX  = W^T dU  (= dV)
//   P  = lower(Q K^T . E)                      dP  = dO U^T,   dW = dU X^T
//   X  = V - Diag(Gam) K S,   U = W X          dS  = Gam_C dS' + (Diag(Gam) Q)^T dO - (Diag(Gam) K)^T dX
//   O  = Diag(Gam) Q S + P U                   dA  = -T^T (dW Diag(b)) T^T   (strictly lower)
//   S' = Gam_C S + K^T Diag(d) U               then dQ, dK, db, dgamma from A, P, X, O, S'
//
// The passes, through a caller-provided workspace:
//   states   the chunk-start states, in order: the forward's own pipelined prep and
//            scan kernels (kla_chunk.hip) in states mode, which write the state at
//            the start of every chunk instead of the outputs.  On the bf16 build the
//            forward prep also leaves its T'^T images (with gamma, Gam, d) and a T^T
//            image of every chunk in the workspace.
//   dstates  dS' of every chunk, in reverse order, by the forward's machinery run as
//            the adjoint scan (kla_chunk.hip, kla_chunk_rev_kernel); the gradient of
//            the initial state is what is left at the start.  On the bf16 build it
//            runs beside the states scan, on a second stream, when both fit one round
//            of workgroups.
//   grads    (chunk, head) in parallel: everything else from S, dS' and the chunk's
//            inputs.  bf16 (chunk 64): kla_bwd_grads2_kernel, over blocks of 64 state
//            columns on 16x16x32 bf16 MFMA, with P, ||k||^2 and b formed from the K
//            and Q rows.  fp32: kla_bwd_prep_kernel first writes b, gamma, ||k||^2, T,
//            P and K K^T . E per (chunk, head), then kla_bwd_grads_kernel streams the
//            state columns 16 at a time on fp32 MFMA (16x16x16 steps as four 16x16x4).
// Sums are fp32 throughout.  There are no atomics, so results are deterministic run
// to run.
#include <mutex>
#include <algorithm>

#include "kla_common.h"
#include "kla_internal.h"
#include "kla_ops.h"

namespace kla {

namespace {

constexpr int kBT = 256;  // default thread count of the tile loaders
constexpr int kGT = 512;  // threads per workgroup of the gradient kernel
constexpr int kNT = 512;  // threads per workgroup of the prep and the two scan kernels
constexpr int kNS = 16;   // state columns per slice
// LDS row strides are multiples of 4 floats so that four consecutive entries of a row are
// one 16-byte read; 4 rows apart is then 16 (mod 64) banks, which keeps the column
// gathers (16 lanes along a row, lane groups 4 rows apart) free of bank conflicts too
constexpr int kLS = kNS + 4;

struct BwdParams {
  const void *q, *k, *v, *g, *eta, *dout;
  float eps;
  const float *s0, *dsfin;
  void *dq, *dk, *dv;
  float *dg, *deta, *ds0;
  const int32_t *cu;
  float *prep;
  void *states, *dstates;  // chunk-start states and chunk-end state gradients, input element type
  const char *fws;         // the forward workspace: T'^T images and gamma, Gam, d per (head, slot)
  const char *timg;        // bf16, chunk 64: the packed T^T images per (head, slot), else nullptr
  int B, H, T, DV, nseq, nslot, nsl;
  int beta_direct;
};

// Per (head, slot) record of the prep kernel: T = (I + A)^-1, P = lower(Q K^T . E) and
// lower(K K^T . E), C x C row-major in the input element type (the bf16 path feeds them to
// bf16 MFMA steps, so a wider copy would only be rounded again on the way in), then b,
// gamma (rows past the chunk's end hold the last value) and ||k||^2 as fp32, and a spare row.
template <typename E, int C> struct PrepRec {
  static constexpr int TM = 0, PM = C * C, GE = 2 * C * C;            // E elements
  static constexpr size_t MAT = 3 * (size_t)C * C * sizeof(E);        // bytes of the matrices
  static constexpr int BETA = 0, GAM = C, NRM = 2 * C, VEC = 4 * C;   // floats after them
  static constexpr size_t BYTES = MAT + VEC * 4;
  static_assert(MAT % 16 == 0 && BYTES % 16 == 0, "16-byte aligned records");
  static __device__ __forceinline__ char *at(float *base, size_t idx) {
    return reinterpret_cast<char *>(base) + idx * BYTES;
  }
  static __device__ __forceinline__ E *mat(char *r) { return reinterpret_cast<E *>(r); }
  static __device__ __forceinline__ float *vec(char *r) { return reinterpret_cast<float *>(r + MAT); }
};

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return min(max(x, lo), hi); }

// Slot of chunk c of sequence n (as the forward workspace): dense batches use
// n * ceil(T/C) + c, packed sequences n + floor(t0_n / C) + c.
struct SeqLoc {
  long long row0;  // token row of the sequence's first token in [B*H*T]
  int len, slot0;
};

__device__ __forceinline__ SeqLoc seq_loc(const BwdParams &p, int n, int h, int C) {
  if (p.cu) {
    const int t0 = clampi(p.cu[n], 0, p.T);
    const int t1 = clampi(p.cu[n + 1], t0, p.T);
    return {(long long)h * p.T + t0, t1 - t0, n + t0 / C};
  }
  const int nchT = (p.T + C - 1) / C;
  return {((long long)n * p.H + h) * p.T, p.T, n * nchT};
}

struct ChunkLoc {
  long long row0;  // token row of the chunk's first token
  int rows;        // tokens in the chunk, 0 if the slot holds no chunk
};

__device__ __forceinline__ ChunkLoc chunk_loc(const BwdParams &p, int slot, int h, int C) {
  int b = 0, t0 = 0, len = p.T, c = slot;
  if (p.cu) {
    // the sequence n with n + floor(cu[n] / C) <= slot (strictly increasing in n)
    int lo = 0, hi = p.nseq - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (mid + clampi(p.cu[mid], 0, p.T) / C <= slot) lo = mid; else hi = mid - 1;
    }
    t0 = clampi(p.cu[lo], 0, p.T);
    len = clampi(p.cu[lo + 1], t0, p.T) - t0;
    c = slot - (lo + t0 / C);
  } else {
    const int nchT = (p.T + C - 1) / C;
    b = slot / nchT;
    c = slot % nchT;
  }
  const bool ok = c >= 0 && c * C < len;
  return {((long long)b * p.H + h) * p.T + t0 + (long long)c * C, ok ? min(C, len - c * C) : 0};
}

template <typename E>
__device__ __forceinline__ float ld(const void *base, long long i) {
  return Elem<E>::to_f32(static_cast<const E *>(base)[i]);
}

// An [R x D] tile of a row-major array (row stride `ld` elements) moved as
// 16-byte vectors: issue() loads this thread's vectors into registers (all of
// them before any is used, so their latencies overlap), put() widens them to
// fp32 into LDS rows of stride LD.  Rows at or past `rows` read as zero.
template <typename E, int R, int D, int LD, int NT = kBT>
struct TileLoad {
  static constexpr int EPV = 16 / (int)sizeof(E);  // elements per vector
  static constexpr int VPR = D / EPV;              // vectors per row
  static constexpr int NV = R * VPR;
  static constexpr int PER = (NV + NT - 1) / NT;
  static_assert(D % EPV == 0, "rows are whole 16-byte vectors");
  uint4 v[PER];

  __device__ __forceinline__ void issue(const void *src, long long row0, int rows, int col0, long long ld) {
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int idx = (int)threadIdx.x + m * NT;
      const int r = idx / VPR, c = (idx % VPR) * EPV;
      v[m] = make_uint4(0u, 0u, 0u, 0u);
      if (idx < NV && r < rows)
        v[m] = *reinterpret_cast<const uint4 *>(static_cast<const E *>(src) + (row0 + r) * ld + col0 + c);
    }
  }
  __device__ __forceinline__ void put(float *dst) const {
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int idx = (int)threadIdx.x + m * NT;
      if (idx < NV) {
        const int r = idx / VPR, c = (idx % VPR) * EPV;
        const E *e = reinterpret_cast<const E *>(&v[m]);
#pragma unroll
        for (int u = 0; u < EPV; ++u) dst[r * LD + c + u] = Elem<E>::to_f32(e[u]);
      }
    }
  }
};

// Rows [0, rows) of a [*, D] array from row `row0` into LDS with row stride LD,
// zeros past `rows` (one batch of vector loads).
template <typename E, int R, int D, int LD, int NT = kBT>
__device__ __forceinline__ void load_rows(float *dst, const void *src, long long row0, int rows, int col0,
                                          long long ld_src) {
  TileLoad<E, R, D, LD, NT> tl;
  tl.issue(src, row0, rows, col0, ld_src);
  tl.put(dst);
}

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// One 16x16x16 product step of the fp32 build's prep and gradient kernels, operands as
// four fp32 values per lane: a[x] = A[row][k0 + 4 lg + x], b[x] = B[k0 + 4 lg + x][col],
// run as four 16x16x4 fp32 MFMAs with the same pairing of contraction indices.  (The
// bf16 build's gradient kernel takes its operands from bf16 LDS rows instead.)
template <typename E> struct Mma16;

template <> struct Mma16<float> {
  static __device__ __forceinline__ f32x4 run(f32x4 a, f32x4 b, f32x4 c) {
#pragma unroll
    for (int x = 0; x < 4; ++x) c = mfma4(a[x], b[x], c);
    return c;
  }
};

// four LDS floats p[0], p[st], p[2 st], p[3 st]; and four consecutive 16-byte aligned ones
__device__ __forceinline__ f32x4 gat4(const float *p, int st) { return f32x4{p[0], p[st], p[2 * st], p[3 * st]}; }
__device__ __forceinline__ f32x4 vec4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }

// ============================================================================
// prep (fp32 build): b, gamma, ||k||^2, T = (I + A)^-1 and P for one (chunk, head)
// ============================================================================
// Four waves.  K K^T and Q K^T run on fp32 MFMA: the lower-triangular 16x16
// tiles split by row blocks {p, NB-1-p} over two waves per product, so a Gram
// wave computes the diagonal tile -- hence the norms and b -- of every row it
// needs.  T = (I + A)^-1 by 16x16 blocks: the diagonal blocks by column-parallel
// forward substitution (one lane per column, one block per 16 lanes), then the
// blocks below the diagonal level by level, T_ij = -T_ii sum_{j<=m<i} A_im T_mj,
// as 16x16x16 fp32 MFMA products.
constexpr int kPT = 256;  // threads per workgroup of the prep kernel

// one 16x16 tile of A B^T, rows of A and B (stride LK) from the given pointers
template <typename E, int DK, int LK> struct PrepTile;

template <int DK, int LK> struct PrepTile<float, DK, LK> {
  static __device__ __forceinline__ f32x4 run(const float *A, const float *B, int lr, int lg) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k0 = 0; k0 < DK; k0 += 16) {
      const f32x4 a = *reinterpret_cast<const f32x4 *>(A + lr * LK + k0 + 4 * lg);
      const f32x4 b = *reinterpret_cast<const f32x4 *>(B + lr * LK + k0 + 4 * lg);
#pragma unroll
      for (int x = 0; x < 4; ++x) acc = mfma4(a[x], b[x], acc);
    }
    return acc;
  }
};

template <typename E, int C, int DK>
struct PrepSmem {
  static constexpr int EPV = 16 / (int)sizeof(E);     // elements per 16-byte vector
  static constexpr int LK = DK + EPV;                  // K, Q rows (elements), 16-byte padded
  static constexpr int LC = C + 4;                     // A, T rows (floats)
  static constexpr int KB = C * LK * (int)sizeof(E);   // bytes of the K (or Q) image
  static constexpr int AB = C * LC * 4;                // bytes of A (or T)
  // K, then Q; T reuses Q's bytes once the scores are out, then A
  static constexpr int K = 0, Q = KB, T = KB, A = KB + (KB > AB ? KB : AB);
  static constexpr int BYTES = A + AB;
};

template <typename E, int C, int DK>
__global__ __launch_bounds__(kPT) void kla_bwd_prep_kernel(BwdParams p) {
  using L = PrepSmem<E, C, DK>;
  using R = PrepRec<E, C>;
  using MM = PrepTile<E, DK, L::LK>;
  constexpr int LK = L::LK, LC = L::LC, NB = C / 16, EPV = L::EPV, VPR = DK / EPV;
  static_assert(C <= 64 && C % 16 == 0 && DK % (4 * EPV) == 0, "tile shapes");
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  E *sK = reinterpret_cast<E *>(smem + L::K), *sQ = reinterpret_cast<E *>(smem + L::Q);
  float *sT = reinterpret_cast<float *>(smem + L::T), *sA = reinterpret_cast<float *>(smem + L::A);
  const int slot = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int w = t >> 6, lane = t & 63, lr = lane & 15, lg = lane >> 4;
  const ChunkLoc cl = chunk_loc(p, slot, h, C);
  if (cl.rows == 0) return;  // uniform: no chunk behind this slot
  const int rows = cl.rows;
  char *recb = R::at(p.prep, (size_t)h * p.nslot + slot);
  E *rm = R::mat(recb);
  float *rv = R::vec(recb);

  // K and Q rows as stored (16-byte vectors; rows past the chunk read as zero)
  for (int idx = t; idx < 2 * C * VPR; idx += kPT) {
    const int m = idx / (C * VPR), e = idx % (C * VPR), r = e / VPR, c = (e % VPR) * EPV;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r < rows) v = ldg16(static_cast<const E *>(m ? p.q : p.k) + (cl.row0 + r) * DK + c);
    *reinterpret_cast<uint4 *>((m ? sQ : sK) + r * LK + c) = v;
  }
  // gate prefix gamma (lane r holds gamma_r; rows past the chunk add zero) and eta
  float gam = lane < rows ? ld<E>(p.g, cl.row0 + lane) : 0.f;
  const float eta = lane < rows ? ld<E>(p.eta, cl.row0 + lane) : 0.f;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float u = __shfl_up(gam, off);
    if (lane >= off) gam += u;
  }
  if (w == 0 && lane < C) rv[R::GAM + lane] = gam;
  __syncthreads();

  // K K^T (waves 0, 1) and Q K^T (waves 2, 3) by row blocks {p, NB-1-p}
  const int pw = w & 1;
  const bool gram = w < 2;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int Rb = pass ? NB - 1 - pw : pw;
    if (Rb < 0 || Rb >= NB || (pass && Rb == pw)) continue;  // uniform per wave
    const float gr = __shfl(gam, 16 * Rb + 4 * lg), gr1 = __shfl(gam, 16 * Rb + 4 * lg + 1);
    const float gr2 = __shfl(gam, 16 * Rb + 4 * lg + 2), gr3 = __shfl(gam, 16 * Rb + 4 * lg + 3);
    const float grow[4] = {gr, gr1, gr2, gr3};
    float brow[4] = {0.f, 0.f, 0.f, 0.f};
    if (gram) {
      // diagonal tile first: the norms and b of this block's rows
      const f32x4 d = MM::run(sK + 16 * Rb * LK, sK + 16 * Rb * LK, lr, lg);
      const float dg = d[lr & 3];  // the diagonal entry when lg == lr >> 2
      const float nrm = __shfl(dg, lr + 16 * (lr >> 2));  // ||k||^2 of row 16 Rb + lr
      const float et = __shfl(eta, 16 * Rb + lr);
      const int r = 16 * Rb + lr;
      const float b = r >= rows ? 0.f : (p.beta_direct ? et : et / (nrm + p.eps));
      if (lg == 0) {
        rv[R::NRM + r] = nrm;
        rv[R::BETA + r] = b;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) brow[i] = __shfl(b, 4 * lg + i);
    }
    const E *rowsA = (gram ? sK : sQ) + 16 * Rb * LK;
    E *out = rm + (gram ? R::GE : R::PM);
    for (int Sb = 0; Sb < NB; ++Sb) {
      const int s = 16 * Sb + lr;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (Sb <= Rb) v = MM::run(rowsA, sK + 16 * Sb * LK, lr, lg);
      const float gc = __shfl(gam, s);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * Rb + 4 * lg + i;
        // mask before the exponential: only s <= r is ever evaluated
        const float ex = s <= r ? __expf(grow[i] - gc) : 0.f;
        const float ge = v[i] * ex;
        out[r * C + s] = Elem<E>::from_f32(ge);
        if (gram && Sb <= Rb) sA[r * LC + s] = s < r ? brow[i] * ge : 0.f;
      }
    }
  }
  __syncthreads();  // A complete; Q no longer needed (T takes its place)

  // diagonal blocks: lane 16b + j solves column j of T_bb = (I + A_bb)^-1
  if (w == 0 && lg < NB) {
    const int b = lg, j = lr;
    const float *Ab = sA + 16 * b * LC + 16 * b;
    float tc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) tc[r] = r == j ? 1.f : 0.f;
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int s4 = 0; s4 < r; s4 += 4) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(Ab + r * LC + s4);
#pragma unroll
        for (int x = 0; x < 4; ++x)
          if (s4 + x < r) acc = fmaf(a[x], tc[s4 + x], acc);
      }
      if (r > j) tc[r] = -acc;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sT[(16 * b + r) * LC + 16 * b + j] = tc[r];
  }
  __syncthreads();
  // blocks below the diagonal, level by level: wave w takes block (L + w, w)
  for (int Lv = 1; Lv < NB; ++Lv) {
    const int bi = Lv + w, bj = w;
    if (bi < NB) {
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
      for (int m = bj; m < bi; ++m) {
        // Y += A_im T_mj, contraction index 4 lg + x
        const f32x4 a = *reinterpret_cast<const f32x4 *>(sA + (16 * bi + lr) * LC + 16 * m + 4 * lg);
#pragma unroll
        for (int x = 0; x < 4; ++x) y = mfma4(a[x], sT[(16 * m + 4 * lg + x) * LC + 16 * bj + lr], y);
      }
      // Z = T_ii Y: lane (lr, lg) holds Y[4 lg + x][lr], the B operand of step x as it stands
      const f32x4 a = *reinterpret_cast<const f32x4 *>(sT + (16 * bi + lr) * LC + 16 * bi + 4 * lg);
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int x = 0; x < 4; ++x) z = mfma4(a[x], y[x], z);
#pragma unroll
      for (int i = 0; i < 4; ++i) sT[(16 * bi + 4 * lg + i) * LC + 16 * bj + lr] = -z[i];
    }
    __syncthreads();
  }
  // T to the record, zero above the diagonal blocks
  for (int e = t; e < C * C / 4; e += kPT) {
    const int r = (4 * e) / C, s = (4 * e) % C;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if ((s >> 4) <= (r >> 4)) v = *reinterpret_cast<const f32x4 *>(sT + r * LC + s);
    E *dt = rm + R::TM + 4 * e;
#pragma unroll
    for (int x = 0; x < 4; ++x) dt[x] = Elem<E>::from_f32(v[x]);
  }
}

// The two scans run their products as 16x16x16 steps (Mma16: lane l supplies
// A[l%16][4(l/16) .. +3] and B[4(l/16) .. +3][l%16]; accumulator element i of lane l
// is row 4(l/16)+i, column l%16).  The state slice (NS = 32 or 16 columns) lives in
// accumulators: wave w holds state rows 16w .. 16w+15 of its column tile and copies
// them to LDS once per chunk for the next chunk's K S (or K dS) product; chunk-row
// products (16-row tiles of C) are spread over the waves by (row tile, column tile).

// One 16-column slice of a chunk-start state stored in the forward scan's
// operand groups (kla_chunk.hip, ChunkParams::states): for each group q of KG
// state rows, 64 lanes x 16 bytes, lane l holding column l & 15 of the slice and
// rows (bf16, KG = 32) 32 q + 16 (x >> 2) + 4 (l >> 4) + (x & 3) or (fp32, KG = 16)
// 16 q + 4 (l >> 4) + x.  One contiguous block per slice, moved as 16-byte pieces
// and scattered into fp32 LDS rows of stride kLS.
template <typename E, int DK> struct GroupLoad {
  static constexpr int EPV = 16 / (int)sizeof(E);  // elements per piece (8 or 4)
  static constexpr int KG = sizeof(E) == 2 ? 32 : 16;
  static constexpr int NP = DK * kNS / EPV;        // pieces per slice
  static constexpr int PER = (NP + kGT - 1) / kGT;
  uint4 v[PER];
  // base: the chunk's states (DK x DV elements); slice js = columns 16 js ..
  __device__ __forceinline__ void issue(const E *base, int js) {
    const uint4 *src = reinterpret_cast<const uint4 *>(base + (size_t)js * DK * kNS);
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int pc = (int)threadIdx.x + m * kGT;
      if (pc < NP) v[m] = src[pc];
    }
  }
  __device__ __forceinline__ void put(float *dst) const {
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int pc = (int)threadIdx.x + m * kGT;
      if (pc < NP) {
        const int q = pc >> 6, l = pc & 63;
        const E *e = reinterpret_cast<const E *>(&v[m]);
#pragma unroll
        for (int x = 0; x < EPV; ++x) {
          const int row = KG == 32 ? 32 * q + 16 * (x >> 2) + 4 * (l >> 4) + (x & 3) : 16 * q + 4 * (l >> 4) + x;
          dst[row * kLS + (l & 15)] = Elem<E>::to_f32(e[x]);
        }
      }
    }
  }
};

// ============================================================================
// grads (fp32 build): dq, dk, dv, dg, deta of one (chunk, head)
// ============================================================================
// On 16x16x4 fp32 MFMA tiles: lane l supplies A[l%16][l/16] and B[l/16][l%16] of
// a 16x4 by 4x16 product; accumulator element i of lane l is row 4(l/16)+i,
// column l%16.  Wave w owns row tile w (16 chunk rows) of every product and every
// accumulator, so the per-slice phases need only two barriers.
template <int C, int DK>
struct GradSmem {
  // K and Q rows 16-byte aligned; a 16-row by 4-column operand read lands on 64
  // distinct banks (row stride = 4 mod 64)
  static constexpr int LK = DK + 4, LC = C + 4;
  static constexpr int K = 0, Q = K + C * LK, T = Q + C * LK, P = T + C * LC;  // P, later dEE
  static constexpr int SL = P + C * LC;                                      // slice region
  static constexpr int S = SL, D = S + DK * kLS, V = D + DK * kLS, O = V + C * kLS, X = O + C * kLS;
  static constexpr int U = X + C * kLS, DU = U + C * kLS, DX = DU + C * kLS, SL_END = DX + C * kLS;
  static constexpr int B1 = SL, B2 = SL + C * LC;  // C x C stage, over the slice region
  static constexpr int SL_SIZE = SL_END - SL > 2 * C * LC ? SL_END - SL : 2 * C * LC;
  static constexpr int VEC = SL + SL_SIZE;
  static constexpr int BETA = VEC, GAM = BETA + C, NRM = GAM + C, ETA = NRM + C, DGAM = ETA + C, DD = DGAM + C;
  static constexpr int DB1 = DD + C, DB2 = DB1 + C, DGE = DB2 + C, CF = DGE + C, GM = CF + C, DEC = GM + C;
  static constexpr int DB3 = DEC + C;  // the partner waves' part of the db row sums
  static constexpr int RED = DB3 + C;
  static constexpr int FLOATS = RED + kGT / 64;
};

template <typename E, int C, int DK>
__global__ __launch_bounds__(kGT) void kla_bwd_grads_kernel(BwdParams p) {
  using L = GradSmem<C, DK>;
  using R = PrepRec<E, C>;
  using MM = Mma16<E>;
  constexpr int LK = L::LK, LC = L::LC;
  constexpr int NRT = C / 16, NKT = DK / 16;
  constexpr int NKH = (NKT + 1) / 2;  // dQ, dK column tiles per wave: b = 2 i + half
  static_assert(C % 16 == 0 && DK % 16 == 0 && NRT <= 4 && kGT == 512, "a wave pair per 16-row tile");
  __shared__ __attribute__((aligned(16))) float sm[L::FLOATS];
  float *sK = sm + L::K, *sQ = sm + L::Q, *sT = sm + L::T, *sP = sm + L::P;
  float *sS = sm + L::S, *sD = sm + L::D, *sV = sm + L::V, *sO = sm + L::O, *sX = sm + L::X;
  float *sU = sm + L::U, *sdU = sm + L::DU, *sdX = sm + L::DX;
  float *sb = sm + L::BETA, *sgam = sm + L::GAM, *snrm = sm + L::NRM, *seta = sm + L::ETA;
  float *sdgam = sm + L::DGAM, *sdd = sm + L::DD, *sdb1 = sm + L::DB1, *sdb2 = sm + L::DB2;
  float *sdb3 = sm + L::DB3;
  float *sdge = sm + L::DGE, *scf = sm + L::CF, *sred = sm + L::RED, *sGm = sm + L::GM, *sdec = sm + L::DEC;
  const int slot = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const ChunkLoc cl = chunk_loc(p, slot, h, C);
  if (cl.rows == 0) return;  // uniform
  const int rows = cl.rows;
  const int w = t >> 6, lane = t & 63, lr = lane & 15, lg = lane >> 4;
  // waves w and w + 4 share row tile a = w & 3; the first of the pair (the lead) runs
  // the per-slice products and the C x C stage, and the pair splits the outer products
  const int a = w & 3, half = w >> 2;
  const bool own = a < NRT;        // (uniform per wave)
  const bool lead = own && half == 0;
  const int ra = 16 * a + lr;      // operand row of this lane
  const size_t sidx = (size_t)h * p.nslot + slot;
  char *recb = R::at(p.prep, sidx);
  const E *rm = R::mat(recb);
  const float *rv = R::vec(recb);
  const E *Sg = static_cast<const E *>(p.states) + sidx * DK * p.DV;
  const E *Dg = static_cast<const E *>(p.dstates) + sidx * DK * p.DV;

  {
    TileLoad<E, C, DK, LK, kGT> lk, lq;
    TileLoad<E, C, C, LC, kGT> lt, lp;
    TileLoad<float, 3, C, C, kGT> lb;  // b, gamma, ||k||^2 (adjacent in the record and in LDS)
    lk.issue(p.k, cl.row0, rows, 0, DK);
    lq.issue(p.q, cl.row0, rows, 0, DK);
    lt.issue(rm + R::TM, 0, C, 0, C);
    lp.issue(rm + R::PM, 0, C, 0, C);
    lb.issue(rv + R::BETA, 0, 3, 0, C);
    lk.put(sK);
    lq.put(sQ);
    lt.put(sT);
    lp.put(sP);
    lb.put(sb);
  }
  const float gC = rv[R::GAM + C - 1];
  for (int r = t; r < C; r += kGT) {
    seta[r] = r < rows ? ld<E>(p.eta, cl.row0 + r) : 0.f;
    sdgam[r] = 0.f;
    sdd[r] = 0.f;
    const float gr = rv[R::GAM + r];
    sGm[r] = __expf(gr);
    sdec[r] = __expf(gC - gr);
  }

  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 accWP[NRT], accQ[NKH], accK[NKH];  // accWP: dW (lead) or dP (its partner)
#pragma unroll
  for (int b = 0; b < NRT; ++b) accWP[b] = z4;
#pragma unroll
  for (int i = 0; i < NKH; ++i) accQ[i] = accK[i] = z4;
  float gcp = 0.f;  // partial <S, dS'>

  // slice js + 1 of S, dS', V and dO is loaded while slice js is computed
  GroupLoad<E, DK> ls, ld_;
  TileLoad<E, C, kNS, kLS, kGT> lv, lo;
  auto issue = [&](int js) {
    const int col0 = js * kNS;
    ls.issue(Sg, js);
    ld_.issue(Dg, js);
    lv.issue(p.v, cl.row0, rows, col0, p.DV);
    lo.issue(p.dout, cl.row0, rows, col0, p.DV);
  };
  issue(0);
  for (int js = 0; js < p.nsl; ++js) {
    const int col0 = js * kNS;
    __syncthreads();
    ls.put(sS);
    ld_.put(sD);
    lv.put(sV);
    lo.put(sO);
    if (js + 1 < p.nsl) issue(js + 1);
    __syncthreads();
    for (int e = t; e < DK * kNS; e += kGT) gcp = fmaf(sS[(e / kNS) * kLS + e % kNS], sD[(e / kNS) * kLS + e % kNS], gcp);
    // Phases A-C for row tile a, split over the wave pair: the lead forms K S, Q S, X, U
    // and dX (= dV) and the dGam row sums; its partner K dS', dU and the dd row sums.
    // (A) lead: K S, Q S and X = V - Diag(Gam) K S; partner: K dS'
    f32x4 ks = z4, qs = z4, kd = z4;
    if (lead) {
#pragma unroll 4
      for (int k0 = 0; k0 < DK; k0 += 16) {
        const int kk = k0 + 4 * lg;
        const f32x4 sv = gat4(sS + kk * kLS + lr, kLS);
        ks = MM::run(vec4(sK + ra * LK + kk), sv, ks);
        qs = MM::run(vec4(sQ + ra * LK + kk), sv, qs);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * a + 4 * lg + i;
        sX[r * kLS + lr] = sV[r * kLS + lr] - sGm[r] * ks[i];
      }
    } else if (own) {
#pragma unroll 4
      for (int k0 = 0; k0 < DK; k0 += 16) {
        const int kk = k0 + 4 * lg;
        kd = MM::run(vec4(sK + ra * LK + kk), gat4(sD + kk * kLS + lr, kLS), kd);
      }
    }
    __syncthreads();
    // (B) lead: U = T Diag(b) X; partner: dU = P^T dO + Diag(d) K dS'  (T, P lower triangular)
    if (lead) {
      f32x4 u = z4;
      for (int k0 = 0; k0 < 16 * (a + 1); k0 += 16) {
        const int s_ = k0 + 4 * lg;
        u = MM::run(vec4(sT + ra * LC + s_) * vec4(sb + s_), gat4(sX + s_ * kLS + lr, kLS), u);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sU[(16 * a + 4 * lg + i) * kLS + lr] = u[i];
    } else if (own) {
      f32x4 du = z4;
      for (int k0 = 16 * a; k0 < C; k0 += 16) {
        const int s_ = k0 + 4 * lg;
        du = MM::run(gat4(sP + s_ * LC + ra, LC), gat4(sO + s_ * kLS + lr, kLS), du);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * a + 4 * lg + i;
        sdU[r * kLS + lr] = fmaf(sdec[r], kd[i], du[i]);
      }
    }
    __syncthreads();
    // (C) lead: dX = Diag(b) T^T dU (= dV) and sum_c (Q S . dO - K S . dX);
    //     partner: sum_c (K dS' . U)
    if (lead) {
      f32x4 dx = z4;
      for (int k0 = 16 * a; k0 < C; k0 += 16) {
        const int s_ = k0 + 4 * lg;
        dx = MM::run(gat4(sT + s_ * LC + ra, LC), gat4(sdU + s_ * kLS + lr, kLS), dx);
      }
      float pg[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * a + 4 * lg + i;
        dx[i] *= sb[r];
        sdX[r * kLS + lr] = dx[i];
        if (r < rows) static_cast<E *>(p.dv)[(cl.row0 + r) * p.DV + col0 + lr] = Elem<E>::from_f32(dx[i]);
        pg[i] = qs[i] * sO[r * kLS + lr] - ks[i] * dx[i];
      }
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1)
#pragma unroll
        for (int i = 0; i < 4; ++i) pg[i] += __shfl_xor(pg[i], off);
      if (lr == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sdgam[16 * a + 4 * lg + i] += pg[i];
      }
    } else if (own) {
      float pd[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pd[i] = kd[i] * sU[(16 * a + 4 * lg + i) * kLS + lr];
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1)
#pragma unroll
        for (int i = 0; i < 4; ++i) pd[i] += __shfl_xor(pd[i], off);
      if (lr == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sdd[16 * a + 4 * lg + i] += pd[i];
      }
    }
    __syncthreads();  // the rows of dU, dX and U the lead waves wrote
    // (D) dW += dU X^T (lead), dP += dO U^T (partner; tiles at or below the diagonal),
    //     dQ += Diag(Gam) dO S^T, dK += -Diag(Gam) dX S^T + Diag(d) U dS'^T (split by column tile)
    static_assert(kNS == 16, "one 16x16x16 step per slice");
    if (own) {
      const int j = 4 * lg;
      const f32x4 ado = vec4(sO + ra * kLS + j);
      if (half == 0) {
        const f32x4 adu = vec4(sdU + ra * kLS + j);
#pragma unroll
        for (int b = 0; b < NRT; ++b) accWP[b] = MM::run(adu, vec4(sX + (16 * b + lr) * kLS + j), accWP[b]);
      } else {
#pragma unroll
        for (int b = 0; b < NRT; ++b)
          if (b <= a) accWP[b] = MM::run(ado, vec4(sU + (16 * b + lr) * kLS + j), accWP[b]);
      }
      const f32x4 aq = sGm[ra] * ado, akx = -sGm[ra] * vec4(sdX + ra * kLS + j);
      const f32x4 aku = sdec[ra] * vec4(sU + ra * kLS + j);
#pragma unroll
      for (int i = 0; i < NKH; ++i) {
        const int b = 2 * i + half;
        if (b < NKT) {
          const f32x4 sv = vec4(sS + (16 * b + lr) * kLS + j), dv = vec4(sD + (16 * b + lr) * kLS + j);
          accQ[i] = MM::run(aq, sv, accQ[i]);
          accK[i] = MM::run(aku, dv, MM::run(akx, sv, accK[i]));
        }
      }
    }
  }

  // ---------------- C x C stage ---------------------------------------------
  // (the slice region now holds B1 and B2; P stays in sP until dEE replaces it)
  float *B1 = sm + L::B1, *B2 = sm + L::B2;
  {
    float gs = gcp;  // <S, dS'>: one partial sum per wave
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) gs += __shfl_xor(gs, off);
    if (lane == 0) sred[w] = gs;
  }
  __syncthreads();
  if (own) {
#pragma unroll
    for (int b = 0; b < NRT; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * a + 4 * lg + i, s_ = 16 * b + lr;
        if (half == 0)
          B1[r * LC + s_] = accWP[b][i];                // dW
        else
          B2[r * LC + s_] = b <= a ? accWP[b][i] : 0.f;  // dP (entries above the diagonal masked below)
      }
  }
  __syncthreads();
  // db_s (first part) = sum_r T_rs dW_rs;  Y = (dW Diag(b)) T^T
  // (eight lanes per column, whole columns per wave: C is a multiple of 8)
  for (int s_ = t >> 3; s_ < C; s_ += kGT / 8) {
    float acc = 0.f;
    for (int r = s_ + (t & 7); r < C; r += 8) acc = fmaf(sT[r * LC + s_], B1[r * LC + s_], acc);
#pragma unroll
    for (int off = 4; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if ((t & 7) == 0) sdb1[s_] = acc;
  }
  // the wave pair of row tile a splits the C x C tiles: column block b goes to the wave
  // whose half equals b mod 2
  f32x4 y[NRT];
#pragma unroll
  for (int b = 0; b < NRT; ++b) y[b] = z4;
  if (own) {
#pragma unroll
    for (int b = 0; b < NRT; ++b) {
      if ((b & 1) != half) continue;
      // Y[r][s] = sum_{m <= s} dW[r][m] b_m T[s][m]
      for (int k0 = 0; k0 < 16 * (b + 1); k0 += 16) {
        const int m = k0 + 4 * lg;
        y[b] = MM::run(vec4(B1 + ra * LC + m) * vec4(sb + m), vec4(sT + (16 * b + lr) * LC + m), y[b]);
      }
    }
  }
  __syncthreads();
  if (own) {
#pragma unroll
    for (int b = 0; b < NRT; ++b)
      if ((b & 1) == half) {
#pragma unroll
        for (int i = 0; i < 4; ++i) B1[(16 * a + 4 * lg + i) * LC + 16 * b + lr] = y[b][i];  // Y over dW
      }
  }
  __syncthreads();
  // dA = -T^T Y (strictly lower); per entry dG = dA b_r E, dQK = dP E,
  // dEE = dA b_r (G . E) + dP P, db_r += dA (G . E)
  f32x4 dgm[NRT], dqk[NRT], dee[NRT];
  float dbr[4] = {0.f, 0.f, 0.f, 0.f};
  if (own) {
#pragma unroll
    for (int b = 0; b < NRT; ++b) {
      if ((b & 1) != half) continue;
      f32x4 da = z4;
      if (b <= a) {
        // dA[r][s] = -sum_{m >= r} T[m][r] Y[m][s]
        for (int k0 = 16 * a; k0 < C; k0 += 16) {
          const int m = k0 + 4 * lg;
          da = MM::run(gat4(sT + m * LC + ra, LC), gat4(B1 + m * LC + 16 * b + lr, LC), da);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * a + 4 * lg + i, s_ = 16 * b + lr;
        dgm[b][i] = dqk[b][i] = dee[b][i] = 0.f;
        if (s_ <= r) {
          const float ex = __expf(sgam[r] - sgam[s_]);
          const float dA = s_ < r ? -da[i] : 0.f;
          const float dP = B2[r * LC + s_];
          const float gE = Elem<E>::to_f32(rm[R::GE + r * C + s_]);
          dgm[b][i] = dA * sb[r] * ex;
          dqk[b][i] = dP * ex;
          dee[b][i] = fmaf(dA * sb[r], gE, dP * sP[r * LC + s_]);
          dbr[i] = fmaf(dA, gE, dbr[i]);
        }
      }
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1)
#pragma unroll
      for (int i = 0; i < 4; ++i) dbr[i] += __shfl_xor(dbr[i], off);
  }
  __syncthreads();
  if (own) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lr == 0) (half ? sdb3 : sdb2)[16 * a + 4 * lg + i] = dbr[i];
#pragma unroll
    for (int b = 0; b < NRT; ++b)
      if ((b & 1) == half) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * a + 4 * lg + i, s_ = 16 * b + lr;
          B1[r * LC + s_] = dgm[b][i];
          B2[r * LC + s_] = dqk[b][i];
          sP[r * LC + s_] = dee[b][i];
        }
      }
  }
  __syncthreads();
  if (own) {
    // dQ += dQK K;  dK += dQK^T Q + (dG + dG^T) K
    for (int k0 = 0; k0 < C; k0 += 16) {
      const int s_ = k0 + 4 * lg;
      const f32x4 aq = vec4(B2 + ra * LC + s_), at = gat4(B2 + s_ * LC + ra, LC);
      const f32x4 ag = vec4(B1 + ra * LC + s_) + gat4(B1 + s_ * LC + ra, LC);
#pragma unroll
      for (int i = 0; i < NKH; ++i) {
        const int b = 2 * i + half;
        if (b < NKT) {
          const f32x4 kv = gat4(sK + s_ * LK + 16 * b + lr, LK), qv = gat4(sQ + s_ * LK + 16 * b + lr, LK);
          accQ[i] = MM::run(aq, kv, accQ[i]);
          accK[i] = MM::run(ag, kv, MM::run(at, qv, accK[i]));
        }
      }
    }
  }
  // per-row scalars: dgamma, then dg = reverse running sum; db, deta, the norm term
  // (eight lanes per row, whole rows per wave: C is a multiple of 8)
  for (int r = t >> 3; r < C; r += kGT / 8) {
    const int j = t & 7;
    float rs = 0.f, cs = 0.f;
    for (int s_ = j; s_ < C; s_ += 8) {
      rs += sP[r * LC + s_];
      cs += sP[s_ * LC + r];
    }
#pragma unroll
    for (int off = 4; off >= 1; off >>= 1) {
      rs += __shfl_xor(rs, off);
      cs += __shfl_xor(cs, off);
    }
    if (j == 0) sdge[r] = sdgam[r] * sGm[r] - sdd[r] * sdec[r] + rs - cs;
  }
  __syncthreads();
  if (w == 0) {
    // the chunk-end terms go to the last row, then dg_r = sum_{r' >= r} dgamma_r' (lane r)
    float gcs = lane < kGT / 64 ? sred[lane] : 0.f;
    float ddd = lane < C ? sdd[lane] * sdec[lane] : 0.f;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      gcs += __shfl_xor(gcs, off);
      ddd += __shfl_xor(ddd, off);
    }
    float v = lane < C ? sdge[lane] : 0.f;
    if (lane == C - 1) v += gcs * __expf(gC) + ddd;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float u = __shfl_down(v, off);
      if (lane + off < 64) v += u;
    }
    if (lane < C) sdge[lane] = v;
  }
  for (int r = t; r < C; r += kGT) {
    const float db = sdb1[r] + sdb2[r] + sdb3[r];
    const float den = snrm[r] + p.eps;
    scf[r] = (p.beta_direct || r >= rows) ? 0.f : -2.f * seta[r] * db / (den * den);
    if (r < rows) p.deta[cl.row0 + r] = p.beta_direct ? db : db / den;
  }
  __syncthreads();
  for (int r = t; r < rows; r += kGT) p.dg[cl.row0 + r] = sdge[r];
  if (own) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * a + 4 * lg + i;
      if (r < rows) {
#pragma unroll
        for (int ii = 0; ii < NKH; ++ii) {
          const int b = 2 * ii + half;
          if (b < NKT) {
            const int c = 16 * b + lr;
            static_cast<E *>(p.dq)[(cl.row0 + r) * DK + c] = Elem<E>::from_f32(accQ[ii][i]);
            static_cast<E *>(p.dk)[(cl.row0 + r) * DK + c] =
                Elem<E>::from_f32(fmaf(scf[r], sK[r * LK + c], accK[ii][i]));
          }
        }
      }
    }
  }
}

// ============================================================================
// grads, bf16: the same gradients on the chunk kernels' operand machinery
// ============================================================================
// One workgroup of eight waves per (chunk, head), as the kernel above, but the
// per-column work runs over blocks of 64 state columns (two for dv = 128, not
// eight slices of 16), every product is a 16x16x32 bf16 MFMA whose operands
// come straight from bf16 LDS rows in the grouped column order of kla_ops.h
// (row reads for contractions along a row, transposing reads for contractions
// down a column).  No prep record: T'^T with gamma, Gam, d is the forward prep
// kernel's image of the chunk (the forward workspace), so T' X and T'^T dU read
// it as the forward and the adjoint scans do; T^T (without beta) is the second
// image the same kernel writes in states mode; P = lower(Q K^T . E), ||k||^2
// and b are formed here from the K and Q rows in LDS.  Waves w and w + 4 share
// row tile w & 3 (16 chunk rows); in the per-block phases each takes two of the
// block's four 16-column tiles; tile (a, b) of a C x C product belongs to the
// wave of row tile a with half = b & 1; dQ, dK column tile b to half b & 1.
//
// The state blocks are kept transposed (S^T, dS'^T: a row per state column,
// grouped over dk), where a 16-byte piece of the operand-group layout the
// states kernels write is one group of a row, so it is stored whole.
// Per block of columns J (S, dS' the chunk-start state and chunk-end state
// gradient restricted to J; V, dO likewise):
//   (A) K S, Q S, K dS'; X = V - Diag(Gam) K S; dU = P^T dO + Diag(d) K dS'
//   (B) U = T' X; dX = T'^T dU (= dV); row sums for dgamma and dd
//   (D) dW += dU X^T, dP += dO U^T, dQ += dO S^T, dK += -Diag(Gam) dX S^T + Diag(d) U dS'^T
template <int DK>
struct Grad2Smem {
  static constexpr int C = 64, JB = 64;
  using TL = TpLayout<bf16, 64>;
  static constexpr int PAD = LdsPad<bf16>::V;
  static constexpr int LDK = DK + PAD;   // K, Q rows
  static constexpr int LDC = TL::LDC;    // T'^T image and P rows
  static constexpr int LDJ = JB + PAD;   // rows of the block arrays
  static constexpr int K = 0;
  static constexpr int Q = K + C * LDK * 2;
  static constexpr int TP = Q + C * LDK * 2;         // T'^T image, then gamma, Gam, d (fp32)
  static constexpr int P = TP + TL::LDS_BYTES;
  static constexpr int S = P + C * LDC * 2;         // S^T of the block: JB rows of DK
  static constexpr int DS = S + JB * LDK * 2;        // dS'^T likewise
  static constexpr int VX = DS + JB * LDK * 2;       // V, then X
  static constexpr int DO = VX + C * LDJ * 2;
  static constexpr int U = DO + C * LDJ * 2;
  static constexpr int UD = U + C * LDJ * 2;         // Diag(d) U
  static constexpr int DU = UD + C * LDJ * 2;
  static constexpr int GX = DU + C * LDJ * 2;        // -Diag(Gam) dX
  static constexpr int BLK_END = GX + C * LDJ * 2;
  // the C x C stage reuses the block arrays: the T^T image, dW, Y, dQK, dG (bf16, grouped
  // columns), dP (fp32), then the per-tile partial sums; dQ, dK are staged (bf16, natural
  // rows) over T .. dQK once those are read
  static constexpr int LCF = C + 4, LDO = DK + 8;
  static constexpr int CT = S, CW = CT + C * LDC * 2, CY = CW + C * LDC * 2, CQK = CY + C * LDC * 2;
  static constexpr int CG = CQK + C * LDC * 2, CDP = CG + C * LDC * 2, CPART = CDP + C * LCF * 4;
  static constexpr int PROW = 0, PCOL = 2 * C, PDB = 6 * C, PCT = 8 * C, NPART = 12 * C;  // floats
  static constexpr int C_END = CPART + NPART * 4;
  static constexpr int SDQ = CT, SDK = SDQ + C * LDO * 2;
  static_assert(SDK + C * LDO * 2 <= CG, "the staged dQ, dK stay clear of dG, dP and the partial sums");
  static_assert(CDP % 16 == 0 && CPART % 16 == 0, "align");
  static constexpr int VEC = (BLK_END > C_END ? BLK_END : C_END);   // fp32 vectors, kept throughout
  static constexpr int BETA = 0, GAM = BETA + C, NRM = GAM + C, ETA = NRM + C, DGAM = ETA + C, DD = DGAM + 2 * C;
  static constexpr int CF = DD + 2 * C, GM = CF + C;
  static constexpr int DEC = GM + C, RED = DEC + C, NVEC = RED + kGT / 64;
  static constexpr int BYTES = VEC + NVEC * 4;
  static_assert(BYTES <= 160 * 1024, "LDS budget");
  static_assert(TP % 16 == 0 && P % 16 == 0 && S % 16 == 0 && VX % 16 == 0 && GX % 16 == 0 && VEC % 16 == 0, "align");
};

template <int DK>
__global__ __launch_bounds__(kGT) void kla_bwd_grads2_kernel(BwdParams p) {
  using L = Grad2Smem<DK>;
  using O = Ops<bf16>;
  using Grp = O::Grp;
  using TLy = TpLayout<bf16, 64>;
  constexpr int C = 64, NRT = 4, NKT = DK / 16, NKH = (NKT + 1) / 2, NQG = DK / 32, JB = L::JB;
  constexpr int LDK = L::LDK, LDC = L::LDC, LDJ = L::LDJ, LCF = L::LCF, LDO = L::LDO;
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  bf16 *bK = reinterpret_cast<bf16 *>(smem + L::K), *bQ = reinterpret_cast<bf16 *>(smem + L::Q);
  bf16 *bTp = reinterpret_cast<bf16 *>(smem + L::TP), *bP = reinterpret_cast<bf16 *>(smem + L::P);
  const float *fvec = reinterpret_cast<const float *>(smem + L::TP + TLy::TP_IMG);  // gamma, Gam, d
  bf16 *bS = reinterpret_cast<bf16 *>(smem + L::S), *bD = reinterpret_cast<bf16 *>(smem + L::DS);
  bf16 *bVX = reinterpret_cast<bf16 *>(smem + L::VX), *bO = reinterpret_cast<bf16 *>(smem + L::DO);
  bf16 *bU = reinterpret_cast<bf16 *>(smem + L::U), *bUD = reinterpret_cast<bf16 *>(smem + L::UD);
  bf16 *bDU = reinterpret_cast<bf16 *>(smem + L::DU), *bGX = reinterpret_cast<bf16 *>(smem + L::GX);
  float *vec = reinterpret_cast<float *>(smem + L::VEC);
  float *sb = vec + L::BETA, *sgam = vec + L::GAM, *snrm = vec + L::NRM, *seta = vec + L::ETA;
  float *sdgam2 = vec + L::DGAM, *sdd2 = vec + L::DD;  // per half of the column tiles
  float *scf = vec + L::CF;
  float *sGm = vec + L::GM, *sdec = vec + L::DEC, *sred = vec + L::RED;

  const int slot = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const ChunkLoc cl = chunk_loc(p, slot, h, C);
  if (cl.rows == 0) return;  // uniform
  const int rows = cl.rows;
  const int w = t >> 6, lane = t & 63, lr = lane & 15, lg = lane >> 4;
  const int a = w & 3, half = w >> 2;
  const bool own = true, lead = half == 0;
  const int ra = 16 * a + lr;
  const size_t sidx = (size_t)h * p.nslot + slot;
  const float *gv = reinterpret_cast<const float *>(p.fws + sidx * TLy::BYTES + TLy::PACK);  // gamma, Gam, d
  const bf16 *Sg = static_cast<const bf16 *>(p.states) + sidx * DK * p.DV;
  const bf16 *Dg = static_cast<const bf16 *>(p.dstates) + sidx * DK * p.DV;
  const int ntile = p.DV / 16;                 // 16-column tiles of the state
  const int nblk = (ntile + 3) / 4;

  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 accWP[NRT], accQ[NKH], accK[NKH];  // accWP: dW (half 0) or dP (half 1)
#pragma unroll
  for (int b = 0; b < NRT; ++b) accWP[b] = z4;
#pragma unroll
  for (int i = 0; i < NKH; ++i) accQ[i] = accK[i] = z4;
  float gcp = 0.f;  // partial <S, dS'>

  // ---- block loads: S, dS' pieces (operand groups), V and dO rows ----------
  // S, dS' of a block: tiles 4 blk .. (up to 4), groups q of 32 rows, 64 lanes of 16 bytes
  constexpr int SPIECES = 4 * NQG * 64;           // pieces of a full block
  constexpr int SPER = (SPIECES + kGT - 1) / kGT;
  uint4 sv[SPER], dv[SPER], vv, ov, tv;  // tv: a 16-byte piece of T (for the C x C stage)
  auto issue = [&](int blk) {
    const int nt = min(4, ntile - 4 * blk);
#pragma unroll
    for (int m = 0; m < SPER; ++m) {
      const int pc = t + m * kGT;
      const int ct = pc / (NQG * 64);
      if (ct < nt) {
        const size_t off = ((size_t)(4 * blk + ct) * NQG) * 64 + (pc % (NQG * 64));  // 16-byte pieces
        sv[m] = reinterpret_cast<const uint4 *>(Sg)[off];
        dv[m] = reinterpret_cast<const uint4 *>(Dg)[off];
      }
    }
    // V and dO rows: 8 columns per piece
    const int r = t >> 3, m8 = t & 7;
    vv = ov = make_uint4(0u, 0u, 0u, 0u);
    if (r < rows && m8 < 2 * nt) {
      const size_t e = (size_t)(cl.row0 + r) * p.DV + JB * blk + 8 * m8;
      vv = *reinterpret_cast<const uint4 *>(static_cast<const bf16 *>(p.v) + e);
      ov = *reinterpret_cast<const uint4 *>(static_cast<const bf16 *>(p.dout) + e);
    }
  };
  auto put = [&](int blk) {
    const int nt = min(4, ntile - 4 * blk);
    if (nt < 4) {
      // a partial block: the missing columns of every block array read as zero
      for (int e = t; e < (JB - 16 * nt) * LDK; e += kGT) {
        bS[16 * nt * LDK + e] = bD[16 * nt * LDK + e] = (bf16)0.f;
      }
      for (int e = t; e < C * (JB - 16 * nt); e += kGT) {
        const int row = e / (JB - 16 * nt), col = O::perm(16 * nt + e % (JB - 16 * nt));
        bU[row * LDJ + col] = bUD[row * LDJ + col] = bDU[row * LDJ + col] = bGX[row * LDJ + col] = (bf16)0.f;
      }
    }
#pragma unroll
    for (int m = 0; m < SPER; ++m) {
      const int pc = t + m * kGT;
      const int ct = pc / (NQG * 64);
      if (ct < nt) {
        // state rows 32 q + 16 (x >> 2) + 4 (l >> 4) + (x & 3), column 16 ct + (l & 15):
        // group 32 q + 8 (l >> 4) of row 16 ct + (l & 15) of S^T
        const int q = (pc / 64) % NQG, l = pc & 63;
        const int off = (16 * ct + (l & 15)) * LDK + 32 * q + 8 * (l >> 4);
        *reinterpret_cast<uint4 *>(bS + off) = sv[m];
        *reinterpret_cast<uint4 *>(bD + off) = dv[m];
        const Grp es = __builtin_bit_cast(Grp, sv[m]), ed = __builtin_bit_cast(Grp, dv[m]);
#pragma unroll
        for (int x = 0; x < 8; ++x) gcp = fmaf((float)es[x], (float)ed[x], gcp);
      }
    }
    const int r = t >> 3, m8 = t & 7;
    O::st_piece(bVX + r * LDJ, m8, vv);
    O::st_piece(bO + r * LDJ, m8, ov);
  };
  // D-layout tile of a grouped block array: M[r16 + 4 lg + j][c0 + lr], j < 4
  auto col4g = [&](const bf16 *M, int r16, int c0) {
    const int x = (lane >> 2) & 3, a4 = lane & 3;
    const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4 *)(M + (r16 + 4 * lg + x) * LDJ + O::perm(c0 + 4 * a4)));
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
  };
  // four bf16 of a D tile into a grouped block array (rows r16 + 4 lg + j, column c0 + lr)
  auto put_d = [&](bf16 *M, int r16, int c0, f32x4 v, int ld = L::LDJ) {
    const int col = O::perm(c0 + lr);
#pragma unroll
    for (int j = 0; j < 4; ++j) M[(r16 + 4 * lg + j) * ld + col] = (bf16)v[j];
  };

  issue(0);  // the first block's loads fly with the chunk's
  // ---- the chunk's K, Q rows, P and T'^T image (grouped columns), vectors -----
  if (w < 2) {
    RowLoad<bf16, DK, AllBlocks<4>> rl;
    rl.issue(static_cast<const bf16 *>(w == 0 ? p.k : p.q) + cl.row0 * DK, rows, lane);
    rl.put(w == 0 ? bK : bQ, LDK, lane, [](int, int row) { return row; });
  } else if (w == 2) {
    ImgCopy<bf16, 64> ic;
    ic.issue(p.fws + sidx * TLy::BYTES, lane);
    ic.put(bTp, lane);
  }
  for (int r = t; r < C; r += kGT) {
    sgam[r] = gv[r];
    sGm[r] = gv[C + r];
    sdec[r] = gv[2 * C + r];
    seta[r] = r < rows ? ld<bf16>(p.eta, cl.row0 + r) : 0.f;
    sdgam2[r] = sdgam2[C + r] = 0.f;
    sdd2[r] = sdd2[C + r] = 0.f;
  }
  const float gC = gv[C - 1];

  for (int blk = 0; blk < nblk; ++blk) {
    lds_barrier();  // the previous block's readers are done (and the chunk's loads are in LDS)
    if (blk == 0) {
      // (before the first block is stored: its loads are still in flight)
      // ||k_r||^2 and b_r (eight lanes per row); P = lower(Q K^T . E), tiles b <= a
      {
        const int r = t >> 3;
        float nr = 0.f;
#pragma unroll
        for (int m = 0; m < DK / 64; ++m) nr += O::sumsq(*reinterpret_cast<const Grp *>(bK + r * LDK + 8 * (t & 7) + 64 * m));
#pragma unroll
        for (int off = 4; off >= 1; off >>= 1) nr += __shfl_xor(nr, off);
        if ((t & 7) == 0) {
          snrm[r] = nr;
          sb[r] = r < rows ? (p.beta_direct ? seta[r] : seta[r] / (nr + p.eps)) : 0.f;
        }
      }
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int b = 2 * cc + half;
        f32x4 pv = z4;
        if (b <= a) {
#pragma unroll
          for (int q = 0; q < NQG; ++q)
            pv = O::mma_grp(O::a_row(bQ + ra * LDK, 32 * q, lg), O::a_row(bK + (16 * b + lr) * LDK, 32 * q, lg), pv);
          const int s_ = 16 * b + lr;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 16 * a + 4 * lg + j;
            pv[j] = s_ <= r ? pv[j] * __expf(sgam[r] - sgam[s_]) : 0.f;
          }
        }
        put_d(bP, 16 * a, 16 * b, pv, LDC);
      }
    }
    put(blk);
    if (blk + 1 < nblk)
      issue(blk + 1);
    else if (t < TLy::PACK / 16)
      tv = reinterpret_cast<const uint4 *>(p.timg + sidx * TLy::PACK)[t];  // the T^T image
    lds_barrier();
    const int nt = min(4, ntile - 4 * blk);
    // ---- (A) K S, Q S, K dS', X, dU for row tile a and column tiles 2 half, 2 half + 1 ----
    f32x4 ks[2], qs[2], kd[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int ct = 2 * half + cc;
      ks[cc] = qs[cc] = kd[cc] = z4;
      if (ct >= nt) continue;
#pragma unroll
      for (int q = 0; q < NQG; ++q) {
        const Grp bs = O::a_row(bS + (16 * ct + lr) * LDK, 32 * q, lg), bd = O::a_row(bD + (16 * ct + lr) * LDK, 32 * q, lg);
        const Grp ak = O::a_row(bK + ra * LDK, 32 * q, lg), aq = O::a_row(bQ + ra * LDK, 32 * q, lg);
        ks[cc] = O::mma_grp(ak, bs, ks[cc]);
        qs[cc] = O::mma_grp(aq, bs, qs[cc]);
        kd[cc] = O::mma_grp(ak, bd, kd[cc]);
      }
    }
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int ct = 2 * half + cc;
      if (ct >= nt) continue;
      // P^T dO (P lower triangular: row block a of P^T needs rows >= 16 a of P)
      f32x4 pd = z4;
#pragma unroll
      for (int q = 0; q < 2; ++q)
        if (q >= a / 2)
          pd = O::mma_grp(O::a_trans(bP, LDC, 32 * q, 16 * a, lane), O::a_trans(bO, LDJ, 32 * q, 16 * ct, lane), pd);
      const f32x4 v4 = col4g(bVX, 16 * a, 16 * ct);
      const f32x4 gm = *reinterpret_cast<const f32x4 *>(fvec + C + 16 * a + 4 * lg);
      const f32x4 d4 = *reinterpret_cast<const f32x4 *>(fvec + 2 * C + 16 * a + 4 * lg);
      // (a V tile is read and overwritten by X only by the wave that owns it)
      put_d(bVX, 16 * a, 16 * ct, v4 - gm * ks[cc]);
      put_d(bDU, 16 * a, 16 * ct, pd + d4 * kd[cc]);
    }
    lds_barrier();
    // ---- (B) U = T' X, dX = T'^T dU (= dV), row sums ----
    float pg[4] = {0.f, 0.f, 0.f, 0.f}, pdd[4] = {0.f, 0.f, 0.f, 0.f};
    // dX^T tiles for the dV stores: lane (lr, lg) holds dV[16 a + lr][16 ct + 4 lg + j]
    f32x4 dxt[2] = {z4, z4};
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int ct = 2 * half + cc;
      if (ct >= nt) continue;
      f32x4 u = z4, dx = z4;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if (32 * q < 16 * (a + 1))
          u = O::mma_grp(O::a_trans(bTp, LDC, 32 * q, 16 * a, lane), O::a_trans(bVX, LDJ, 32 * q, 16 * ct, lane), u);
        if (q >= a / 2) {
          const Grp tr = O::a_row(bTp + ra * LDC, 32 * q, lg), du = O::a_trans(bDU, LDJ, 32 * q, 16 * ct, lane);
          dx = O::mma_grp(tr, du, dx);
          dxt[cc] = O::mma_grp(du, tr, dxt[cc]);  // the operands swapped: the transposed tile
        }
      }
      const f32x4 gm = *reinterpret_cast<const f32x4 *>(fvec + C + 16 * a + 4 * lg);
      const f32x4 d4 = *reinterpret_cast<const f32x4 *>(fvec + 2 * C + 16 * a + 4 * lg);
      put_d(bU, 16 * a, 16 * ct, u);
      put_d(bUD, 16 * a, 16 * ct, d4 * u);
      put_d(bGX, 16 * a, 16 * ct, -(gm * dx));
      const f32x4 o4 = col4g(bO, 16 * a, 16 * ct);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pg[j] += qs[cc][j] * o4[j] - ks[cc][j] * dx[j];
        pdd[j] += kd[cc][j] * u[j];
      }
    }
    {
      // dV: the lanes lg = 2 m and 2 m + 1 of a row swap 8-byte halves so that the even
      // one holds columns 8 m .. 8 m + 7 of tile 2 half and the odd one those of tile
      // 2 half + 1; a row's 64 bytes then leave as four 16-byte stores
      const bf16x4 h0 = {(bf16)dxt[0][0], (bf16)dxt[0][1], (bf16)dxt[0][2], (bf16)dxt[0][3]};
      const bf16x4 h1 = {(bf16)dxt[1][0], (bf16)dxt[1][1], (bf16)dxt[1][2], (bf16)dxt[1][3]};
      const uint2 m0 = __builtin_bit_cast(uint2, h0), m1 = __builtin_bit_cast(uint2, h1);
      const bool odd = (lg & 1) != 0;
      const uint2 snd = odd ? m0 : m1;
      const uint2 rcv = make_uint2((unsigned)__shfl_xor((int)snd.x, 16), (unsigned)__shfl_xor((int)snd.y, 16));
      const uint4 piece = odd ? make_uint4(rcv.x, rcv.y, m1.x, m1.y) : make_uint4(m0.x, m0.y, rcv.x, rcv.y);
      const int ctp = 2 * half + (odd ? 1 : 0);
      const int r = 16 * a + lr;
      if (r < rows && ctp < nt)
        *reinterpret_cast<uint4 *>(static_cast<bf16 *>(p.dv) + (cl.row0 + r) * p.DV + JB * blk + 16 * ctp +
                                   8 * (lg >> 1)) = piece;
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pg[j] += __shfl_xor(pg[j], off);
        pdd[j] += __shfl_xor(pdd[j], off);
      }
    if (lr == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sdgam2[half * C + 16 * a + 4 * lg + j] += pg[j];
        sdd2[half * C + 16 * a + 4 * lg + j] += pdd[j];
      }
    }
    lds_barrier();
    // ---- (D) dW += dU X^T (half 0), dP += dO U^T (half 1, tiles at or below the diagonal),
    //      dQ += dO S^T, dK += GX S^T + UD dS'^T (column tiles b = 2 i + half) ----
#pragma unroll
    for (int q = 0; q < JB / 32; ++q) {
      if (32 * q >= 16 * nt) continue;
      const Grp adu = O::a_row(bDU + ra * LDJ, 32 * q, lg), ado = O::a_row(bO + ra * LDJ, 32 * q, lg);
      const Grp agx = O::a_row(bGX + ra * LDJ, 32 * q, lg), aud = O::a_row(bUD + ra * LDJ, 32 * q, lg);
      if (half == 0) {
#pragma unroll
        for (int b = 0; b < NRT; ++b) accWP[b] = O::mma_grp(adu, O::a_row(bVX + (16 * b + lr) * LDJ, 32 * q, lg), accWP[b]);
      } else {
#pragma unroll
        for (int b = 0; b < NRT; ++b)
          if (b <= a) accWP[b] = O::mma_grp(ado, O::a_row(bU + (16 * b + lr) * LDJ, 32 * q, lg), accWP[b]);
      }
#pragma unroll
      for (int i = 0; i < NKH; ++i) {
        const int b = 2 * i + half;
        if (b < NKT) {
          const Grp srow = O::a_trans(bS, LDK, 32 * q, 16 * b, lane);
          accQ[i] = O::mma_grp(ado, srow, accQ[i]);
          accK[i] = O::mma_grp(aud, O::a_trans(bD, LDK, 32 * q, 16 * b, lane), O::mma_grp(agx, srow, accK[i]));
        }
      }
    }
  }
  // dQ so far is dO S^T: rows scaled by Gam
  {
    const f32x4 gm = *reinterpret_cast<const f32x4 *>(fvec + C + 16 * a + 4 * lg);
#pragma unroll
    for (int i = 0; i < NKH; ++i) accQ[i] = gm * accQ[i];
  }
  {
    float gs = gcp;  // <S, dS'>: one partial sum per wave
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) gs += __shfl_xor(gs, off);
    if (lane == 0) sred[w] = gs;
  }
  lds_barrier();  // the block arrays are dead

  // ---------------- C x C stage ----------------------------------------------
  // With T = (I + A)^-1 (so T' = T Diag(b)), dW = dU X^T and dP = dO U^T:
  //   db_s  = sum_r T_rs dW_rs + sum_s' dA_ss' (G . E)_ss'
  //   Y     = dW T'^T,   dA = -T^T Y (strictly lower)
  //   dG    = Diag(b) dA . E,   dQK = dP . E,   dEE = Diag(b) dA . G . E + dP . P
  //   dQ   += dQK K,   dK += dQK^T Q + (dG + dG^T) K
  //   dgamma_r += sum_s dEE_rs - sum_s dEE_sr
  // Tile (a, b) of a C x C product belongs to the wave of row tile a with half = b & 1.
  for (int r = t; r < C; r += kGT) {
    sdgam2[r] += sdgam2[C + r];
    sdd2[r] += sdd2[C + r];
  }
  const float *sdgam = sdgam2, *sdd = sdd2;
  bf16 *cT = reinterpret_cast<bf16 *>(smem + L::CT), *cW = reinterpret_cast<bf16 *>(smem + L::CW);
  bf16 *cY = reinterpret_cast<bf16 *>(smem + L::CY), *cQK = reinterpret_cast<bf16 *>(smem + L::CQK);
  bf16 *cG = reinterpret_cast<bf16 *>(smem + L::CG);
  float *cdP = reinterpret_cast<float *>(smem + L::CDP), *part = reinterpret_cast<float *>(smem + L::CPART);
  float *prow = part + L::PROW, *pcol = part + L::PCOL, *pdb = part + L::PDB, *pct = part + L::PCT;
  if (t < TLy::PACK / 16) *reinterpret_cast<uint4 *>(cT + TLy::piece_to_lds(t)) = tv;  // T^T
  for (int e = t; e < L::NPART; e += kGT) part[e] = 0.f;
  if (half == 0) {
#pragma unroll
    for (int b = 0; b < NRT; ++b) put_d(cW, 16 * a, 16 * b, accWP[b], LDC);
  } else {
#pragma unroll
    for (int b = 0; b < NRT; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) cdP[(16 * a + 4 * lg + j) * LCF + 16 * b + lr] = b <= a ? accWP[b][j] : 0.f;
  }
  lds_barrier();
  // Y tiles; the column sums of T . dW (the dW tiles are still in the half-0 registers)
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    const int b = 2 * cc + half;
    f32x4 y = z4;
#pragma unroll
    for (int q = 0; q < 2; ++q)  // T'^T rows m <= s: contraction block q reaches column tile b
      if (32 * q < 16 * (b + 1))
        y = O::mma_grp(O::a_row(cW + ra * LDC, 32 * q, lg), O::a_trans(bTp, LDC, 32 * q, 16 * b, lane), y);
    put_d(cY, 16 * a, 16 * b, y, LDC);
  }
  if (half == 0) {
#pragma unroll
    for (int b = 0; b < NRT; ++b) {
      if (b > a) continue;
      const int s_ = 16 * b + lr;
      float cs = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * a + 4 * lg + j;
        if (s_ <= r) cs = fmaf((float)cT[s_ * LDC + O::perm(r)], accWP[b][j], cs);  // T^T[s][r]
      }
      cs += __shfl_xor(cs, 16);
      cs += __shfl_xor(cs, 32);
      if (lg == 0) pct[a * C + s_] = cs;
    }
  }
  lds_barrier();
  // dA, G . E and the entrywise terms for the tiles at or below the diagonal
  {
    float re[4] = {0.f, 0.f, 0.f, 0.f}, rb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int b = 2 * cc + half;
      f32x4 dg4 = z4, dq4 = z4;
      if (b <= a) {
        f32x4 da = z4, gk = z4;
#pragma unroll
        for (int q = 0; q < 2; ++q)  // T^T row r: rows m >= r of T
          if (q >= a / 2)
            da = O::mma_grp(O::a_row(cT + ra * LDC, 32 * q, lg), O::a_trans(cY, LDC, 32 * q, 16 * b, lane), da);
#pragma unroll
        for (int q = 0; q < NQG; ++q)
          gk = O::mma_grp(O::a_row(bK + ra * LDK, 32 * q, lg), O::a_row(bK + (16 * b + lr) * LDK, 32 * q, lg), gk);
        const int s_ = 16 * b + lr;
        float ce = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * a + 4 * lg + j;
          if (s_ <= r) {
            const float ex = __expf(sgam[r] - sgam[s_]);
            const float dA = s_ < r ? -da[j] : 0.f;
            const float ge = gk[j] * ex, dP = cdP[r * LCF + s_];
            dg4[j] = dA * sb[r] * ex;
            dq4[j] = dP * ex;
            const float dee = fmaf(dA * sb[r], ge, dP * (float)bP[r * LDC + O::perm(s_)]);
            re[j] += dee;
            ce += dee;
            rb[j] = fmaf(dA, ge, rb[j]);
          }
        }
        ce += __shfl_xor(ce, 16);
        ce += __shfl_xor(ce, 32);
        if (lg == 0) pcol[a * C + s_] = ce;
      }
      put_d(cG, 16 * a, 16 * b, dg4, LDC);  // zero above the diagonal
      put_d(cQK, 16 * a, 16 * b, dq4, LDC);
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        re[j] += __shfl_xor(re[j], off);
        rb[j] += __shfl_xor(rb[j], off);
      }
    if (lr == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        prow[half * C + 16 * a + 4 * lg + j] = re[j];
        pdb[half * C + 16 * a + 4 * lg + j] = rb[j];
      }
    }
  }
  lds_barrier();
  // dQ += dQK K;  dK += dQK^T Q + dG K + dG^T K  (contraction over the chunk rows s)
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const bool lo = 32 * q < 16 * (a + 1), up = q >= a / 2;  // row r: s <= r; column r: s >= r
    Grp aqk = O::zero_grp(), ag = O::zero_grp(), aqt = O::zero_grp(), agt = O::zero_grp();
    if (lo) {
      aqk = O::a_row(cQK + ra * LDC, 32 * q, lg);
      ag = O::a_row(cG + ra * LDC, 32 * q, lg);
    }
    if (up) {
      aqt = O::a_trans(cQK, LDC, 32 * q, 16 * a, lane);
      agt = O::a_trans(cG, LDC, 32 * q, 16 * a, lane);
    }
#pragma unroll
    for (int i = 0; i < NKH; ++i) {
      const int b = 2 * i + half;
      if (b < NKT) {
        const Grp kb = O::a_trans(bK, LDK, 32 * q, 16 * b, lane);
        if (lo) {
          accQ[i] = O::mma_grp(aqk, kb, accQ[i]);
          accK[i] = O::mma_grp(ag, kb, accK[i]);
        }
        if (up) accK[i] = O::mma_grp(agt, kb, O::mma_grp(aqt, O::a_trans(bQ, LDK, 32 * q, 16 * b, lane), accK[i]));
      }
    }
  }
  // per-row scalars (wave 0, lane = chunk row): dgamma, the chunk-end terms on the last
  // row, dg = reverse running sum; db, deta and the norm term of dk
  if (w == 0) {
    const int r = lane;
    float v = sdgam[r] * sGm[r] - sdd[r] * sdec[r] + prow[r] + prow[C + r] -
              (pcol[r] + pcol[C + r] + pcol[2 * C + r] + pcol[3 * C + r]);
    float gcs = lane < kGT / 64 ? sred[lane] : 0.f, ddd = sdd[r] * sdec[r];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      gcs += __shfl_xor(gcs, off);
      ddd += __shfl_xor(ddd, off);
    }
    if (r == C - 1) v += gcs * __expf(gC) + ddd;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float u = __shfl_down(v, off);
      if (lane + off < 64) v += u;
    }
    const float db = pct[r] + pct[C + r] + pct[2 * C + r] + pct[3 * C + r] + pdb[r] + pdb[C + r];
    const float den = snrm[r] + p.eps;
    scf[r] = (p.beta_direct || r >= rows) ? 0.f : -2.f * seta[r] * db / (den * den);
    if (r < rows) {
      p.dg[cl.row0 + r] = v;
      p.deta[cl.row0 + r] = p.beta_direct ? db : db / den;
    }
  }
  lds_barrier();  // T .. dQK are read; scf is set
  // dQ, dK (with the norm term) staged as natural rows, then stored in 16-byte pieces
  bf16 *sdq = reinterpret_cast<bf16 *>(smem + L::SDQ), *sdk = reinterpret_cast<bf16 *>(smem + L::SDK);
#pragma unroll
  for (int i = 0; i < NKH; ++i) {
    const int b = 2 * i + half;
    if (b < NKT) {
      const int c = 16 * b + lr;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * a + 4 * lg + j;
        sdq[r * LDO + c] = (bf16)accQ[i][j];
        sdk[r * LDO + c] = (bf16)fmaf(scf[r], (float)bK[r * LDK + O::perm(c)], accK[i][j]);
      }
    }
  }
  lds_barrier();
  constexpr int PPR = DK / 8;  // 16-byte pieces per row
  for (int pc = t; pc < C * PPR; pc += kGT) {
    const int r = pc / PPR, m = pc % PPR;
    if (r < rows) {
      const size_t e = (size_t)(cl.row0 + r) * DK + 8 * m;
      *reinterpret_cast<uint4 *>(static_cast<bf16 *>(p.dq) + e) = *reinterpret_cast<const uint4 *>(sdq + r * LDO + 8 * m);
      *reinterpret_cast<uint4 *>(static_cast<bf16 *>(p.dk) + e) = *reinterpret_cast<const uint4 *>(sdk + r * LDO + 8 * m);
    }
  }
}

// ============================================================================
// host side
// ============================================================================
// Per device: its CU count, and a second stream with two events on which the backward
// runs its adjoint scan beside the states pass (created on first use, default priority,
// kept until the process ends).  `lock` serialises the fork and join of concurrent calls
// so that each waits on its own events.
struct SideStream {
  std::mutex lock;
  bool ready = false;
  int cus = 0;
  hipStream_t stream = nullptr;
  hipEvent_t prep_done = nullptr, rev_done = nullptr;
};
static SideStream *side_stream() {
  static SideStream side[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  SideStream &s = side[dev];
  std::lock_guard<std::mutex> g(s.lock);
  if (!s.ready) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return nullptr;
    if (hipStreamCreateWithFlags(&s.stream, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&s.prep_done, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&s.rev_done, hipEventDisableTiming) != hipSuccess)
      return nullptr;
    s.cus = n;
    s.ready = true;
  }
  return &s;
}

template <typename E, int C, int DK>
struct BwdLayout {
  // workspace: prep records, then chunk-start states, then chunk-end state gradients
  // (bf16, chunk 64: no prep records; the T^T images of the forward prep kernel instead)
  static constexpr bool kImg = std::is_same<E, bf16>::value && C == 64;
  static size_t prep_bytes(const ChunkArgs &a, int nslot) {
    const size_t per = kImg ? (size_t)TpLayout<bf16, 64>::PACK : PrepRec<E, C>::BYTES;
    return ((size_t)a.H * nslot * per + 255) / 256 * 256;
  }
  static size_t state_bytes(const ChunkArgs &a, int nslot) {
    return ((size_t)a.H * nslot * DK * a.dv * sizeof(E) + 255) / 256 * 256;
  }
};

template <int C>
int bwd_slots(const ChunkArgs &a) {
  return a.cu_seqlens ? a.T / C + a.num_seqs + 1 : a.B * ((a.T + C - 1) / C);
}

// After the two state regions: the forward's own workspace, used by the forward
// kernels that produce the chunk-start states (launch_chunk_states).
template <typename E, int C, int DK>
size_t bwd_workspace_bytes_t(const ChunkArgs &a) {
  const int ns = bwd_slots<C>(a);
  return BwdLayout<E, C, DK>::prep_bytes(a, ns) + 2 * BwdLayout<E, C, DK>::state_bytes(a, ns) +
         chunk_workspace_bytes(a);
}

template <typename E, int C, int DK>
hipError_t launch_bwd_t(const ChunkArgs &a, const ChunkBwdArgs &b, hipStream_t st) {
  static_assert(PrepSmem<E, C, DK>::BYTES <= 64 * 1024, "prep LDS (kept small: several workgroups per CU)");
  static_assert(GradSmem<C, DK>::FLOATS * 4 <= 160 * 1024, "grads LDS");
  BwdParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.g = a.g;
  p.eta = a.eta;
  p.dout = b.dout;
  p.eps = a.eps;
  p.s0 = a.initial_state;
  p.dsfin = b.dfinal_state;
  p.dq = b.dq;
  p.dk = b.dk;
  p.dv = b.dv;
  p.dg = b.dg;
  p.deta = b.deta;
  p.ds0 = b.dinitial_state;
  p.cu = a.cu_seqlens;
  p.B = a.B;
  p.H = a.H;
  p.T = a.T;
  p.DV = a.dv;
  p.nseq = a.num_seqs;
  p.nslot = bwd_slots<C>(a);
  p.nsl = a.dv / kNS;
  p.beta_direct = a.beta_direct;
  char *ws = static_cast<char *>(a.workspace);
  constexpr bool img = BwdLayout<E, C, DK>::kImg;
  p.prep = img ? nullptr : reinterpret_cast<float *>(ws);
  p.timg = img ? ws : nullptr;
  const size_t pb = BwdLayout<E, C, DK>::prep_bytes(a, p.nslot), sb = BwdLayout<E, C, DK>::state_bytes(a, p.nslot);
  p.states = ws + pb;
  p.dstates = ws + pb + sb;
  p.fws = ws + pb + 2 * sb;
  const unsigned seq_blocks = (unsigned)((long long)a.num_seqs * a.H * p.nsl);
  // the two scans: (sequence, head) groups padded to whole rounds of 8, times the slices
  const unsigned groups8 = (unsigned)(((long long)a.num_seqs * a.H + 7) / 8 * 8);
  const unsigned ns32 = a.dv % 32 == 0 ? 1u : 0u;
  const unsigned scan_blocks = groups8 * (unsigned)(a.dv / (ns32 ? 32 : 16));
  const bool tokens = (long long)a.B * a.T > 0 && p.nslot > 0;
  if (tokens) {
    if constexpr (!img) {
      hipLaunchKernelGGL((kla_bwd_prep_kernel<E, C, DK>), dim3((unsigned)p.nslot, (unsigned)a.H), dim3(kPT), 0, st, p);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    // the chunk-start states: the forward's pipelined prep and scan kernels in states
    // mode (no outputs), into p.states as operand groups (and, for bf16, the T^T images)
    ChunkArgs fa = a;
    fa.o = nullptr;
    fa.final_state = nullptr;
    fa.workspace = ws + pb + 2 * sb;
    if constexpr (img) {
      SideStream *side = side_stream();
      if (side && bwd_scans_concurrent(fa, side->cus)) {
        // the states pass on `st`, the adjoint scan on the side stream once the prep's
        // workspace is complete; `st` waits for both before the gradient kernel
        std::lock_guard<std::mutex> g(side->lock);
        hipError_t e = launch_chunk_states(fa, p.states, st, ws, true, side->prep_done);
        if (e == hipSuccess) e = hipStreamWaitEvent(side->stream, side->prep_done, 0);
        if (e == hipSuccess) e = launch_chunk_rev(fa, p.dsfin, p.dout, p.ds0, p.dstates, side->stream, true);
        if (e == hipSuccess) e = hipEventRecord(side->rev_done, side->stream);
        if (e == hipSuccess) e = hipStreamWaitEvent(st, side->rev_done, 0);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((kla_bwd_grads2_kernel<DK>), dim3((unsigned)p.nslot, (unsigned)a.H), dim3(kGT), 0, st, p);
        return hipGetLastError();
      }
    }
    const hipError_t e = launch_chunk_states(fa, p.states, st, img ? ws : nullptr);
    if (e != hipSuccess) return e;
  }
  if (seq_blocks > 0 && (tokens || p.ds0)) {
    // the chunk-end state gradients, in reverse, on the forward's machinery (with no
    // tokens this only copies dS_final, or zeros, to the initial-state gradient)
    ChunkArgs fa = a;
    fa.o = nullptr;
    fa.final_state = nullptr;
    fa.workspace = ws + pb + 2 * sb;
    const hipError_t e = launch_chunk_rev(fa, p.dsfin, p.dout, p.ds0, p.dstates, st);
    if (e != hipSuccess) return e;
  }
  if (tokens) {
    if constexpr (std::is_same<E, bf16>::value && C == 64)
      hipLaunchKernelGGL((kla_bwd_grads2_kernel<DK>), dim3((unsigned)p.nslot, (unsigned)a.H), dim3(kGT), 0, st, p);
    else
      hipLaunchKernelGGL((kla_bwd_grads_kernel<E, C, DK>), dim3((unsigned)p.nslot, (unsigned)a.H), dim3(kGT), 0, st, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

bool chunk_bwd_supported(int dtype, int dk, int dv, int chunk) { return fast_chunk_supported(dtype, dk, dv, chunk); }

size_t chunk_bwd_workspace_bytes(const ChunkArgs &a) {
  if (a.dtype == 0) return a.dk == 128 ? bwd_workspace_bytes_t<bf16, 64, 128>(a) : bwd_workspace_bytes_t<bf16, 64, 64>(a);
  if (a.chunk == 16) {
    switch (a.dk) {
      case 16: return bwd_workspace_bytes_t<float, 16, 16>(a);
      case 32: return bwd_workspace_bytes_t<float, 16, 32>(a);
      case 64: return bwd_workspace_bytes_t<float, 16, 64>(a);
      default: return bwd_workspace_bytes_t<float, 16, 128>(a);
    }
  }
  return a.dk == 16 ? bwd_workspace_bytes_t<float, 64, 16>(a) : bwd_workspace_bytes_t<float, 64, 32>(a);
}

hipError_t launch_chunk_bwd(const ChunkArgs &a, const ChunkBwdArgs &b, hipStream_t st) {
  if (a.dtype == 0) {
    if (a.dk == 128) return launch_bwd_t<bf16, 64, 128>(a, b, st);
    if (a.dk == 64) return launch_bwd_t<bf16, 64, 64>(a, b, st);
    return hipErrorInvalidValue;
  }
  if (a.chunk == 16) {
    switch (a.dk) {
      case 16: return launch_bwd_t<float, 16, 16>(a, b, st);
      case 32: return launch_bwd_t<float, 16, 32>(a, b, st);
      case 64: return launch_bwd_t<float, 16, 64>(a, b, st);
      case 128: return launch_bwd_t<float, 16, 128>(a, b, st);
    }
  } else if (a.chunk == 64) {
    switch (a.dk) {
      case 16: return launch_bwd_t<float, 64, 16>(a, b, st);
      case 32: return launch_bwd_t<float, 64, 32>(a, b, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace kla
