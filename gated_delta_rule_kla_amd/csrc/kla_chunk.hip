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
// Mapping onto the chip.  Two kernels (below).  The prep kernel does the
// S-independent work of every chunk -- gate scan, ||k||^2 and beta, K K^T and A,
// the blockwise triangular solve for T' -- for all chunks and heads in parallel,
// into a workspace.  In the scan kernel one workgroup owns one (sequence, head,
// slice of DVT = 16 NCT state columns), or one segment of a sequence in segment
// mode, and walks its chunks in order.  The state slice never leaves the chip:
// it lives in the MFMA accumulators of the chain waves (fp32) for the whole
// sequence.  Seven role-specialised waves form a software pipeline over the
// chunks with one LDS-only barrier per step (see "Roles and LDS plan" below):
// loader waves bring K, Q, the T' image and the V slice ahead of the chain, the
// chain waves advance the state, and the P waves form the causal scores and the
// output rows.
//
// Every K and Q row is read with coalesced 16-byte buffer loads and goes
// through LDS into the MFMA operand layout: loads that give each lane its own
// row (the operand layout) cost the texture-address unit four times more.
// The chain never round-trips its own data through LDS: every right operand
// (S, X, U~, Diag(d) U~) is fed to the next MFMA straight from the accumulator
// registers, by ordering each instruction's contraction index the way the
// accumulator layout holds it (see Ops below); the matching left operands (K
// and Q rows) are stored with their columns permuted into that order, and K^T,
// T' (stored transposed) and the V slice are read with gfx950's transposing
// LDS read.
#include "kla.h"
#include "kla_common.h"
#include "kla_internal.h"
#include "kla_ops.h"

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

namespace kla {

// ---------------------------------------------------------------------------
// Two kernels
// ---------------------------------------------------------------------------
// Prep: the S-independent work of every chunk, all chunks in parallel: gate
// scan, ||k||^2 and beta, K K^T and A, T = (I + A)^-1, T' = T Diag(beta).  It
// writes the packed T'^T image and the row vectors gamma, Gam, d per (chunk,
// head) into a workspace, laid out as the scan kernel's loader expands them
// into LDS.  bf16: kla_chunk_prep_wave_kernel, one wave per run of chunks of
// one head; fp32: kla_chunk_prep_kernel, a workgroup of role waves pipelining
// a run of consecutive chunks.
//
// kla_chunk_kernel: one workgroup per (sequence, head, slice of state
// columns), the chunks of the sequence in order -- the causal scores, the
// state scan and the output.  Because T' is computed once per chunk and head,
// the column slices of a head do not each redo the solve.

struct ChunkParams {
  const void *q, *k, *v, *g, *eta;
  float eps;
  const float *s0;
  void *o;
  float *sfin;
  const int32_t *cu;
  char *ws;
  const int *order;  // packed sequences, longest first (in the workspace), or nullptr
  int H, T, dv, n_tiles, ngroups, nseq, nslot;
  int pslots;  // prep kernel: workspace slots per workgroup (1 .. kPrepSlots)
  int beta_direct;  // 1: `eta` holds beta itself (gated delta rule); eps unused
  // States mode (the backward pass's chunk-start states): when set, the scan
  // writes the state at the start of every chunk here instead of the outputs,
  // as the chain's operand groups: slot (h * nslot + slot of the chunk), then
  // 16-column tile, then group q of KG state rows, 64 lanes x 16 bytes (lane l,
  // element x: column l & 15 of the tile; bf16 rows 16 (x >> 2) + 4 (l >> 4) +
  // (x & 3), fp32 rows 4 (l >> 4) + x, of the group).  o and sfin are unused.
  char *states;
  // With states (bf16 prep kernel only): also the packed image of T^T, T = (I + A)^-1
  // without the Diag(beta) of T', per (head, slot) at timg + (h * nslot + slot) *
  // TpLayout<bf16, 64>::PACK (the gradient kernel's T), or nullptr.
  char *timg;
  // PGDN (bf16, chunk 64): the write keys W = P (.) K per (head, slot), C x dk bf16 rows,
  // written by the prep kernel and read by the scan in place of K where the state is
  // written (the update and the causal scores); the key accumulator at each chunk's
  // start per (head, slot), dk fp32; ln(band) of the preconditioner's squash.
  char *pg_w;
  float *pg_acc;
  float band_c;
  const float *pg_acc0;  // [N, H, dk] accumulator at each sequence's start, or nullptr (zeros)
  float *pg_accfin;      // [N, H, dk] at each sequence's end, or nullptr
  // Segments (forward scan only; seg_first == nullptr: one segment per sequence).
  // Sequence n is cut into segments of seg_chunks chunks (the last may be shorter,
  // an empty sequence is one empty segment); its segments are seg_first[n] ..
  // seg_first[n + 1] - 1 (N + 1 prefix sums), and group g of the scan grid is
  // (segment g / H, head g % H).  A group's first n_vtiles column tiles carry v's
  // columns: a sequence's first segment starts from s0, a later one from zero, and
  // each writes its end state to seg_d.  The other n_tiles - n_vtiles tiles (later
  // segments only) carry the identity: zero v, start state I (dk x dk), outputs to
  // eout in o's place, end state (the segment's transfer map) to seg_m.
  const int *seg_first;
  int seg_chunks, n_vtiles;
  void *eout;    // [B, H, T, dk] element type: the identity tiles' outputs
  float *seg_d;  // [nseg, H, dk, dv]
  float *seg_m;  // [nseg, H, dk, dk]
};

// The sequence of segment s: the largest n with seg_first[n] <= s (n < nseq).
__device__ __forceinline__ int seg_sequence(const int *seg_first, int nseq, int s) {
  int lo = 0, hi = nseq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seg_first[mid] <= s) lo = mid; else hi = mid - 1;
  }
  return lo;
}



// ---------------------------------------------------------------------------
// prep kernel
// ---------------------------------------------------------------------------
// One workgroup per (head, run of p.pslots <= kPrepSlots consecutive workspace
// slots):
// four role-specialised waves in a pipeline over the run, one LDS-only
// barrier per step.  Step s (s = -1 .. p.pslots) has
//   PLOAD    K rows, g and eta of slot s+1 into LDS (coalesced loads issued a
//            step ahead)
//   PG[2]    slot s: K K^T of the owned rows, ||k||^2, the gate scan, beta,
//            A, and the owned diagonal blocks T_bb = (I + A_bb)^-1 and of T'^T
//   POFFD    slot s-1: the off-diagonal blocks of T and of T' = T Diag(beta)
//            (the Gram waves wrote the diagonal ones); the T'^T image goes to
//            the workspace with gamma, Gam, d
// One wave per SIMD.
enum PrepRole { PG0 = 0, PG1 = 1, POFFD = 2, PLOAD = 3 };
constexpr int kPrepWaves = 4;
constexpr int kPrepSlots = 16;  // most workspace slots per workgroup

template <typename E, int C, int DK>
struct PrepShape {
  static constexpr int NB = C / 16;
  static constexpr int NT = 64 * kPrepWaves;
  static constexpr int PAD = LdsPad<E>::V;
  static constexpr int LDK = DK + PAD;         // K and Q rows (grouped columns)
  static constexpr int LDC = TpLayout<E, C>::LDC;
  static constexpr int LDA = 16 + PAD / 2;     // rows of one 16x16 off-diagonal A^T block
  static constexpr int LDD = 20;               // fp32 16-wide rows of diagonal blocks
  static constexpr int KG = Ops<E>::KG;
  static constexpr int NOFF = NB * (NB - 1) / 2;
  static constexpr int K_SLOT = C * LDK * (int)sizeof(E);
  static constexpr int GE_SLOT = 2 * C * 4;                // g (0 past the end), eta
  static constexpr int A_SLOT = (NOFF > 0 ? NOFF : 1) * 16 * LDA * (int)sizeof(E);
  static constexpr int TD_SLOT = NB * 16 * LDD * 4;        // diagonal blocks (A, then T), transposed, fp32
  static constexpr int BV_SLOT = 4 * C * 4;                // gamma, Gam, d, beta
  static constexpr int GP = 3 * C * 4;                     // per Gram wave: gamma, ||k||^2, beta
  static constexpr int OFF_K = 0;
  static constexpr int OFF_GE = OFF_K + 2 * K_SLOT;
  static constexpr int OFF_A = OFF_GE + 2 * GE_SLOT;
  static constexpr int OFF_TD = OFF_A + 2 * A_SLOT;
  static constexpr int OFF_BV = OFF_TD + 2 * TD_SLOT;
  static constexpr int IMG_SLOT = TpLayout<E, C>::TP_IMG;
  static constexpr int OFF_IMG = OFF_BV + 2 * BV_SLOT;
  static constexpr int OFF_GP = OFF_IMG + 2 * IMG_SLOT;
  static constexpr int OFF_SLOT = OFF_GP + 2 * GP;         // per slot: token offset (8 B), rows (4 B), pad
  static constexpr int BYTES = OFF_SLOT + kPrepSlots * 16;
  static_assert(K_SLOT % 16 == 0 && A_SLOT % 16 == 0 && TD_SLOT % 16 == 0, "lds align");
  // bf16: two workgroups per CU (the fp32 debug build may take one)
  static_assert(BYTES <= (sizeof(E) == 2 ? 80 : 160) * 1024, "LDS budget");
};

template <typename E, int C, int DK>
__global__ __launch_bounds__(64 * kPrepWaves) void kla_chunk_prep_kernel(ChunkParams p) {
  using Sh = PrepShape<E, C, DK>;
  using TL = TpLayout<E, C>;
  using O = Ops<E>;
  using Grp = typename O::Grp;
  constexpr int NB = Sh::NB, LDK = Sh::LDK, LDC = Sh::LDC, LDA = Sh::LDA, LDD = Sh::LDD;
  constexpr int KG = O::KG, TPG = KG / 16, NQG = DK / KG;

  __shared__ __attribute__((aligned(16))) char smem[Sh::BYTES];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int h = blockIdx.y;
  const int nps = p.pslots;
  const int slot_base = blockIdx.x * nps;

  // ---- the chunk behind each slot of the run: token offset and row count ---
  // (row count 0: no chunk -- an unused slot or past the end)
  long long *slot_tok = reinterpret_cast<long long *>(smem + Sh::OFF_SLOT);
  int *slot_rows = reinterpret_cast<int *>(smem + Sh::OFF_SLOT + 8);
  if (threadIdx.x < nps) {
    const int slot = slot_base + threadIdx.x;
    int b = 0, t0 = 0, len = p.T, c = slot;
    if (p.cu) {
      // sequence n with n + floor(cu[n] / C) <= slot (strictly increasing in n)
      int lo = 0, hi = p.nseq - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (mid + min(max(p.cu[mid], 0), p.T) / C <= slot) lo = mid; else hi = mid - 1;
      }
      t0 = min(max(p.cu[lo], 0), p.T);
      len = min(max(p.cu[lo + 1], t0), p.T) - t0;
      c = slot - (lo + t0 / C);
    } else {
      const int nchT = (p.T + C - 1) / C;
      b = slot / nchT;
      c = slot % nchT;
      if (b >= p.nseq) len = 0;
    }
    const bool ok = slot < p.nslot && c >= 0 && c * C < len;
    slot_tok[2 * threadIdx.x] = ((long long)b * p.H + h) * p.T + t0 + (long long)c * C;
    slot_rows[4 * threadIdx.x] = ok ? min(C, len - c * C) : 0;
  }
  // (values read from LDS are per lane to the compiler: make them scalar)
  auto nrow_of = [&](int s) {
    return (s >= 0 && s < nps) ? __builtin_amdgcn_readfirstlane(slot_rows[4 * s]) : 0;
  };
  auto tok_of = [&](int s) {
    const long long t = slot_tok[2 * min(max(s, 0), nps - 1)];
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)t), hi = __builtin_amdgcn_readfirstlane((unsigned)(t >> 32));
    return (size_t)(((unsigned long long)hi << 32) | lo);
  };
  auto ws_of = [&](int s) { return p.ws + ((size_t)h * p.nslot + slot_base + s) * TL::BYTES; };

  auto sK = [&](int s) { return reinterpret_cast<E *>(smem + Sh::OFF_K + (s & 1) * Sh::K_SLOT); };
  auto sGE = [&](int s) { return reinterpret_cast<float *>(smem + Sh::OFF_GE + (s & 1) * Sh::GE_SLOT); };
  auto sA = [&](int s) { return reinterpret_cast<E *>(smem + Sh::OFF_A + (s & 1) * Sh::A_SLOT); };
  auto sTd = [&](int s) { return reinterpret_cast<float *>(smem + Sh::OFF_TD + (s & 1) * Sh::TD_SLOT); };
  // gamma, Gam = exp(gamma), d = exp(gamma_C - gamma), beta
  auto sBV = [&](int s) { return reinterpret_cast<float *>(smem + Sh::OFF_BV + (s & 1) * Sh::BV_SLOT); };
  auto sImg = [&](int s) { return reinterpret_cast<E *>(smem + Sh::OFF_IMG + (s & 1) * Sh::IMG_SLOT); };

  // strictly-upper blocks of T' (strictly-lower ones of the T'^T image) and the
  // pads are zero and never rewritten
  for (int i = threadIdx.x; i < 2 * C * LDC; i += Sh::NT) {
    const int rr = (i / LDC) % C, cc = i % LDC;
    if (cc >= C || (rr >> 4) > (cc >> 4))
      sImg(i / (C * LDC))[rr * LDC + (cc < C ? O::perm(cc) : cc)] = Elem<E>::from_f32(0.f);
  }

  if (wave == PLOAD) {
    // =================== K, Q, g, eta of slot s+1 ============================
    RowLoad<E, DK, AllBlocks<NB>> kin;
    typename std::conditional<sizeof(E) == 2, unsigned short, unsigned>::type graw = 0, eraw = 0;
    auto issue = [&](int s) {
      const int nrow = nrow_of(s);
      const size_t tok = tok_of(s);
      kin.issue(static_cast<const E *>(p.k) + tok * DK, nrow, lane);
      // g and eta of row `lane` (0 past the end; lanes >= C read nothing)
      const E *gp = static_cast<const E *>(p.g) + tok, *ep = static_cast<const E *>(p.eta) + tok;
      graw = buffer_ld_elem(buffer_rsrc(gp, nrow * (int)sizeof(E)), lane, gp);
      eraw = buffer_ld_elem(buffer_rsrc(ep, nrow * (int)sizeof(E)), lane, ep);
    };
    __syncthreads();
    issue(0);
    for (int s = -1; s <= nps; ++s) {
      if (s + 1 < nps) {
        kin.put(sK(s + 1), LDK, lane, [](int, int row) { return row; });
        float *ge = sGE(s + 1);
        if (lane < C) {
          ge[lane] = elem_bits_to_f32(graw);
          ge[C + lane] = elem_bits_to_f32(eraw);
        }
        issue(s + 2);
      }
      lds_barrier();
    }
  } else if (wave == PG0 || wave == PG1) {
    // =================== Gram waves: slot s ==================================
    auto gram = [&](auto part_c) {
      constexpr int part = decltype(part_c)::value;
      using OB = OwnBlocks<NB, part>;
      constexpr int NREAD = part == 0 ? NB : NB - 1;  // blocks 0 .. largest owned block
      float *gp = reinterpret_cast<float *>(smem + Sh::OFF_GP + part * Sh::GP);
      float *sGam = gp, *sNrm = gp + C, *sBet = gp + 2 * C;
      __syncthreads();
      for (int s = -1; s <= nps; ++s) {
        const int nrow = nrow_of(s);
        if (OB::N > 0 && nrow > 0) {
          const E *K = sK(s);
          const float *ge = sGE(s);
          E *Ablk = sA(s);
          float *Td = sTd(s);
          float *bv = sBV(s);
          Grp kb[NREAD > 0 ? NREAD : 1][NQG];
#pragma unroll
          for (int k = 0; k < NREAD; ++k)
#pragma unroll
            for (int q = 0; q < NQG; ++q) kb[k][q] = O::a_row(K + (16 * k + li) * LDK, q * KG, lg);
          f32x4 G[NB][NB];
#pragma unroll
          for (int rt = 0; rt < NB; ++rt) {
            if (!owns_block(NB, part, rt)) continue;
#pragma unroll
            for (int st = 0; st <= rt; ++st) {
              G[rt][st] = zero4();
#pragma unroll
              for (int q = 0; q < NQG; ++q) G[rt][st] = O::mma_grp(kb[rt][q], kb[st][q], G[rt][st]);
            }
            // ||k_r||^2 of row 16 rt + li sits on the diagonal of tile (rt, rt):
            // lane group li >> 2, element li & 3
            const f32x4 d = G[rt][rt];
            const int j = li & 3;
            const float nr = j == 0 ? d[0] : j == 1 ? d[1] : j == 2 ? d[2] : d[3];
            if (lg == (li >> 2)) sNrm[16 * rt + li] = nr;
          }
          // gate scan and beta (lane = chunk row); beta of rows beyond the
          // sequence end is 0 (not 0/0 when eps = 0)
          const float gam = wave_inclusive_scan(lane < C ? ge[lane] : 0.f);
          const float gamC = lane_value(gam, C - 1);
          if (lane < C) {
            sGam[lane] = gam;
            if (part == 0) {
              bv[lane] = gam;
              bv[C + lane] = __expf(gam);             // Gam_r
              bv[2 * C + lane] = __expf(gamC - gam);  // d_r
            }
            if (owns_block(NB, part, lane >> 4)) {
              const float beta =
                  (lane < nrow) ? (p.beta_direct ? ge[C + lane] : ge[C + lane] / (sNrm[lane] + p.eps)) : 0.f;
              sBet[lane] = beta;
              bv[3 * C + lane] = beta;
            }
          }
          // A = beta_r (K K^T)_rs exp(gamma_r - gamma_s), r > s
#pragma unroll
          for (int rt = 0; rt < NB; ++rt) {
            if (!owns_block(NB, part, rt)) continue;
            const f32x4 gr4 = *reinterpret_cast<const f32x4 *>(sGam + 16 * rt + 4 * lg);
            const f32x4 br4 = *reinterpret_cast<const f32x4 *>(sBet + 16 * rt + 4 * lg);
#pragma unroll
            for (int st = 0; st <= rt; ++st) {
              const float gs = sGam[16 * st + li];
              const f32x4 acc = G[rt][st];
              f32x4 av;
              if (st < rt) {
#pragma unroll
                for (int j = 0; j < 4; ++j) av[j] = br4[j] * acc[j] * __expf(gr4[j] - gs);
                // off-diagonal block, stored transposed: A^T[s'][r']
                store4(Ablk + (rt * (rt - 1) / 2 + st) * 16 * LDA + li * LDA + 4 * lg, av);
              } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  const bool below = 4 * lg + j > li;
                  const float dec = below ? __expf(gr4[j] - gs) : 0.f;
                  av[j] = below ? br4[j] * acc[j] * dec : 0.f;
                }
                // diagonal block, fp32, stored transposed (At[s'][r'])
                *reinterpret_cast<f32x4 *>(Td + (rt * 16 + li) * LDD + 4 * lg) = av;
              }
            }
          }
          // the owned diagonal blocks T_bb = (I + A_bb)^-1 by column-parallel
          // forward substitution in fp32: lane = (owned block lg, column li);
          // T_bb replaces A_bb, also transposed (row li = column li of T_bb)
          asm volatile("" ::: "memory");  // A_bb (written by other lanes of this wave) before the solve reads it
          if (lg < OB::N) {
            const int bb = lg == 0 ? OB::at(0) : OB::at(OB::N > 1 ? 1 : 0);
            float *At = Td + bb * 16 * LDD;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = (r == li) ? 1.f : 0.f;
            f32x4 cur[4], nxt[4];
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) cur[qd] = *reinterpret_cast<const f32x4 *>(At + 4 * qd);
#pragma unroll
            for (int s2 = 0; s2 < 15; ++s2) {
              if (s2 + 1 < 15) {
#pragma unroll
                for (int qd = 0; qd < 4; ++qd)
                  if (4 * qd + 3 > s2 + 1) nxt[qd] = *reinterpret_cast<const f32x4 *>(At + (s2 + 1) * LDD + 4 * qd);
              }
#pragma unroll
              for (int r = s2 + 1; r < 16; ++r) x[r] = fmaf(-cur[r >> 2][r & 3], x[s2], x[r]);
#pragma unroll
              for (int qd = 0; qd < 4; ++qd) cur[qd] = nxt[qd];
            }
            // T_bb replaces A_bb (transposed, for the off-diagonal blocks); the
            // diagonal block of the T'^T image is column li of T_bb times beta
            float *dst = At + li * LDD;
            E *irow = sImg(s) + (16 * bb + li) * LDC;
            const float bs = sBet[16 * bb + li];
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
              const f32x4 t4 = {x[4 * qd], x[4 * qd + 1], x[4 * qd + 2], x[4 * qd + 3]};
              *reinterpret_cast<f32x4 *>(dst + 4 * qd) = t4;
              store4(irow + O::perm(16 * bb + 4 * qd), bs * t4);
            }
          }
        }
        lds_barrier();
      }
    };
    if (wave == PG0)
      gram(std::integral_constant<int, 0>{});
    else
      gram(std::integral_constant<int, 1>{});
  } else if (wave == POFFD) {
    // =================== off-diagonal solve: slot s-1 ========================
    using M = Mm16<E>;
    __syncthreads();
    for (int s = -1; s <= nps; ++s) {
      const int sp = s - 1;
      if (nrow_of(sp) > 0) {
        const E *Ablk = sA(sp);
        const float *Td = sTd(sp);
        const float *bv = sBV(sp);
        const float *beta = bv + 3 * C;
        E *img = sImg(sp);
        // off-diagonal blocks level by level: T_ij = -T_ii sum_m A_im T_mj
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
                // A_im[li][4lg + e] (block stored transposed); B operand T_mj[4lg + e][li]
                const typename M::Op a = M::ld_t(Ablk + (i * (i - 1) / 2 + m) * 16 * LDA, LDA, lane);
                const f32x4 bt = (m == j) ? *reinterpret_cast<const f32x4 *>(Td + (j * 16 + li) * LDD + 4 * lg)
                                          : Toff[m][j];
                y = M::mma(a, M::cvt(bt), y);
              }
              // A operand T_ii[li][4lg + e] = T_ii^T[4lg + e][li]
              f32x4 ti;
#pragma unroll
              for (int e = 0; e < 4; ++e) ti[e] = Td[(i * 16 + 4 * lg + e) * LDD + li];
              const f32x4 t = -M::mma(M::cvt(ti), M::cvt(y), zero4());
              Toff[i][j] = t;
              // T'^T[16 j + li][16 i + 4 lg + e] = T_ij[4 lg + e][li] beta_(16 j + li)
              store4(img + (16 * j + li) * LDC + O::perm(16 * i + 4 * lg), beta[16 * j + li] * t);
            }
          }
        }
        // the packed T'^T image and gamma, Gam, d to the workspace (16-byte
        // pieces; all LDS reads first, then the stores)
        constexpr int NI = TL::PACK / 16, NP = NI + TL::VEC3 / 16, NPL = (NP + 63) / 64;
        u32x4 *dst = reinterpret_cast<u32x4 *>(ws_of(sp));
        const u32x4 *vs = reinterpret_cast<const u32x4 *>(bv);
        u32x4 pc[NPL];
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
          const int i = min(lane + 64 * j, NP - 1);
          pc[j] = i < NI ? *reinterpret_cast<const u32x4 *>(img + TL::piece_to_lds(i)) : vs[i - NI];
        }
#pragma unroll
        for (int j = 0; j < NPL; ++j)
          if (NP % 64 == 0 || lane + 64 * j < NP) dst[lane + 64 * j] = pc[j];
      }
      lds_barrier();
    }
  }
}

// ---------------------------------------------------------------------------
// prep kernel, one wave per (chunk, head): the bf16 build
// ---------------------------------------------------------------------------
// The same S-independent work and the same workspace image as the pipelined
// prep kernel above, organised for latency hiding instead of a pipeline: each
// workgroup is one wave that owns one (chunk, head) from start to end, and a CU
// holds eight of them, whose load, MFMA and solve phases overlap.  Global
// memory is only touched with coalesced 16-byte accesses (consecutive lanes,
// consecutive bytes): K rows come in four rows per instruction into a padded
// LDS tile and go from there into the Gram MFMA operands (the same registers
// serve as both operands of K K^T); the packed T'^T image is assembled in the
// same LDS area once K is in registers, and leaves in 16-byte pieces.  (Loads
// or stores that give each lane its own row cost the texture-address unit
// several times more per instruction; with one wave per chunk that unit, not
// the arithmetic, set the kernel's time.)
template <int DK, bool PG = false>
struct PrepWaveShape {
  static constexpr int C = 64, NB = 4;
  static constexpr int RB = DK * 2 + 16;   // padded K row in LDS: 16 rows hit distinct banks
  static constexpr int LDA = 24;           // bf16 rows of one transposed 16x16 off-diagonal A block
  static constexpr int LDD = 20;           // fp32 rows of the diagonal blocks (A, then T), transposed
  static constexpr int TD_BYTES = NB * 16 * LDD * 4;
  // the T'^T image in LDS: the workspace's packed rows, padded by 16 bytes (rows < 32:
  // 72 elements, rows >= 32: 40) so that a column written by 16 lanes (one row each)
  // hits distinct banks; the copy to the workspace drops the padding
  static constexpr int IL0 = 64 + 8, IL1 = 32 + 8;
  static constexpr int IMG_BYTES = (32 * IL0 + 32 * IL1) * 2;
  // R holds the K rows until the Gram tiles are formed, then the image, the diagonal
  // blocks and the off-diagonal A blocks (all written after the K rows are dead)
  static constexpr int A_BYTES = 6 * 16 * LDA * 2;
  static constexpr int OFF_TD = IMG_BYTES;                    // inside R, after the image
  static constexpr int OFF_A = IMG_BYTES + TD_BYTES;          // inside R, after the diagonal blocks
  static constexpr int R_BYTES = C * RB > OFF_A + A_BYTES ? C * RB : OFF_A + A_BYTES;
  static constexpr int OFF_VEC = R_BYTES;                     // ||k||^2 (PGDN: k . w), gamma, beta, PGDN mean
  static constexpr int OFF_W = OFF_VEC + 4 * C * 4;           // PGDN: the write keys, rows as K's
  static constexpr int BYTES = OFF_W + (PG ? C * RB : 0);
  static_assert(IMG_BYTES % 16 == 0 && OFF_TD % 16 == 0 && OFF_A % 16 == 0 && OFF_VEC % 16 == 0 &&
                OFF_W % 16 == 0, "lds align");
  static_assert(BYTES * (PG ? 4 : 8) <= 160 * 1024, "eight (PGDN: four) workgroups per CU");
};

// TIMG: also write the T^T image (p.timg).  PG: PGDN -- A and beta from K W^T with the
// write keys W of p.pg_w.  Two waves per SIMD (eight per CU, the LDS allows as many) caps
// the registers at 256; without the cap the T^T image's live blocks took a few more and
// halved the waves per CU (PGDN's LDS tile allows four per CU anyway).
template <int DK, bool TIMG, bool PG>
__global__ __launch_bounds__(64, PG ? 1 : 2) void kla_chunk_prep_wave_kernel(ChunkParams p) {
  using Sh = PrepWaveShape<DK, PG>;
  using TL = TpLayout<bf16, 64>;
  using M = Mm16<bf16>;
  constexpr int C = 64, NB = 4, LDA = Sh::LDA, LDD = Sh::LDD, NQ = DK / 32, PPR = DK * 2 / 16;
  constexpr int NLD = C * PPR / 64;
  __shared__ __attribute__((aligned(16))) char smem[Sh::BYTES];
  const int lane = threadIdx.x;
  const int li = lane & 15, lg = lane >> 4;
  const int h = blockIdx.y;
  // this wave's run of p.pslots consecutive slots of head h
  const int s0 = blockIdx.x * p.pslots, s1 = min(s0 + p.pslots, p.nslot);

  // the chunk behind a slot (as in the pipelined prep kernel): its first token
  // and row count (0 = no chunk)
  auto describe = [&](int slot, size_t &tok, int &nrow) {
    int b = 0, t0 = 0, len = p.T, c = slot;
    if (p.cu) {
      int lo = 0, hi = p.nseq - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (mid + min(max(p.cu[mid], 0), p.T) / C <= slot) lo = mid; else hi = mid - 1;
      }
      t0 = min(max(p.cu[lo], 0), p.T);
      len = min(max(p.cu[lo + 1], t0), p.T) - t0;
      c = slot - (lo + t0 / C);
    } else {
      const int nchT = (p.T + C - 1) / C;
      b = slot / nchT;
      c = slot % nchT;
      if (b >= p.nseq) len = 0;
    }
    nrow = __builtin_amdgcn_readfirstlane((slot < s1 && c >= 0 && c * C < len) ? min(C, len - c * C) : 0);
    const size_t t = ((size_t)b * p.H + h) * (size_t)p.T + (size_t)t0 + (size_t)max(c, 0) * C;
    const unsigned lo32 = __builtin_amdgcn_readfirstlane((unsigned)t), hi32 = __builtin_amdgcn_readfirstlane((unsigned)(t >> 32));
    tok = ((size_t)hi32 << 32) | lo32;
  };
  // K rows (coalesced; rows past the end read as zero), g and eta of row `lane`
  uint4 kr[NLD];
  unsigned short lgraw = 0, leraw = 0;
  auto issue = [&](size_t tok, int nrow) {
    const bf16 *gk = static_cast<const bf16 *>(p.k) + tok * DK;
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(gk, nrow * DK * 2);
#pragma unroll
    for (int j = 0; j < NLD; ++j) kr[j] = buffer_ld16(rk, (64 * j + lane) * 16);
    const bf16 *gp = static_cast<const bf16 *>(p.g) + tok, *ep = static_cast<const bf16 *>(p.eta) + tok;
    lgraw = buffer_ld_elem(buffer_rsrc(gp, nrow * 2), lane, gp);
    leraw = buffer_ld_elem(buffer_rsrc(ep, nrow * 2), lane, ep);
  };

  char *R = smem;  // K rows, then the packed image and the diagonal blocks
  bf16 *img = reinterpret_cast<bf16 *>(R);
  float *Td = reinterpret_cast<float *>(R + Sh::OFF_TD);
  bf16 *Ablk = reinterpret_cast<bf16 *>(smem + Sh::OFF_A);
  float *sNrm = reinterpret_cast<float *>(smem + Sh::OFF_VEC);
  float *sGam = sNrm + C, *sBet = sNrm + 2 * C;
  char *Wt = smem + Sh::OFF_W;

  // the loaded K rows into the LDS tile (waits for those loads)
  auto stage = [&]() {
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int pc = 64 * j + lane;
      *reinterpret_cast<uint4 *>(R + (pc / PPR) * Sh::RB + (pc % PPR) * 16) = kr[j];
    }
  };
  // everything else for one slot, from the staged K rows and its g, eta
  auto process = [&](int slot, int nrow, unsigned short graw, unsigned short eraw) {
    char *ws = p.ws + ((size_t)h * p.nslot + slot) * TL::BYTES;
    if constexpr (PG) {
      // PGDN: the chunk's write keys (kla_pgdn_wkeys_kernel wrote them) into their LDS tile
      // (four 16-byte pieces in flight at a time: a whole-tile register array spills)
      const uint4 *wg = reinterpret_cast<const uint4 *>(p.pg_w + ((size_t)h * p.nslot + slot) * (C * DK * 2));
      auto wput = [&](int pc, uint4 v) {
        *reinterpret_cast<uint4 *>(Wt + (pc / (DK / 8)) * Sh::RB + (pc % (DK / 8)) * 16) = v;
      };
      for (int j = 0; j < C * DK / 8 / 64; j += 4) {
        const uint4 w0 = wg[64 * j + lane], w1 = wg[64 * (j + 1) + lane];
        const uint4 w2 = wg[64 * (j + 2) + lane], w3 = wg[64 * (j + 3) + lane];
        wput(64 * j + lane, w0);
        wput(64 * (j + 1) + lane, w1);
        wput(64 * (j + 2) + lane, w2);
        wput(64 * (j + 3) + lane, w3);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // operand layout: lane supplies row 16 rb + li, columns 32 q + 8 lg .. + 7
    bf16x8 kf[NB][NQ];
#pragma unroll
    for (int rb = 0; rb < NB; ++rb)
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        kf[rb][q] = *reinterpret_cast<const bf16x8 *>(R + (16 * rb + li) * Sh::RB + (32 * q + 8 * lg) * 2);

    // ---- Gram tiles G[rt][st] = K_rt W_st^T (st <= rt; W = K outside PGDN) and the
    // diagonal k_r . w_r (||k_r||^2); PGDN's write-key operands are read from their LDS
    // tile as the products need them (a register copy of the tile would leave the
    // wave too many registers for two waves per SIMD) --------------------------------
    auto wop = [&](int st, int q) -> bf16x8 {
      if constexpr (PG)
        return *reinterpret_cast<const bf16x8 *>(Wt + (16 * st + li) * Sh::RB + (32 * q + 8 * lg) * 2);
      else
        return kf[st][q];
    };
    f32x4 G[NB][NB];
#pragma unroll
    for (int st = 0; st < NB; ++st) {
      bf16x8 w[NQ];  // block st of the write keys (of K outside PGDN), as right operands
#pragma unroll
      for (int q = 0; q < NQ; ++q) w[q] = wop(st, q);
#pragma unroll
      for (int rt = st; rt < NB; ++rt) {
        f32x4 acc = zero4();
#pragma unroll
        for (int q = 0; q < NQ; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[rt][q], w[q], acc, 0, 0, 0);
        G[rt][st] = acc;
      }
      if constexpr (PG) __builtin_amdgcn_sched_barrier(0);  // keep the next block's reads after these
    }
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      // ||k_r||^2 of row 16 rt + li: diagonal tile, lane group li >> 2, element li & 3
      const f32x4 d = G[rt][rt];
      const int j = li & 3;
      const float nr = j == 0 ? d[0] : j == 1 ? d[1] : j == 2 ? d[2] : d[3];
      if (lg == (li >> 2)) sNrm[16 * rt + li] = nr;
    }
    // gate scan, Gam, d, beta (lane = chunk row); beta past the sequence end is 0
    const float gam = wave_inclusive_scan(elem_bits_to_f32(graw));
    const float gamC = lane_value(gam, C - 1);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the norms, written by other lanes
    const float el = elem_bits_to_f32(eraw);
    const float beta = lane < nrow ? (p.beta_direct ? el : el / (sNrm[lane] + p.eps)) : 0.f;
    sGam[lane] = gam;
    sBet[lane] = beta;
    {
      float *vec = reinterpret_cast<float *>(ws + TL::PACK);
      vec[lane] = gam;
      vec[C + lane] = __expf(gam);
      vec[2 * C + lane] = __expf(gamC - gam);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

    // ---- A = beta_r (K K^T)_rs exp(gamma_r - gamma_s), r > s ---------------------
    // (the K rows in R are dead: every lane's operand reads completed before the Gram)
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      const f32x4 gr4 = *reinterpret_cast<const f32x4 *>(sGam + 16 * rt + 4 * lg);
      const f32x4 br4 = *reinterpret_cast<const f32x4 *>(sBet + 16 * rt + 4 * lg);
#pragma unroll
      for (int st = 0; st <= rt; ++st) {
        const float gs = sGam[16 * st + li];
        const f32x4 acc = G[rt][st];
        f32x4 av;
        if (st < rt) {
#pragma unroll
          for (int j = 0; j < 4; ++j) av[j] = br4[j] * acc[j] * __expf(gr4[j] - gs);
          store4(Ablk + (rt * (rt - 1) / 2 + st) * 16 * LDA + li * LDA + 4 * lg, av);  // A^T[s'][r']
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool below = 4 * lg + j > li;
            av[j] = below ? br4[j] * acc[j] * __expf(gr4[j] - gs) : 0.f;
          }
          *reinterpret_cast<f32x4 *>(Td + (rt * 16 + li) * LDD + 4 * lg) = av;  // A_bb^T, fp32
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

    // packed image position of T'^T[s][col], col in grouped order (perm)
    auto pk = [&](int s, int pc) {
      return s < TL::RW ? s * Sh::IL0 + pc : TL::RW * Sh::IL0 + (s - TL::RW) * Sh::IL1 + (pc - TL::RW);
    };
    // LDS byte offset of 16-byte piece q of the packed workspace image
    auto piece_src = [&](int q) {
      const int e = 8 * q;
      return 2 * (e < TL::RW * C ? (e / C) * Sh::IL0 + e % C
                                 : TL::RW * Sh::IL0 + ((e - TL::RW * C) / (C - TL::RW)) * Sh::IL1 +
                                       (e - TL::RW * C) % (C - TL::RW));
    };
    auto put4 = [&](int s, int col, f32x4 v) {  // four consecutive columns col..col+3 (col % 4 == 0)
      store4(img + pk(s, Ops<bf16>::perm(col)), v);
    };

    // ---- diagonal blocks T_bb = (I + A_bb)^-1: lane = (block lg, column li) -----
    {
      float *At = Td + lg * 16 * LDD;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = (r == li) ? 1.f : 0.f;
      f32x4 cur[4], nxt[4];
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) cur[qd] = *reinterpret_cast<const f32x4 *>(At + 4 * qd);
#pragma unroll
      for (int s2 = 0; s2 < 15; ++s2) {
        if (s2 + 1 < 15) {
#pragma unroll
          for (int qd = 0; qd < 4; ++qd)
            if (4 * qd + 3 > s2 + 1) nxt[qd] = *reinterpret_cast<const f32x4 *>(At + (s2 + 1) * LDD + 4 * qd);
        }
#pragma unroll
        for (int r = s2 + 1; r < 16; ++r) x[r] = fmaf(-cur[r >> 2][r & 3], x[s2], x[r]);
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) cur[qd] = nxt[qd];
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // every lane has read its A_bb rows
      const float bs = sBet[16 * lg + li];
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const f32x4 t4 = {x[4 * qd], x[4 * qd + 1], x[4 * qd + 2], x[4 * qd + 3]};
        *reinterpret_cast<f32x4 *>(At + li * LDD + 4 * qd) = t4;  // T_bb, transposed
        put4(16 * lg + li, 16 * lg + 4 * qd, bs * t4);           // diagonal block of T'^T
      }
    }
    // the zero blocks inside the packed part: rows 16..31 x columns 0..15 and rows 48..63 x 32..47
    put4(16 + li, 4 * lg, zero4());
    put4(48 + li, 32 + 4 * lg, zero4());
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

    // ---- off-diagonal blocks level by level: T_ij = -T_ii sum_m A_im T_mj ---------
    f32x4 Toff[NB][NB];  // (live past this block only with TIMG)
    {
#pragma unroll
      for (int dist = 1; dist < NB; ++dist) {
#pragma unroll
        for (int i = dist; i < NB; ++i) {
          const int j = i - dist;
          f32x4 y = zero4();
#pragma unroll
          for (int m = j; m < i; ++m) {
            const M::Op a = M::ld_t(Ablk + (i * (i - 1) / 2 + m) * 16 * LDA, LDA, lane);
            const f32x4 bt = (m == j) ? *reinterpret_cast<const f32x4 *>(Td + (j * 16 + li) * LDD + 4 * lg) : Toff[m][j];
            y = M::mma(a, M::cvt(bt), y);
          }
          f32x4 ti;
#pragma unroll
          for (int e = 0; e < 4; ++e) ti[e] = Td[(i * 16 + 4 * lg + e) * LDD + li];
          const f32x4 t = -M::mma(M::cvt(ti), M::cvt(y), zero4());
          Toff[i][j] = t;
          put4(16 * j + li, 16 * i + 4 * lg, sBet[16 * j + li] * t);  // T'^T[16j + li][16i + 4lg + e]
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

    // ---- the packed image to the workspace, 16-byte pieces ----------------------
    static_assert(TL::PACK % 1024 == 0, "whole instructions of 16-byte pieces");
#pragma unroll
    for (int j = 0; j < TL::PACK / 1024; ++j) {
      const int pc = 64 * j + lane;
      reinterpret_cast<uint4 *>(ws)[pc] = *reinterpret_cast<const uint4 *>(R + piece_src(pc));
    }
    if constexpr (TIMG) {
      // the same image of T^T (no beta): the diagonal blocks from their transposed
      // copies in Td, the off-diagonal ones from registers, the zero blocks again
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the image above is read
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        put4(16 * lg + li, 16 * lg + 4 * qd, *reinterpret_cast<const f32x4 *>(Td + (lg * 16 + li) * LDD + 4 * qd));
      put4(16 + li, 4 * lg, zero4());
      put4(48 + li, 32 + 4 * lg, zero4());
#pragma unroll
      for (int dist = 1; dist < NB; ++dist)
#pragma unroll
        for (int i = dist; i < NB; ++i) put4(16 * (i - dist) + li, 16 * i + 4 * lg, Toff[i][i - dist]);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      char *wt = p.timg + ((size_t)h * p.nslot + slot) * TL::PACK;
#pragma unroll
      for (int j = 0; j < TL::PACK / 1024; ++j) {
        const int pc = 64 * j + lane;
        reinterpret_cast<uint4 *>(wt)[pc] = *reinterpret_cast<const uint4 *>(R + piece_src(pc));
      }
    }
    // the LDS of this slot is reused by the next: its reads have all completed
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };

  // ---- the run: the next slot's loads are in flight while this one computes ----
  // (one register set: the current slot's rows are in LDS before the next
  // slot's loads reuse the registers)
  if (s0 >= s1) return;
  size_t cur_tok;
  int cur_rows;
  describe(s0, cur_tok, cur_rows);
  if (cur_rows > 0) issue(cur_tok, cur_rows);
  for (int slot = s0; slot < s1; ++slot) {
    size_t nxt_tok;
    int nxt_rows;
    describe(slot + 1, nxt_tok, nxt_rows);
    const unsigned short graw = lgraw, eraw = leraw;
    if (cur_rows > 0) stage();
    if (nxt_rows > 0) issue(nxt_tok, nxt_rows);
    if (cur_rows > 0) process(slot, cur_rows, graw, eraw);
    cur_tok = nxt_tok;
    cur_rows = nxt_rows;
  }
}

// ---------------------------------------------------------------------------
// PGDN: the key accumulator at every chunk's start
// ---------------------------------------------------------------------------
// Token t's preconditioner needs A_t = A_0 + sum_{t' <= t} k_t' (.) k_t' over the whole
// sequence ("Preconditioned DeltaNet", section 2.C).  Two small passes before the prep
// kernel: the sum of k (.) k over each chunk's rows (all chunks at once, one thread per
// key coordinate, coalesced row reads), then a running sum over each sequence's chunks
// that leaves in every slot the accumulator at its chunk's start and writes the
// sequence's final accumulator.  Slots hold chunks as in the workspace.
template <int DK>
__global__ __launch_bounds__(128) void kla_pgdn_chunk_sum_kernel(ChunkParams p) {
  constexpr int C = 64, NT = 128, PPR = DK / 8, RPI = NT / PPR;  // pieces per row, rows per instruction
  __shared__ float red[RPI][DK];
  const int slot = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  int b = 0, t0 = 0, len = p.T, c = slot;
  if (p.cu) {
    int lo = 0, hi = p.nseq - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (mid + min(max(p.cu[mid], 0), p.T) / C <= slot) lo = mid; else hi = mid - 1;
    }
    t0 = min(max(p.cu[lo], 0), p.T);
    len = min(max(p.cu[lo + 1], t0), p.T) - t0;
    c = slot - (lo + t0 / C);
  } else {
    const int nchT = (p.T + C - 1) / C;
    b = slot / nchT;
    c = slot % nchT;
    if (b >= p.nseq) len = 0;
  }
  const int nrow = (c >= 0 && c * C < len) ? min(C, len - c * C) : 0;
  const bf16 *gk = static_cast<const bf16 *>(p.k) +
                   (((size_t)b * p.H + h) * (size_t)p.T + (size_t)t0 + (size_t)max(c, 0) * C) * DK;
  // thread t: coordinates 8 (t % PPR) .. +7 of rows t / PPR + RPI m (16-byte pieces, rows
  // past the chunk's end read as zero)
  const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(gk, nrow * DK * 2);
  uint4 kv[C / RPI];
#pragma unroll
  for (int m = 0; m < C / RPI; ++m) kv[m] = buffer_ld16(rk, (t + NT * m) * 16);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < C / RPI; ++m) {
    const bf16x8 e = __builtin_bit_cast(bf16x8, kv[m]);
#pragma unroll
    for (int x = 0; x < 8; ++x) acc[x] = fmaf((float)e[x], (float)e[x], acc[x]);
  }
#pragma unroll
  for (int x = 0; x < 8; ++x) red[t / PPR][8 * (t % PPR) + x] = acc[x];
  __syncthreads();
  if (t < DK) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < RPI; ++j) s += red[j][t];
    p.pg_acc[((size_t)h * p.nslot + slot) * DK + t] = s;
  }
}

template <int DK>
__global__ __launch_bounds__(DK) void kla_pgdn_acc_scan_kernel(ChunkParams p) {
  constexpr int C = 64;
  const int nh = blockIdx.x, i = threadIdx.x;
  const int n = nh / p.H, h = nh % p.H;
  int t0 = 0, t1 = p.T, slot0;
  if (p.cu) {
    t0 = min(max(p.cu[n], 0), p.T);
    t1 = min(max(p.cu[n + 1], t0), p.T);
    slot0 = n + t0 / C;
  } else {
    slot0 = n * ((p.T + C - 1) / C);
  }
  const int nch = (t1 - t0 + C - 1) / C;
  float a = p.pg_acc0 ? p.pg_acc0[(size_t)nh * DK + i] : 0.f;
  float *acc = p.pg_acc + ((size_t)h * p.nslot + slot0) * DK + i;
  for (int c0 = 0; c0 < nch; c0 += 16) {  // 16 chunk sums in flight at a time
    float sv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) sv[j] = c0 + j < nch ? acc[(size_t)(c0 + j) * DK] : 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (c0 + j < nch) acc[(size_t)(c0 + j) * DK] = a;
      a += sv[j];
    }
  }
  if (p.pg_accfin) p.pg_accfin[(size_t)nh * DK + i] = a;
}

// The write keys of one chunk (one workgroup of four waves per (chunk, head)): with
// A_start the accumulator at the chunk's start, A_r = A_start + sum_{t <= r} k_t (.) k_t
// per coordinate (each thread walks 32 rows of one coordinate) and the row's mean of A_r
// from the prefix of ||k_t||^2; w_r,i = p(A_r,i, mean_r) k_r,i, written as C rows of dk
// bf16 (rows past the chunk's end are zero).
template <int DK>
struct WkeysShape {
  static constexpr int C = 64, NT = 256;
  static constexpr int OFF_K = 0;                      // K rows, bf16 (then W)
  static constexpr int OFF_V = C * DK * 2;             // norms, then log2 of the row means; start sum
  static constexpr int OFF_T = OFF_V + (C + 4) * 4;    // per coordinate: sum of squares of rows 0..31
  static constexpr int BYTES = OFF_T + DK * 4;
};

template <int DK>
__global__ __launch_bounds__(256) void kla_pgdn_wkeys_kernel(ChunkParams p) {
  using Sh = WkeysShape<DK>;
  constexpr int C = 64, NT = Sh::NT;
  __shared__ __attribute__((aligned(16))) char smem[Sh::BYTES];
  bf16 *sk = reinterpret_cast<bf16 *>(smem + Sh::OFF_K);
  float *sv = reinterpret_cast<float *>(smem + Sh::OFF_V);
  float *stot = reinterpret_cast<float *>(smem + Sh::OFF_T);
  const int slot = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  int b = 0, t0 = 0, len = p.T, c = slot;
  if (p.cu) {
    int lo = 0, hi = p.nseq - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (mid + min(max(p.cu[mid], 0), p.T) / C <= slot) lo = mid; else hi = mid - 1;
    }
    t0 = min(max(p.cu[lo], 0), p.T);
    len = min(max(p.cu[lo + 1], t0), p.T) - t0;
    c = slot - (lo + t0 / C);
  } else {
    const int nchT = (p.T + C - 1) / C;
    b = slot / nchT;
    c = slot % nchT;
    if (b >= p.nseq) len = 0;
  }
  const int nrow = (c >= 0 && c * C < len) ? min(C, len - c * C) : 0;
  if (nrow == 0) return;  // uniform: no chunk in this slot
  const bf16 *gk = static_cast<const bf16 *>(p.k) +
                   (((size_t)b * p.H + h) * (size_t)p.T + (size_t)t0 + (size_t)c * C) * DK;
  const float *a0 = p.pg_acc + ((size_t)h * p.nslot + slot) * DK;
  // K rows (16-byte pieces; rows past the end as zero)
  {
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(gk, nrow * DK * 2);
    constexpr int NP = C * DK / 8 / NT;
    uint4 kv[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) kv[j] = buffer_ld16(rk, (t + NT * j) * 16);
#pragma unroll
    for (int j = 0; j < NP; ++j) reinterpret_cast<uint4 *>(sk)[t + NT * j] = kv[j];
  }
  __syncthreads();
  // row norms (four threads per row) and the start accumulator's sum
  {
    const int r = t >> 2, part = t & 3;
    float nk = 0.f;
#pragma unroll
    for (int m = 0; m < DK / 32; ++m)
      nk += Ops<bf16>::sumsq(*reinterpret_cast<const bf16x8 *>(sk + r * DK + 8 * (part + 4 * m)));
    nk += __shfl_xor(nk, 1);
    nk += __shfl_xor(nk, 2);
    if (part == 0) sv[r] = nk;
    if (t < 64) {
      float s0 = 0.f;
#pragma unroll
      for (int m = 0; m < DK / 64; ++m) s0 += a0[t + 64 * m];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) s0 += __shfl_xor(s0, off);
      if (t == 0) sv[C] = s0;
    }
    for (int i = t; i < DK; i += NT) {  // the first half's rows per coordinate (K still intact)
      float a = 0.f;
#pragma unroll 8
      for (int r = 0; r < 32; ++r) {
        const float kv = (float)sk[r * DK + i];
        a = fmaf(kv, kv, a);
      }
      stot[i] = a;
    }
  }
  __syncthreads();
  if (t < 64) {  // log2 of the row means: (start sum + prefix of the norms) / dk, lane = row
    const float m = (sv[C] + wave_inclusive_scan(sv[t])) * (1.f / DK);
    sv[t] = pgdn_log2_mean(m);
  }
  __syncthreads();
  // thread (coordinate i, half hf) walks its 32 rows with the accumulator in a register
  // (the second half starts from the first half's total) and replaces k by w in place
  const PgdnK pk = pgdn_k(p.band_c);
  for (int e = t; e < 2 * DK; e += NT) {
    const int i = e % DK, hf = e / DK;
    const float a00 = a0[i];
    float a = hf ? a00 + stot[i] : a00;
#pragma unroll 4
    for (int r = 32 * hf; r < 32 * hf + 32; ++r) {
      const float kv = (float)sk[r * DK + i];
      a = fmaf(kv, kv, a);
      sk[r * DK + i] = (bf16)(pgdn_precond(a, sv[r], pk) * kv);
    }
  }
  __syncthreads();
  char *wg = p.pg_w + ((size_t)h * p.nslot + slot) * (C * DK * 2);
#pragma unroll
  for (int j = 0; j < C * DK / 8 / NT; ++j)
    reinterpret_cast<uint4 *>(wg)[t + NT * j] = reinterpret_cast<const uint4 *>(sk)[t + NT * j];
}

// ---------------------------------------------------------------------------
// scan kernel: roles and LDS plan
// ---------------------------------------------------------------------------
// Waves of a workgroup.  Step i (one barrier each, i = -1 .. nch) has
//   CHAIN[2] the state scan of chunk i (half of the state columns each)
//   PW[2]    Diag(Gam) Q S and the causal scores of chunk i; output of chunk i-1
//   LOADK    K rows of chunk i+1 into LDS (coalesced loads issued three steps ahead)
//   LOADT    T'^T, gamma/Gam/d and the V slice of chunk i+1 into LDS
//   LOADQ    Q rows of chunk i+1 into LDS (likewise)
// The P waves issue no global loads: their output stores would otherwise sit
// in the same wait counter as the loads.  Waves w and w+4 share a SIMD.
enum Role { CHAIN0 = 0, CHAIN1 = 1, PW0 = 2, PW1 = 3, LOADK = 4, LOADT = 5, LOADQ = 6, LOADW = 7 };
constexpr int kWaves = 7;  // (PGDN: an eighth, LOADW, brings the write keys of chunk i+1)

template <typename E, int C, int DK, int NCT, bool PG = false>
struct ChunkShape {
  static constexpr int NB = C / 16;            // 16-row blocks per chunk
  static constexpr int DVT = 16 * NCT;         // state columns per workgroup
  static constexpr int NCW = (NCT + 1) / 2;    // 16-column tiles per chain wave
  static constexpr int NT = 64 * (kWaves + (PG ? 1 : 0));
  static constexpr int PAD = LdsPad<E>::V;
  static constexpr int LDK = DK + PAD;         // K and Q rows (grouped columns)
  static constexpr int LDC = TpLayout<E, C>::LDC;
  // V slice rows (natural); a row length of 32 mod 64 bytes keeps the
  // transposing reads conflict-free
  static constexpr int LDV = ((DVT + PAD) * (int)sizeof(E)) % 64 == 32 ? DVT + PAD : DVT + 2 * PAD;
  static constexpr int KG = Ops<E>::KG;
  // sizes in bytes
  static constexpr int K_SLOT = C * LDK * (int)sizeof(E);
  static constexpr int V_SLOT = C * LDV * (int)sizeof(E);
  // T'^T image, then gamma, Gam, d; compact (rows >= 32 hold their last 32 columns only,
  // all the T' X products read there) where four column tiles or PGDN's write keys need the room
  static constexpr bool COMPACT = NCT > 2 || PG;
  static constexpr int TP_SLOT = COMPACT ? TpLayout<E, C>::LDS_BYTES_C : TpLayout<E, C>::LDS_BYTES;
  static constexpr int TP_VEC = COMPACT ? TpLayout<E, C>::TP_IMG_C : TpLayout<E, C>::TP_IMG;
  static constexpr int SU_S = NCT * (DK / KG) * 64 * 16;   // chunk-start S groups, 16 B per lane
  static constexpr int SU_U = NCT * (C / KG) * 64 * 16;    // U~ groups
  static constexpr int SU_SLOT = SU_S + SU_U;
  // offsets
  static constexpr int OFF_K = 0;
  static constexpr int OFF_V = OFF_K + 2 * K_SLOT;
  static constexpr int OFF_TP = OFF_V + 2 * V_SLOT;
  static constexpr int OFF_SU = OFF_TP + 2 * TP_SLOT;
  static constexpr int OFF_Q = OFF_SU + 2 * SU_SLOT;
  // PGDN: write-key rows, 16-byte padding (the LDS budget allows no more)
  static constexpr int LDW = DK + 16 / (int)sizeof(E);
  static constexpr int W_SLOT = PG ? C * LDW * (int)sizeof(E) : 0;
  static constexpr int OFF_W = OFF_Q + 2 * K_SLOT;
  static constexpr int BYTES = OFF_W + 2 * W_SLOT;

  static_assert(C == 16 || C == 64, "chunk");
  static_assert(C % KG == 0 && DK % KG == 0 && DK % Ops<E>::KSTEP == 0, "dk");
  static_assert(K_SLOT % 16 == 0 && V_SLOT % 16 == 0 && TP_SLOT % 16 == 0,
                "lds align");
  static_assert((LDK * (int)sizeof(E)) % 16 == 0 && (LDC * (int)sizeof(E)) % 16 == 0 &&
                    (LDV * (int)sizeof(E)) % 16 == 0, "row align");
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <typename E, int C, int DK, int NCT, bool PG = false>
__global__ __launch_bounds__(64 * (kWaves + (PG ? 1 : 0))) void kla_chunk_kernel(ChunkParams p) {
  using Sh = ChunkShape<E, C, DK, NCT, PG>;
  using TL = TpLayout<E, C>;
  using O = Ops<E>;
  using Grp = typename O::Grp;
  constexpr int NB = Sh::NB, DVT = Sh::DVT, LDK = Sh::LDK, LDC = Sh::LDC, LDV = Sh::LDV;
  constexpr int KG = O::KG, TPG = KG / 16;
  constexpr int NQG = DK / KG;  // contraction groups over dk
  constexpr int NCG = C / KG;   // contraction groups over the chunk

  __shared__ __attribute__((aligned(16))) char smem[Sh::BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15;  // row / column inside a 16-wide tile
  const int lg = lane >> 4;  // lane group 0..3

  // ---- which (sequence, head, column slice) this workgroup owns ----------
  // Workgroups are dispatched in blockIdx order and blockIdx % 8 picks the
  // XCD.  (sequence, head) groups go round-robin over the XCDs with all
  // column slices of a group on one XCD (they share K, Q and the workspace
  // through its L2); packed sequences come longest first (order[]), so the
  // longest chains start first.  The grid is padded to whole rounds of 8.
  const int xcd = blockIdx.x & 7, i8 = blockIdx.x >> 3;
  const int gidx = (i8 / p.n_tiles) * 8 + xcd;
  if (gidx >= p.ngroups) return;  // padding (uniform per workgroup)
  const int jt = i8 % p.n_tiles;
  const int h = gidx % p.H;
  // segment (ChunkParams::seg_first): segment g of sequence n, its chunks from c_lo on
  int n, seg = 0, g = 0;
  if (p.seg_first) {
    seg = gidx / p.H;
    if (seg >= p.seg_first[p.nseq]) return;  // (only with a cu_seqlens that disagrees with its mirror)
    n = seg_sequence(p.seg_first, p.nseq, seg);
    g = seg - p.seg_first[n];
  } else {
    n = p.order ? p.order[gidx / p.H] : gidx / p.H;
  }
  const bool idt = jt >= p.n_vtiles;  // an identity tile
  if (idt && g == 0) return;          // a first segment needs no transfer map
  const int nh = n * p.H + h;  // (sequence, head) index of the state arrays
  int b = n, t0 = 0, t1 = p.T, slot0;
  if (p.cu) {
    b = 0;
    t0 = min(max(p.cu[n], 0), p.T);
    t1 = min(max(p.cu[n + 1], t0), p.T);
    slot0 = n + t0 / C;
  } else {
    slot0 = n * ((p.T + C - 1) / C);
  }
  if (p.seg_first) {
    // (a segment past the sequence's end, possible only with a cu_seqlens that
    // disagrees with its mirror, is empty)
    const int c_lo = (int)min((long long)g * p.seg_chunks, (long long)(t1 - t0 + C - 1) / C);
    slot0 += c_lo;
    t0 = (int)min((long long)t0 + (long long)c_lo * C, (long long)t1);
    t1 = (int)min((long long)t1, (long long)t0 + (long long)p.seg_chunks * C);
  }
  const int len = t1 - t0;
  const int nch = (len + C - 1) / C;
  const size_t row0 = ((size_t)b * p.H + h) * (size_t)p.T + (size_t)t0;
  const E *gq = static_cast<const E *>(p.q);
  const E *gk = static_cast<const E *>(p.k);
  const E *gv = static_cast<const E *>(p.v);
  const char *ws = p.ws + (size_t)h * p.nslot * TL::BYTES;
  const int dv = p.dv;
  // this tile's state arrays (row stride ld_s, first column col_s): start (nullptr:
  // zero, or I for an identity tile) and end; its output rows (row stride ld_s)
  const int ld_s = idt ? DK : dv;
  const int col_s = (idt ? jt - p.n_vtiles : jt) * DVT;
  const float *s_init = idt || g > 0 || !p.s0 ? nullptr : p.s0 + (size_t)nh * DK * dv;
  float *s_fin;
  if (!p.seg_first)
    s_fin = p.sfin ? p.sfin + (size_t)nh * DK * dv : nullptr;
  else if (idt)
    s_fin = p.seg_m + ((size_t)seg * p.H + h) * DK * DK;
  else
    s_fin = p.seg_d + ((size_t)seg * p.H + h) * DK * dv;
  E *go = static_cast<E *>(idt ? p.eout : p.o);
  auto s_start = [&](int row, int col) {
    return idt ? (row == col ? 1.f : 0.f) : (s_init ? s_init[(size_t)row * ld_s + col] : 0.f);
  };
  auto nrow_of = [&](int c) { return min(C, len - c * C); };
  auto tok0_of = [&](int c) { return row0 + (size_t)c * C; };
  // a prefetch past the last chunk re-reads the last chunk
  auto clampc = [&](int c) { return min(max(c, 0), nch - 1); };
  // steps run from -1 to iend (an even count: the load waves alternate two
  // register sets); steps past nch do nothing but the barrier
  const int iend = nch + (nch & 1);

  if (nch == 0) {
    // empty sequence (or segment): the final state is the initial state
    if (s_fin) {
      for (int e = threadIdx.x; e < DK * DVT; e += Sh::NT) {
        const int row = e / DVT, col = col_s + e % DVT;
        s_fin[(size_t)row * ld_s + col] = s_start(row, col);
      }
    }
    return;
  }

  // ---- LDS views (chunk c in slot c & 1) --------------------------------------
  auto sK = [&](int c) { return reinterpret_cast<E *>(smem + Sh::OFF_K + (c & 1) * Sh::K_SLOT); };
  auto sQ = [&](int c) { return reinterpret_cast<E *>(smem + Sh::OFF_Q + (c & 1) * Sh::K_SLOT); };
  auto sV = [&](int c) { return reinterpret_cast<E *>(smem + Sh::OFF_V + (c & 1) * Sh::V_SLOT); };
  auto sTp = [&](int c) { return reinterpret_cast<E *>(smem + Sh::OFF_TP + (c & 1) * Sh::TP_SLOT); };
  // per-chunk row vectors: gamma, Gam = exp(gamma), d = exp(gamma_C - gamma)
  auto sVec = [&](int c) {
    return reinterpret_cast<float *>(smem + Sh::OFF_TP + (c & 1) * Sh::TP_SLOT + Sh::TP_VEC);
  };
  auto sSuS = [&](int c) { return reinterpret_cast<Grp *>(smem + Sh::OFF_SU + (c & 1) * Sh::SU_SLOT); };
  // the rows the state is written with: K, or PGDN's write keys
  auto sWk = [&](int c) {
    return PG ? reinterpret_cast<E *>(smem + Sh::OFF_W + (c & 1) * Sh::W_SLOT) : sK(c);
  };
  constexpr int LDWK = PG ? Sh::LDW : LDK;
  auto sSuU = [&](int c) {
    return reinterpret_cast<Grp *>(smem + Sh::OFF_SU + (c & 1) * Sh::SU_SLOT + Sh::SU_S);
  };

  if (wave == CHAIN0 || wave == CHAIN1) {
    // =================== chain: the sequential state scan ====================
    // Two chain waves, each with NCW of the workgroup's 16-column tiles (the
    // columns of S evolve independently; with one tile the second is idle).
    // Its part of S (DK rows, fp32) lives in the accumulators for the whole
    // sequence: accS[ct][it] is the 16x16 tile (rows 16 it.., columns
    // 16 (CT0 + ct)..).
    auto chain = [&](auto ct0_c) {
    constexpr int CT0 = decltype(ct0_c)::value;
    constexpr int NCW = CT0 < NCT ? (NCT - CT0 < Sh::NCW ? NCT - CT0 : Sh::NCW) : 0;
    constexpr int NCW1 = NCW > 0 ? NCW : 1;
    f32x4 accS[NCW1][DK / 16];
#pragma unroll
    for (int ct = 0; ct < NCW; ++ct) {
      const int col = col_s + 16 * (CT0 + ct) + li;
#pragma unroll
      for (int it = 0; it < DK / 16; ++it)
#pragma unroll
        for (int j = 0; j < 4; ++j) accS[ct][it][j] = s_start(16 * it + 4 * lg + j, col);
    }
    // chunk-start S as right operands, straight from the accumulators; also
    // published for the P waves (their Q S of that chunk)
    Grp sb[NCW1][NQG];
    auto publish = [&](int c) {
      Grp *suS = sSuS(c);
#pragma unroll
      for (int ct = 0; ct < NCW; ++ct)
#pragma unroll
        for (int q = 0; q < NQG; ++q) {
          sb[ct][q] = O::b_from_d(&accS[ct][q * TPG]);
          suS[((CT0 + ct) * NQG + q) * 64 + lane] = sb[ct][q];
        }
      if (p.states) {
        // the chunk-start state of chunk c, in operand groups (coalesced 16-byte stores)
        const size_t slot = (size_t)h * p.nslot + slot0 + c;
#pragma unroll
        for (int ct = 0; ct < NCW; ++ct)
#pragma unroll
          for (int q = 0; q < NQG; ++q) {
            const size_t grp = (slot * (size_t)(dv / 16) + (size_t)(jt * NCT + CT0 + ct)) * NQG + q;
            reinterpret_cast<Grp *>(p.states + grp * 64 * 16)[lane] = sb[ct][q];
          }
      }
    };
    __syncthreads();
    for (int i = -1; i <= iend; ++i) {
      if (i == -1) publish(0);
      if (NCW > 0 && i >= 0 && i < nch) {
        const int c = i;
        const E *K = sK(c);
        const E *V = sV(c);
        const E *TpT = sTp(c);
        const float *vec = sVec(c);
        Grp *suU = sSuU(c);
        // K S
        f32x4 x[NCW1][NB];
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
          for (int ct = 0; ct < NCW; ++ct) x[ct][rt] = zero4();
#pragma unroll
          for (int q = 0; q < NQG; ++q) {
            const Grp a = O::a_row(K + (16 * rt + li) * LDK, q * KG, lg);
#pragma unroll
            for (int ct = 0; ct < NCW; ++ct) x[ct][rt] = O::mma_grp(a, sb[ct][q], x[ct][rt]);
          }
        }
        // X = V - Diag(Gam) K S
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) {
          const f32x4 gm = *reinterpret_cast<const f32x4 *>(vec + C + 16 * rt + 4 * lg);
#pragma unroll
          for (int ct = 0; ct < NCW; ++ct) x[ct][rt] = O::col4(V, LDV, 16 * rt, 16 * (CT0 + ct), lane) - gm * x[ct][rt];
        }
        Grp xb[NCW1][NCG];
#pragma unroll
        for (int ct = 0; ct < NCW; ++ct)
#pragma unroll
          for (int q = 0; q < NCG; ++q) xb[ct][q] = O::b_from_d(&x[ct][q * TPG]);
        // U~ = T' X   (T' lower triangular: skip the zero groups; T' is stored
        // transposed)
        f32x4 u[NCW1][NB];
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
          for (int ct = 0; ct < NCW; ++ct) u[ct][rt] = zero4();
#pragma unroll
          for (int q = 0; q * KG < 16 * (rt + 1); ++q) {
            Grp a;
            if (Sh::COMPACT && q * KG >= TL::RW)
              a = O::a_trans(TpT + TL::RW * LDC, TL::LD2, q * KG - TL::RW, 16 * rt - TL::RW, lane);
            else
              a = O::a_trans(TpT, LDC, q * KG, 16 * rt, lane);
#pragma unroll
            for (int ct = 0; ct < NCW; ++ct) u[ct][rt] = O::mma_grp(a, xb[ct][q], u[ct][rt]);
          }
        }
        // U~ groups for the P waves; Diag(d) U~ groups for the update
        Grp dub[NCW1][NCG];
#pragma unroll
        for (int ct = 0; ct < NCW; ++ct)
#pragma unroll
          for (int q = 0; q < NCG; ++q) {
            suU[((CT0 + ct) * NCG + q) * 64 + lane] = O::b_from_d(&u[ct][q * TPG]);
            f32x4 du[TPG];
#pragma unroll
            for (int tt = 0; tt < TPG; ++tt) {
              const int r16 = 16 * (q * TPG + tt);
              du[tt] = *reinterpret_cast<const f32x4 *>(vec + 2 * C + r16 + 4 * lg) * u[ct][q * TPG + tt];
            }
            dub[ct][q] = O::b_from_d(du);
          }
        // S <- Gam_C S + K^T Diag(d) U~  (PGDN: W^T)
        const float gC = vec[C + C - 1];
        const E *Wk = sWk(c);
#pragma unroll
        for (int it = 0; it < DK / 16; ++it) {
#pragma unroll
          for (int ct = 0; ct < NCW; ++ct) accS[ct][it] = gC * accS[ct][it];
#pragma unroll
          for (int q = 0; q < NCG; ++q) {
            const Grp a = O::a_trans(Wk, LDWK, q * KG, 16 * it, lane);
#pragma unroll
            for (int ct = 0; ct < NCW; ++ct) accS[ct][it] = O::mma_grp(a, dub[ct][q], accS[ct][it]);
          }
        }
        if (c + 1 < nch) publish(c + 1);
      }
      lds_barrier();
    }
    if (s_fin) {
#pragma unroll
      for (int ct = 0; ct < NCW; ++ct) {
        const int col = col_s + 16 * (CT0 + ct) + li;
#pragma unroll
        for (int it = 0; it < DK / 16; ++it)
#pragma unroll
          for (int j = 0; j < 4; ++j) s_fin[(size_t)(16 * it + 4 * lg + j) * ld_s + col] = accS[ct][it][j];
      }
    }
    };
    if (wave == CHAIN0)
      chain(std::integral_constant<int, 0>{});
    else
      chain(std::integral_constant<int, Sh::NCW>{});
  } else if (wave == PW0 || wave == PW1) {
    // =================== P waves: scores and output rows ======================
    // For its row blocks rt, a P wave forms the causal scores of chunk i as
    // P^T = K Q^T (the accumulator layout of P^T is exactly the left-operand
    // layout P needs in P U~, so P stays in registers) and Diag(Gam) Q S with
    // the chunk-start state; one step later, when the chain has U~, it adds
    // P U~ and writes those output rows.
    auto pwave = [&](auto part_c) {
      constexpr int part = decltype(part_c)::value;
      using BL = OwnBlocks<NB, part>;
      constexpr int NOWN = BL::N;
      constexpr int NOW1 = NOWN > 0 ? NOWN : 1;
      f32x4 ao[NCT][NOW1];  // output of the pending chunk, as O^T tiles
      Grp pa[NOW1][NCG];    // its P rows as left operands
      const bool outputs = p.states == nullptr;  // states mode writes no outputs
      __syncthreads();
      for (int i = -1; i <= iend; ++i) {
        if (NOWN > 0 && outputs && i >= 1 && i <= nch) {
          // ---- output of chunk i-1: O = Diag(Gam) Q S + P U~ ----
          const int c = i - 1;
          const int nrow = nrow_of(c);
          const size_t tok0 = tok0_of(c);
          const Grp *suU = sSuU(c);
          // ao holds O^T tiles (lane: one output row, 4 consecutive columns),
          // so the rows go straight to memory
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            Grp ub[NCG];
#pragma unroll
            for (int q = 0; q < NCG; ++q) ub[q] = suU[(ct * NCG + q) * 64 + lane];
#pragma unroll
            for (int k = 0; k < NOWN; ++k) {
              const int rt = BL::at(k);
#pragma unroll
              for (int q = 0; q * KG < 16 * (rt + 1); ++q) ao[ct][k] = O::mma_grp(ub[q], pa[k][q], ao[ct][k]);
            }
          }
#pragma unroll
          for (int k = 0; k < NOWN; ++k) {
            const int r = 16 * BL::at(k) + li;
            if (r < nrow) {
              E *orow = go + (tok0 + r) * (size_t)ld_s + col_s + 4 * lg;
#pragma unroll
              for (int ct = 0; ct < NCT; ++ct) store4(orow + 16 * ct, ao[ct][k]);
            }
          }
        }
        if (NOWN > 0 && outputs && i >= 0 && i < nch) {
          // ---- chunk i: P rows and Diag(Gam) Q S ----
          const int c = i;
          const E *Q = sQ(c);
          const E *K = sWk(c);  // the causal scores use the write keys (PGDN: W)
          const float *vec = sVec(c);
          const Grp *suS = sSuS(c);
          Grp qa[NOW1][NQG];
#pragma unroll
          for (int k = 0; k < NOWN; ++k)
#pragma unroll
            for (int q = 0; q < NQG; ++q) qa[k][q] = O::a_row(Q + (16 * BL::at(k) + li) * LDK, q * KG, lg);
          // P^T tiles: D[s][r] = K_s . q_r, lane column r = 16 rt + li, rows s = 16 st + 4 lg + j
          f32x4 pt[NOW1][NB];
#pragma unroll
          for (int st = 0; st < NB; ++st) {
            if (st > BL::at(NOWN - 1)) continue;
            Grp kb[NQG];
#pragma unroll
            for (int q = 0; q < NQG; ++q) kb[q] = O::a_row(K + (16 * st + li) * LDWK, q * KG, lg);
#pragma unroll
            for (int k = 0; k < NOWN; ++k) {
              if (st > BL::at(k)) continue;
              pt[k][st] = zero4();
#pragma unroll
              for (int q = 0; q < NQG; ++q) pt[k][st] = O::mma_grp(kb[q], qa[k][q], pt[k][st]);
            }
          }
          // decay and causal mask; the accumulator layout of P^T is the
          // left-operand layout of the P rows in P U~
#pragma unroll
          for (int k = 0; k < NOWN; ++k) {
            const int rt = BL::at(k);
            const float gr = vec[16 * rt + li];
#pragma unroll
            for (int st = 0; st <= rt; ++st) {
              const f32x4 gs = *reinterpret_cast<const f32x4 *>(vec + 16 * st + 4 * lg);
#pragma unroll
              for (int j = 0; j < 4; ++j)
                pt[k][st][j] = (st < rt || 4 * lg + j <= li) ? pt[k][st][j] * __expf(gr - gs[j]) : 0.f;
            }
#pragma unroll
            for (int q = 0; q * KG < 16 * (rt + 1); ++q) {
              f32x4 tl[TPG];
#pragma unroll
              for (int tt = 0; tt < TPG; ++tt) tl[tt] = (q * TPG + tt <= rt) ? pt[k][q * TPG + tt] : zero4();
              pa[k][q] = O::b_from_d(tl);
            }
          }
          // Diag(Gam) Q S
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            Grp sbq[NQG];
#pragma unroll
            for (int q = 0; q < NQG; ++q) sbq[q] = suS[(ct * NQG + q) * 64 + lane];
#pragma unroll
            for (int k = 0; k < NOWN; ++k) {
              ao[ct][k] = zero4();
#pragma unroll
              for (int q = 0; q < NQG; ++q) ao[ct][k] = O::mma_grp(sbq[q], qa[k][q], ao[ct][k]);
            }
          }
          // Diag(Gam): lane li holds row 16 rt + li
#pragma unroll
          for (int k = 0; k < NOWN; ++k) {
            const float gm = vec[C + 16 * BL::at(k) + li];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) ao[ct][k] = gm * ao[ct][k];
          }
        }
        lds_barrier();
      }
    };
    if (wave == PW0)
      pwave(std::integral_constant<int, 0>{});
    else
      pwave(std::integral_constant<int, 1>{});
  } else if (wave == LOADK) {
    // =================== K rows of chunk i+1 ==================================
    // Three register sets, loads issued three steps ahead (the steps rotate
    // through them, so the set is a compile-time choice).  Stores past the
    // last chunk rewrite a slot nobody reads any more.
    RowLoad<E, DK, AllBlocks<NB>> kin[3];
    kin[0].issue(gk + tok0_of(0) * DK, nrow_of(0), lane);
    kin[1].issue(gk + tok0_of(clampc(1)) * DK, nrow_of(clampc(1)), lane);
    kin[2].issue(gk + tok0_of(clampc(2)) * DK, nrow_of(clampc(2)), lane);
    __syncthreads();
    auto step = [&](int i, auto set_c) {
      constexpr int S = decltype(set_c)::value;
      kin[S].put(sK(i + 1), LDK, lane, [](int, int row) { return row; });
      kin[S].issue(gk + tok0_of(clampc(i + 4)) * DK, nrow_of(clampc(i + 4)), lane);
      lds_barrier();
    };
    // set (i + 1) mod 3 holds chunk i + 1 at step i; the steps run from -1 to iend
    int i = -1;
    for (; i + 2 <= iend; i += 3) {
      step(i, std::integral_constant<int, 0>{});
      step(i + 1, std::integral_constant<int, 1>{});
      step(i + 2, std::integral_constant<int, 2>{});
    }
    if (i <= iend) step(i++, std::integral_constant<int, 0>{});
    if (i <= iend) step(i++, std::integral_constant<int, 1>{});
  } else if (PG && wave == LOADW) {
    // =================== PGDN write keys of chunk i+1 (two sets, two steps ahead) ====
    const E *gw = reinterpret_cast<const E *>(p.pg_w) + ((size_t)h * p.nslot + slot0) * (C * DK);
    RowLoad<E, DK, AllBlocks<NB>> win[2];
    win[0].issue(gw, C, lane);
    win[1].issue(gw + (size_t)clampc(1) * (C * DK), C, lane);
    __syncthreads();
    auto step = [&](int i, auto set_c) {
      constexpr int S = decltype(set_c)::value;
      win[S].put(sWk(i + 1), Sh::LDW, lane, [](int, int row) { return row; });
      win[S].issue(gw + (size_t)clampc(i + 3) * (C * DK), C, lane);
      lds_barrier();
    };
    for (int i = -1; i <= iend; i += 2) {
      step(i, std::integral_constant<int, 0>{});
      step(i + 1, std::integral_constant<int, 1>{});
    }
  } else if (wave == LOADQ) {
    // =================== Q rows of chunk i+1 (three sets, three steps ahead) ====
    if (p.states) {
      // states mode has no outputs, so nothing reads Q: keep the barrier count only
      __syncthreads();
      for (int i = -1; i <= iend; ++i) lds_barrier();
      return;
    }
    RowLoad<E, DK, AllBlocks<NB>> qin[3];
    qin[0].issue(gq + tok0_of(0) * DK, nrow_of(0), lane);
    qin[1].issue(gq + tok0_of(clampc(1)) * DK, nrow_of(clampc(1)), lane);
    qin[2].issue(gq + tok0_of(clampc(2)) * DK, nrow_of(clampc(2)), lane);
    __syncthreads();
    auto step = [&](int i, auto set_c) {
      constexpr int S = decltype(set_c)::value;
      qin[S].put(sQ(i + 1), LDK, lane, [](int, int row) { return row; });
      qin[S].issue(gq + tok0_of(clampc(i + 4)) * DK, nrow_of(clampc(i + 4)), lane);
      lds_barrier();
    };
    int i = -1;
    for (; i + 2 <= iend; i += 3) {
      step(i, std::integral_constant<int, 0>{});
      step(i + 1, std::integral_constant<int, 1>{});
      step(i + 2, std::integral_constant<int, 2>{});
    }
    if (i <= iend) step(i++, std::integral_constant<int, 0>{});
    if (i <= iend) step(i++, std::integral_constant<int, 1>{});
  } else {
    // =================== T'^T, gamma/Gam/d and the V slice of chunk i+1 ========
    // (two sets, two steps ahead, as for K, when the registers allow)
    using TC = ImgCopy<E, C, Sh::COMPACT>;
    constexpr int NSET = TC::NPL <= 20 ? 2 : 1;
    TC tin[NSET];
    VSliceLoad<E, C, DVT> vin[NSET];
    auto fetch = [&](int c, auto set_c) {
      constexpr int S = decltype(set_c)::value;
      tin[S].issue(ws + (size_t)(slot0 + c) * TL::BYTES, lane);
      // an identity tile's v is zero: a load range of no rows reads zeros
      vin[S].issue(gv + tok0_of(c) * dv, idt ? 0 : nrow_of(c), dv, idt ? 0 : jt * DVT, lane);
    };
    fetch(0, std::integral_constant<int, 0>{});
    if constexpr (NSET == 2) fetch(clampc(1), std::integral_constant<int, NSET - 1>{});
    __syncthreads();
    auto step = [&](int i, auto set_c) {
      constexpr int S = decltype(set_c)::value;
      tin[S].put(sTp(i + 1), lane);
      vin[S].put(sV(i + 1), LDV, lane);
      fetch(clampc(i + 1 + NSET), set_c);
      lds_barrier();
    };
    for (int i = -1; i <= iend; i += 2) {
      step(i, std::integral_constant<int, 0>{});
      step(i + 1, std::integral_constant<int, NSET - 1>{});
    }
  }
}

// ---------------------------------------------------------------------------
// reverse scan kernel: the backward pass's state gradients
// ---------------------------------------------------------------------------
// The gradient of a scalar loss with respect to the chunk-end state, dS', runs
// backwards through the chunks by the adjoint of the chunk step above (T' =
// T Diag(beta), Gam, d and Gam_C of the chunk; P the decayed causal scores):
//
//   Y   = P^T dO + Diag(d) K dS'              (the gradient of U~)
//   dX  = T'^T Y                              (the gradient of X)
//   dS  = Gam_C dS' + Q^T Diag(Gam) dO - K^T Diag(Gam) dX
//
// and dS becomes the dS' of the previous chunk.  It runs on the forward's own
// machinery: the same T'^T images and gamma/Gam/d vectors (the forward prep
// kernel's workspace), the same loaders (dO in place of V, chunks in reverse
// order), and a chain wave per 16 state columns holding dS' in MFMA
// accumulators -- K dS' is the forward's K S, K^T and Q^T products its state
// update, T'^T Y reads the T'^T image by rows where the forward reads it by
// columns.  The P waves form P (as Q K^T) for the column blocks they own and
// P^T dO for the matching rows of Y, which only the chunk's inputs determine;
// they hand it to the chain through LDS in the middle of the step, so a step
// has two LDS-only barriers: (1) chain: K dS' and Gam_C dS' + Q^T Diag(Gam) dO,
// P waves: P^T dO; (2) chain: Y, dX and the K^T term.  In ChunkParams:
// s0 = dL/dS_final (or nullptr), sfin = the initial-state gradient (or
// nullptr), v = dO, states = where dS' of every chunk goes (the operand-group
// layout of states mode), ws = the forward workspace.
template <typename E, int C, int DK, int NCT>
struct RevShape {
  using F = ChunkShape<E, C, DK, NCT>;
  // four column tiles: eight waves, four chain waves of one tile each (the chain's
  // products dominate a step: 108 MFMAs per chain wave with two tiles each against 32
  // per P wave) and one loader for both K and Q
  static constexpr bool W8 = NCT == 4;
  static constexpr int NW = W8 ? 8 : kWaves;
  static constexpr int NB = F::NB, DVT = F::DVT, NCW = W8 ? 1 : F::NCW, NT = 64 * NW;
  static constexpr int LDK = F::LDK, LDC = F::LDC, LDV = F::LDV;
  static constexpr int K_SLOT = F::K_SLOT, V_SLOT = F::V_SLOT, TP_SLOT = TpLayout<E, C>::LDS_BYTES;
  static constexpr int YP = NCT * NB * 64 * 16;  // P^T dO tiles, fp32 accumulator layout
  static constexpr int OFF_K = 0;
  static constexpr int OFF_V = OFF_K + 2 * K_SLOT;
  static constexpr int OFF_TP = OFF_V + 2 * V_SLOT;
  static constexpr int OFF_YP = OFF_TP + 2 * TP_SLOT;
  static constexpr int OFF_Q = OFF_YP + YP;
  static constexpr int BYTES = OFF_Q + 2 * K_SLOT;
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <int NCT>
constexpr int rev_threads() { return 64 * (NCT == 4 ? 8 : kWaves); }

template <typename E, int C, int DK, int NCT>
__global__ __launch_bounds__(rev_threads<NCT>()) void kla_chunk_rev_kernel(ChunkParams p) {
  static_assert(rev_threads<NCT>() == RevShape<E, C, DK, NCT>::NT, "workgroup size");
  using Sh = RevShape<E, C, DK, NCT>;
  using TL = TpLayout<E, C>;
  using O = Ops<E>;
  using Grp = typename O::Grp;
  constexpr int NB = Sh::NB, DVT = Sh::DVT, LDK = Sh::LDK, LDC = Sh::LDC, LDV = Sh::LDV;
  constexpr int KG = O::KG, TPG = KG / 16;
  constexpr int NQG = DK / KG;  // contraction groups over dk
  constexpr int NCG = C / KG;   // contraction groups over the chunk

  __shared__ __attribute__((aligned(16))) char smem[Sh::BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15;
  const int lg = lane >> 4;

  // ---- which (sequence, head, column slice): as the forward scan -------------
  const int xcd = blockIdx.x & 7, i8 = blockIdx.x >> 3;
  const int gidx = (i8 / p.n_tiles) * 8 + xcd;
  if (gidx >= p.ngroups) return;  // padding (uniform per workgroup)
  const int jt = i8 % p.n_tiles;
  const int h = gidx % p.H;
  const int n = p.order ? p.order[gidx / p.H] : gidx / p.H;
  const int nh = n * p.H + h;
  int b = n, t0 = 0, t1 = p.T, slot0;
  if (p.cu) {
    b = 0;
    t0 = min(max(p.cu[n], 0), p.T);
    t1 = min(max(p.cu[n + 1], t0), p.T);
    slot0 = n + t0 / C;
  } else {
    slot0 = n * ((p.T + C - 1) / C);
  }
  const int len = t1 - t0;
  const int nch = (len + C - 1) / C;
  const size_t row0 = ((size_t)b * p.H + h) * (size_t)p.T + (size_t)t0;
  const E *gq = static_cast<const E *>(p.q);
  const E *gk = static_cast<const E *>(p.k);
  const E *gdo = static_cast<const E *>(p.v);
  const char *ws = p.ws + (size_t)h * p.nslot * TL::BYTES;
  const int dv = p.dv;
  // step i handles chunk nch - 1 - i
  auto chunk_of = [&](int i) { return min(max(nch - 1 - i, 0), nch - 1); };
  auto nrow_of = [&](int c) { return min(C, len - c * C); };
  auto tok0_of = [&](int c) { return row0 + (size_t)c * C; };
  const int iend = nch + (nch & 1);

  if (nch == 0) {
    // no tokens: the initial-state gradient is dL/dS_final
    if (p.sfin) {
      const size_t sbase = (size_t)nh * DK * (size_t)dv;
      for (int e = threadIdx.x; e < DK * DVT; e += Sh::NT) {
        const size_t off = sbase + (size_t)(e / DVT) * dv + (size_t)jt * DVT + (e % DVT);
        p.sfin[off] = p.s0 ? p.s0[off] : 0.f;
      }
    }
    return;
  }

  auto sK = [&](int i) { return reinterpret_cast<E *>(smem + Sh::OFF_K + (i & 1) * Sh::K_SLOT); };
  auto sQ = [&](int i) { return reinterpret_cast<E *>(smem + Sh::OFF_Q + (i & 1) * Sh::K_SLOT); };
  auto sV = [&](int i) { return reinterpret_cast<E *>(smem + Sh::OFF_V + (i & 1) * Sh::V_SLOT); };
  auto sTp = [&](int i) { return reinterpret_cast<E *>(smem + Sh::OFF_TP + (i & 1) * Sh::TP_SLOT); };
  auto sVec = [&](int i) {
    return reinterpret_cast<float *>(smem + Sh::OFF_TP + (i & 1) * Sh::TP_SLOT + TL::TP_IMG);
  };
  f32x4 *sYp = reinterpret_cast<f32x4 *>(smem + Sh::OFF_YP);

  constexpr bool W8 = Sh::W8;
  if (wave == CHAIN0 || wave == CHAIN1 || (W8 && wave >= LOADQ)) {
    auto chain = [&](auto ct0_c) {
      constexpr int CT0 = decltype(ct0_c)::value;
      constexpr int NCW = CT0 < NCT ? (NCT - CT0 < Sh::NCW ? NCT - CT0 : Sh::NCW) : 0;
      constexpr int NCW1 = NCW > 0 ? NCW : 1;
      f32x4 accS[NCW1][DK / 16];  // dS'
      const size_t sbase = (size_t)nh * DK * (size_t)dv;
#pragma unroll
      for (int ct = 0; ct < NCW; ++ct) {
        const int col = jt * DVT + 16 * (CT0 + ct) + li;
#pragma unroll
        for (int it = 0; it < DK / 16; ++it)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            accS[ct][it][j] = p.s0 ? p.s0[sbase + (size_t)(16 * it + 4 * lg + j) * dv + col] : 0.f;
      }
      Grp sb[NCW1][NQG];
      // dS' of chunk c as operand groups, also to the output
      auto publish = [&](int c) {
        const size_t slot = (size_t)h * p.nslot + slot0 + c;
#pragma unroll
        for (int ct = 0; ct < NCW; ++ct)
#pragma unroll
          for (int q = 0; q < NQG; ++q) {
            sb[ct][q] = O::b_from_d(&accS[ct][q * TPG]);
            const size_t grp = (slot * (size_t)(dv / 16) + (size_t)(jt * NCT + CT0 + ct)) * NQG + q;
            reinterpret_cast<Grp *>(p.states + grp * 64 * 16)[lane] = sb[ct][q];
          }
      };
      f32x4 x[NCW1][NB];
      __syncthreads();
      for (int i = -1; i <= iend; ++i) {
        const bool live = NCW > 0 && i >= 0 && i < nch;
        const int c = chunk_of(i);
        if (NCW > 0 && i == -1) publish(nch - 1);
        // ---- phase 1: K dS' and Gam_C dS' + Q^T Diag(Gam) dO ----
        if (live) {
          const E *K = sK(i);
          const E *Q = sQ(i);
          const E *V = sV(i);
          const float *vec = sVec(i);
#pragma unroll
          for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
            for (int ct = 0; ct < NCW; ++ct) x[ct][rt] = zero4();
#pragma unroll
            for (int q = 0; q < NQG; ++q) {
              const Grp a = O::a_row(K + (16 * rt + li) * LDK, q * KG, lg);
#pragma unroll
              for (int ct = 0; ct < NCW; ++ct) x[ct][rt] = O::mma_grp(a, sb[ct][q], x[ct][rt]);
            }
          }
          // Diag(Gam) dO as B groups
          Grp gob[NCW1][NCG];
#pragma unroll
          for (int ct = 0; ct < NCW; ++ct)
#pragma unroll
            for (int q = 0; q < NCG; ++q) {
              f32x4 t[TPG];
#pragma unroll
              for (int tt = 0; tt < TPG; ++tt) {
                const int r16 = 16 * (q * TPG + tt);
                t[tt] = *reinterpret_cast<const f32x4 *>(vec + C + r16 + 4 * lg) * O::col4(V, LDV, r16, 16 * (CT0 + ct), lane);
              }
              gob[ct][q] = O::b_from_d(t);
            }
          const float gC = vec[C + C - 1];
#pragma unroll
          for (int it = 0; it < DK / 16; ++it) {
#pragma unroll
            for (int ct = 0; ct < NCW; ++ct) accS[ct][it] = gC * accS[ct][it];
#pragma unroll
            for (int q = 0; q < NCG; ++q) {
              const Grp a = O::a_trans(Q, LDK, q * KG, 16 * it, lane);
#pragma unroll
              for (int ct = 0; ct < NCW; ++ct) accS[ct][it] = O::mma_grp(a, gob[ct][q], accS[ct][it]);
            }
          }
        }
        lds_barrier();
        // ---- phase 2: Y, dX = T'^T Y, and - K^T Diag(Gam) dX ----
        if (live) {
          const E *K = sK(i);
          const E *TpT = sTp(i);
          const float *vec = sVec(i);
          Grp yb[NCW1][NCG];
#pragma unroll
          for (int ct = 0; ct < NCW; ++ct) {
            f32x4 y[NB];
#pragma unroll
            for (int rt = 0; rt < NB; ++rt) {
              const f32x4 d4 = *reinterpret_cast<const f32x4 *>(vec + 2 * C + 16 * rt + 4 * lg);
              y[rt] = sYp[((CT0 + ct) * NB + rt) * 64 + lane] + d4 * x[ct][rt];
            }
#pragma unroll
            for (int q = 0; q < NCG; ++q) yb[ct][q] = O::b_from_d(&y[q * TPG]);
          }
          // dX: row block rt of T'^T is zero left of column block rt (T' lower triangular)
          Grp gxb[NCW1][NCG];
          f32x4 u[NCW1][NB];
#pragma unroll
          for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
            for (int ct = 0; ct < NCW; ++ct) u[ct][rt] = zero4();
#pragma unroll
            for (int q = rt / TPG; q < NCG; ++q) {
              const Grp a = O::a_row(TpT + (16 * rt + li) * LDC, q * KG, lg);
#pragma unroll
              for (int ct = 0; ct < NCW; ++ct) u[ct][rt] = O::mma_grp(a, yb[ct][q], u[ct][rt]);
            }
          }
#pragma unroll
          for (int ct = 0; ct < NCW; ++ct)
#pragma unroll
            for (int q = 0; q < NCG; ++q) {
              f32x4 t[TPG];
#pragma unroll
              for (int tt = 0; tt < TPG; ++tt) {
                const int r16 = 16 * (q * TPG + tt);
                t[tt] = -(*reinterpret_cast<const f32x4 *>(vec + C + r16 + 4 * lg)) * u[ct][q * TPG + tt];
              }
              gxb[ct][q] = O::b_from_d(t);
            }
#pragma unroll
          for (int it = 0; it < DK / 16; ++it)
#pragma unroll
            for (int q = 0; q < NCG; ++q) {
              const Grp a = O::a_trans(K, LDK, q * KG, 16 * it, lane);
#pragma unroll
              for (int ct = 0; ct < NCW; ++ct) accS[ct][it] = O::mma_grp(a, gxb[ct][q], accS[ct][it]);
            }
          if (c > 0) publish(c - 1);
        }
        lds_barrier();
      }
      if (p.sfin) {
#pragma unroll
        for (int ct = 0; ct < NCW; ++ct) {
          const int col = jt * DVT + 16 * (CT0 + ct) + li;
#pragma unroll
          for (int it = 0; it < DK / 16; ++it)
#pragma unroll
            for (int j = 0; j < 4; ++j) p.sfin[sbase + (size_t)(16 * it + 4 * lg + j) * dv + col] = accS[ct][it][j];
        }
      }
    };
    if constexpr (W8) {
      // column tiles 0, 1 on waves 0, 1 and 2, 3 on waves 6, 7 (two SIMDs each)
      if (wave == CHAIN0)
        chain(std::integral_constant<int, 0>{});
      else if (wave == CHAIN1)
        chain(std::integral_constant<int, 1>{});
      else if (wave == LOADQ)
        chain(std::integral_constant<int, 2>{});
      else
        chain(std::integral_constant<int, 3>{});
    } else {
      if (wave == CHAIN0)
        chain(std::integral_constant<int, 0>{});
      else
        chain(std::integral_constant<int, Sh::NCW>{});
    }
  } else if (wave == PW0 || wave == PW1) {
    // ---- P waves: P^T dO for the rows of Y whose column block they own ----
    auto pwave = [&](auto part_c) {
      constexpr int part = decltype(part_c)::value;
      using BL = OwnBlocks<NB, part>;
      constexpr int NOWN = BL::N;
      __syncthreads();
      for (int i = -1; i <= iend; ++i) {
        if (NOWN > 0 && i >= 0 && i < nch) {
          const E *Q = sQ(i);
          const E *K = sK(i);
          const E *V = sV(i);
          const float *vec = sVec(i);
          // dO of the slice as B groups (contraction over the chunk rows)
          Grp ob[NCT][NCG];
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int q = 0; q < NCG; ++q) {
              f32x4 t[TPG];
#pragma unroll
              for (int tt = 0; tt < TPG; ++tt) t[tt] = O::col4(V, LDV, 16 * (q * TPG + tt), 16 * ct, lane);
              ob[ct][q] = O::b_from_d(t);
            }
#pragma unroll
          for (int k = 0; k < NOWN; ++k) {
            const int st = BL::at(k);
            Grp kb[NQG];
#pragma unroll
            for (int q = 0; q < NQG; ++q) kb[q] = O::a_row(K + (16 * st + li) * LDK, q * KG, lg);
            const float gs = vec[16 * st + li];
            // P tiles (rt, st), rt >= st: D[r][s] = q_r . k_s exp(gamma_r - gamma_s), r >= s
            f32x4 pt[NB];
#pragma unroll
            for (int rt = 0; rt < NB; ++rt) {
              pt[rt] = zero4();
              if (rt < st) continue;
#pragma unroll
              for (int q = 0; q < NQG; ++q) pt[rt] = O::mma_grp(O::a_row(Q + (16 * rt + li) * LDK, q * KG, lg), kb[q], pt[rt]);
              const f32x4 gr = *reinterpret_cast<const f32x4 *>(vec + 16 * rt + 4 * lg);
#pragma unroll
              for (int j = 0; j < 4; ++j)
                pt[rt][j] = (rt > st || 4 * lg + j >= li) ? pt[rt][j] * __expf(gr[j] - gs) : 0.f;
            }
            // the D layout of P is the left-operand layout of P^T: rows s of Y
            Grp pa[NCG];
#pragma unroll
            for (int q = 0; q < NCG; ++q) pa[q] = O::b_from_d(&pt[q * TPG]);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
              f32x4 y = zero4();
#pragma unroll
              for (int q = st / TPG; q < NCG; ++q) y = O::mma_grp(pa[q], ob[ct][q], y);
              sYp[(ct * NB + st) * 64 + lane] = y;
            }
          }
        }
        lds_barrier();
        lds_barrier();
      }
    };
    if (wave == PW0)
      pwave(std::integral_constant<int, 0>{});
    else
      pwave(std::integral_constant<int, 1>{});
  } else if (W8 && wave == LOADK) {
    // ---- K and Q rows of the next step's chunk (one register set each, one step ahead) ----
    RowLoad<E, DK, AllBlocks<NB>> kin, qin;
    kin.issue(gk + tok0_of(chunk_of(0)) * DK, nrow_of(chunk_of(0)), lane);
    qin.issue(gq + tok0_of(chunk_of(0)) * DK, nrow_of(chunk_of(0)), lane);
    __syncthreads();
    for (int i = -1; i <= iend; ++i) {
      kin.put(sK(i + 1), LDK, lane, [](int, int row) { return row; });
      qin.put(sQ(i + 1), LDK, lane, [](int, int row) { return row; });
      kin.issue(gk + tok0_of(chunk_of(i + 2)) * DK, nrow_of(chunk_of(i + 2)), lane);
      qin.issue(gq + tok0_of(chunk_of(i + 2)) * DK, nrow_of(chunk_of(i + 2)), lane);
      lds_barrier();
      lds_barrier();
    }
  } else if (wave == LOADK) {
    // ---- K rows of the next step's chunk (two register sets, two steps ahead) ----
    RowLoad<E, DK, AllBlocks<NB>> kin[2];
    kin[0].issue(gk + tok0_of(chunk_of(0)) * DK, nrow_of(chunk_of(0)), lane);
    kin[1].issue(gk + tok0_of(chunk_of(1)) * DK, nrow_of(chunk_of(1)), lane);
    __syncthreads();
    auto step = [&](int i, auto set_c) {
      constexpr int S = decltype(set_c)::value;
      kin[S].put(sK(i + 1), LDK, lane, [](int, int row) { return row; });
      kin[S].issue(gk + tok0_of(chunk_of(i + 3)) * DK, nrow_of(chunk_of(i + 3)), lane);
      lds_barrier();
      lds_barrier();
    };
    for (int i = -1; i <= iend; i += 2) {
      step(i, std::integral_constant<int, 0>{});
      step(i + 1, std::integral_constant<int, 1>{});
    }
  } else if (wave == LOADQ) {
    RowLoad<E, DK, AllBlocks<NB>> qin[2];
    qin[0].issue(gq + tok0_of(chunk_of(0)) * DK, nrow_of(chunk_of(0)), lane);
    qin[1].issue(gq + tok0_of(chunk_of(1)) * DK, nrow_of(chunk_of(1)), lane);
    __syncthreads();
    auto step = [&](int i, auto set_c) {
      constexpr int S = decltype(set_c)::value;
      qin[S].put(sQ(i + 1), LDK, lane, [](int, int row) { return row; });
      qin[S].issue(gq + tok0_of(chunk_of(i + 3)) * DK, nrow_of(chunk_of(i + 3)), lane);
      lds_barrier();
      lds_barrier();
    };
    for (int i = -1; i <= iend; i += 2) {
      step(i, std::integral_constant<int, 0>{});
      step(i + 1, std::integral_constant<int, 1>{});
    }
  } else {
    // ---- T'^T, gamma/Gam/d and the dO slice of the next step's chunk ----
    using TC = ImgCopy<E, C>;
    constexpr int NSET = TC::NPL <= 20 ? 2 : 1;
    TC tin[NSET];
    VSliceLoad<E, C, DVT> vin[NSET];
    auto fetch = [&](int i, auto set_c) {
      constexpr int S = decltype(set_c)::value;
      const int c = chunk_of(i);
      tin[S].issue(ws + (size_t)(slot0 + c) * TL::BYTES, lane);
      vin[S].issue(gdo + tok0_of(c) * dv, nrow_of(c), dv, jt * DVT, lane);
    };
    fetch(0, std::integral_constant<int, 0>{});
    if constexpr (NSET == 2) fetch(1, std::integral_constant<int, NSET - 1>{});
    __syncthreads();
    auto step = [&](int i, auto set_c) {
      constexpr int S = decltype(set_c)::value;
      tin[S].put(sTp(i + 1), lane);
      vin[S].put(sV(i + 1), LDV, lane);
      fetch(i + 1 + NSET, set_c);
      lds_barrier();
      lds_barrier();
    };
    for (int i = -1; i <= iend; i += 2) {
      step(i, std::integral_constant<int, 0>{});
      step(i + 1, std::integral_constant<int, NSET - 1>{});
    }
  }
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------
// Packed sequences, longest first: order[rank] = n, rank = the number of
// sequences longer than n (ties by index).  O(N) per thread, so only run for
// N <= kMaxOrdered; beyond that the scan takes sequences in index order.
constexpr int kMaxOrdered = 2048;

__global__ __launch_bounds__(256) void kla_seq_order_kernel(const int32_t *cu, int nseq, int T, int *order) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= nseq) return;
  auto len = [&](int n) {
    const int a = min(max(cu[n], 0), T);
    return min(max(cu[n + 1], a), T) - a;
  };
  const int lt = len(t);
  int rank = 0;
  for (int m = 0; m < nseq; ++m) {
    const int lm = len(m);
    rank += (lm > lt || (lm == lt && m < t)) ? 1 : 0;
  }
  order[rank] = t;
}

template <typename E, int C>
static size_t order_offset_t(const ChunkArgs &a) {
  const size_t img = (size_t)a.H * slots_per_head(a.cu_seqlens != nullptr, a.B, a.T, a.num_seqs, C) *
                     TpLayout<E, C>::BYTES;
  return (img + 255) / 256 * 256;
}

template <typename E, int C>
static size_t workspace_bytes_t(const ChunkArgs &a) {
  // per-chunk images, then (packed sequences) the longest-first order
  return order_offset_t<E, C>(a) + (a.cu_seqlens ? ((size_t)a.num_seqs * 4 + 255) / 256 * 256 : 0);
}

size_t chunk_workspace_bytes(const ChunkArgs &a) {
  // the general kernel (shapes outside the pipelined ones) needs no workspace
  if (!fast_chunk_supported(a.dtype, a.dk, a.dv, a.chunk)) return 0;
  if (a.dtype == 0) return workspace_bytes_t<bf16, 64>(a);
  return a.chunk == 16 ? workspace_bytes_t<float, 16>(a) : workspace_bytes_t<float, 64>(a);
}

struct PgArgs {
  char *w;
  float *acc;
  float band_c;
  const float *acc0;
  float *accfin;
};

// The segment-parallel scan's buffers (ChunkParams::seg_first and after).
struct SegArgs {
  const int *seg_first;
  int seg_chunks;
  long long nseg;
  void *eout;
  float *seg_d, *seg_m;
};

template <typename E, int C, int DK, int NCT, bool PG = false>
static hipError_t launch_chunk_t(const ChunkArgs &a, hipStream_t st, char *states = nullptr,
                                  char *timg = nullptr, const PgArgs *pg = nullptr,
                                  hipEvent_t after_prep = nullptr, const SegArgs *seg = nullptr) {
  using Sh = ChunkShape<E, C, DK, NCT, PG>;
  static_assert(DK % Sh::DVT == 0, "identity tiles cover dk");
  ChunkParams p;
  p.seg_first = nullptr;
  p.seg_chunks = 0;
  p.eout = nullptr;
  p.seg_d = p.seg_m = nullptr;
  p.states = states;
  p.timg = timg;
  p.pg_w = pg ? pg->w : nullptr;
  p.pg_acc = pg ? pg->acc : nullptr;
  p.band_c = pg ? pg->band_c : 0.f;
  p.pg_acc0 = pg ? pg->acc0 : nullptr;
  p.pg_accfin = pg ? pg->accfin : nullptr;
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
  p.ws = static_cast<char *>(a.workspace);
  p.H = a.H;
  p.T = a.T;
  p.dv = a.dv;
  p.n_tiles = a.dv / Sh::DVT;
  p.n_vtiles = p.n_tiles;
  p.nseq = a.num_seqs;
  p.beta_direct = a.beta_direct;
  p.nslot = slots_per_head(a.cu_seqlens != nullptr, a.B, a.T, a.num_seqs, C);
  p.ngroups = a.num_seqs * a.H;
  p.order = nullptr;
  if (p.ngroups == 0) return hipSuccess;
  if (!seg && a.cu_seqlens && a.num_seqs > 1 && a.num_seqs <= kMaxOrdered && (long long)a.B * a.T > 0) {
    int *order = reinterpret_cast<int *>(static_cast<char *>(a.workspace) + order_offset_t<E, C>(a));
    hipLaunchKernelGGL(kla_seq_order_kernel, dim3((unsigned)((a.num_seqs + 255) / 256)), dim3(256), 0, st,
                       a.cu_seqlens, a.num_seqs, a.T, order);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    p.order = order;
  }
  if constexpr (PG) {
    // the key accumulator at every chunk's start (also with no tokens: final = initial)
    if ((long long)a.B * a.T > 0 && p.nslot > 0) {
      hipLaunchKernelGGL((kla_pgdn_chunk_sum_kernel<DK>), dim3((unsigned)p.nslot, (unsigned)a.H), dim3(128), 0, st, p);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((kla_pgdn_acc_scan_kernel<DK>), dim3((unsigned)p.ngroups), dim3(DK), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if ((long long)a.B * a.T > 0 && p.nslot > 0) {
      hipLaunchKernelGGL((kla_pgdn_wkeys_kernel<DK>), dim3((unsigned)p.nslot, (unsigned)a.H), dim3(256), 0, st, p);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if ((long long)a.B * a.T > 0 && p.nslot > 0) {
    if constexpr (std::is_same<E, bf16>::value && C == 64) {
      // bf16: one wave per run of consecutive slots of one head, each run
      // prefetching its next slot while it computes the current one.  Runs of
      // one slot up to about sixteen rounds of the eight one-wave workgroups a
      // CU holds (16,384 chunk-heads: 90 us against 98-107 us for runs of 2-16);
      // longer runs beyond that, where the prefetch overlaps every round (75,008
      // chunk-heads: 362-371 us for runs of 2-8, 431 us for runs of one).
      const long long total = (long long)p.nslot * a.H;
      const long long units = total / (2 * 8 * 256);
      p.pslots = units <= 8 ? 1 : (int)std::min<long long>(8, units / 2);
      const unsigned runs = (unsigned)((p.nslot + p.pslots - 1) / p.pslots);
      if (p.pg_w)
        hipLaunchKernelGGL((kla_chunk_prep_wave_kernel<DK, false, true>), dim3(runs, (unsigned)a.H), dim3(64), 0, st, p);
      else if (timg)
        hipLaunchKernelGGL((kla_chunk_prep_wave_kernel<DK, true, false>), dim3(runs, (unsigned)a.H), dim3(64), 0, st, p);
      else
        hipLaunchKernelGGL((kla_chunk_prep_wave_kernel<DK, false, false>), dim3(runs, (unsigned)a.H), dim3(64), 0, st, p);
    } else {
      // slots per workgroup: the longest run that still gives two workgroups
      // per CU (the pipeline is latency-bound; two resident workgroups overlap)
      const long long work = (long long)p.nslot * a.H;
      p.pslots = (int)std::min<long long>(kPrepSlots, std::max<long long>(2, work / 512));
      const unsigned runs = (unsigned)((p.nslot + p.pslots - 1) / p.pslots);
      hipLaunchKernelGGL((kla_chunk_prep_kernel<E, C, DK>), dim3(runs, (unsigned)a.H),
                         dim3(PrepShape<E, C, DK>::NT), 0, st, p);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (after_prep) {  // the workspace (images, order) is complete once this event has fired
    const hipError_t e = hipEventRecord(after_prep, st);
    if (e != hipSuccess) return e;
  }
  if (seg) {
    // groups are (segment, head); later segments add the identity tiles
    p.seg_first = seg->seg_first;
    p.seg_chunks = seg->seg_chunks;
    p.eout = seg->eout;
    p.seg_d = seg->seg_d;
    p.seg_m = seg->seg_m;
    p.n_tiles = p.n_vtiles + DK / Sh::DVT;
    p.ngroups = (int)(seg->nseg * a.H);
  }
  const long long nblk = ((long long)p.ngroups + 7) / 8 * 8 * p.n_tiles;
  hipLaunchKernelGGL((kla_chunk_kernel<E, C, DK, NCT, PG>), dim3((unsigned)nblk), dim3(Sh::NT), 0, st, p);
  return hipGetLastError();
}

bool chunk_supported(int dtype, int dk, int dv, int chunk) {
  return fast_chunk_supported(dtype, dk, dv, chunk) || general_supported(dtype, dk, dv, chunk);
}

// The shapes the pipelined prep + scan kernels are compiled for.
bool fast_chunk_supported(int dtype, int dk, int dv, int chunk) {
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
// redundant S-independent work per column).  The forward scan takes 32 columns
// down to half a workgroup per CU: with 16-column slices every step reloads K, Q
// and T' per 16 columns, and for few long sequences that L2 traffic costs more than
// the idle CUs (T=65536 H=16 dv=256: 1.20 ms with 128 two-tile workgroups against
// 1.34 ms with 256 one-tile ones).
static bool use_two_column_tiles(const ChunkArgs &a, bool fwd = false) {
  return a.dv % 32 == 0 && (long long)a.num_seqs * a.H * (a.dv / 32) >= (fwd ? 128 : 256);
}
// 64 columns (four tiles) when that still leaves at least eight workgroups per CU
// (throughput-bound grids: a step costs about 1.5x the two-tile step for twice
// the columns, 1.94 -> 1.50 ms on 32 packed sequences x 32 heads)
static bool use_four_column_tiles(const ChunkArgs &a) {
  return a.dv % 64 == 0 && (long long)a.num_seqs * a.H * (a.dv / 64) >= 8 * 256;
}

static hipError_t launch_fast(const ChunkArgs &a, hipStream_t st, char *states, char *timg = nullptr,
                              bool four = false, hipEvent_t after_prep = nullptr) {
  if (a.dtype == 0) {
    if ((four || !states) && a.dv % 64 == 0 && (four || use_four_column_tiles(a))) {
      if (a.dk == 128) return launch_chunk_t<bf16, 64, 128, 4>(a, st, states, timg, nullptr, after_prep);
      if (a.dk == 64) return launch_chunk_t<bf16, 64, 64, 4>(a, st, states, timg, nullptr, after_prep);
    }
    const bool two = use_two_column_tiles(a, states == nullptr);
    if (a.dk == 128)
      return two ? launch_chunk_t<bf16, 64, 128, 2>(a, st, states, timg, nullptr, after_prep)
                 : launch_chunk_t<bf16, 64, 128, 1>(a, st, states, timg, nullptr, after_prep);
    if (a.dk == 64)
      return two ? launch_chunk_t<bf16, 64, 64, 2>(a, st, states, timg, nullptr, after_prep)
                 : launch_chunk_t<bf16, 64, 64, 1>(a, st, states, timg, nullptr, after_prep);
    return hipErrorInvalidValue;
  }
  if (timg || four || after_prep) return hipErrorInvalidValue;  // bf16 paths only
  if (a.chunk == 16) {
    switch (a.dk) {
      case 16: return launch_chunk_t<float, 16, 16, 1>(a, st, states);
      case 32: return launch_chunk_t<float, 16, 32, 1>(a, st, states);
      case 64: return launch_chunk_t<float, 16, 64, 1>(a, st, states);
      case 128: return launch_chunk_t<float, 16, 128, 1>(a, st, states);
    }
  } else if (a.chunk == 64) {
    switch (a.dk) {
      case 16: return launch_chunk_t<float, 64, 16, 1>(a, st, states);
      case 32: return launch_chunk_t<float, 64, 32, 1>(a, st, states);
    }
  }
  return hipErrorInvalidValue;
}

// PGDN on the pipelined kernels: bf16, chunk 64, dk 64 or 128.
bool pgdn_fast_supported(int dtype, int dk, int dv, int chunk) {
  return dtype == 0 && chunk == 64 && (dk == 64 || dk == 128) && dv % 16 == 0 && dv >= 16 && dv <= 256;
}

// The forward workspace, then the chunk-start key accumulators (dk fp32 per (head,
// slot)), then the write keys (C x dk bf16 per (head, slot)).
static size_t pgdn_acc_offset(const ChunkArgs &a) { return (chunk_workspace_bytes(a) + 255) / 256 * 256; }
static size_t pgdn_w_offset(const ChunkArgs &a) {
  const int ns = slots_per_head(a.cu_seqlens != nullptr, a.B, a.T, a.num_seqs, 64);
  return pgdn_acc_offset(a) + ((size_t)a.H * ns * a.dk * 4 + 255) / 256 * 256;
}
size_t pgdn_workspace_bytes(const ChunkArgs &a) {
  if (!pgdn_fast_supported(a.dtype, a.dk, a.dv, a.chunk)) return 0;
  const int ns = slots_per_head(a.cu_seqlens != nullptr, a.B, a.T, a.num_seqs, 64);
  return pgdn_w_offset(a) + (size_t)a.H * ns * 64 * a.dk * 2;
}

hipError_t launch_pgdn_fast(const ChunkArgs &a, const GenExtra &x, hipStream_t st) {
  if (!pgdn_fast_supported(a.dtype, a.dk, a.dv, a.chunk)) return hipErrorInvalidValue;
  char *ws = static_cast<char *>(a.workspace);
  const PgArgs pg{ws + pgdn_w_offset(a), reinterpret_cast<float *>(ws + pgdn_acc_offset(a)), x.band_c,
                  x.initial_acc, x.final_acc};
  const bool two = use_two_column_tiles(a, true);
  if (a.dk == 128)
    return two ? launch_chunk_t<bf16, 64, 128, 2, true>(a, st, nullptr, nullptr, &pg)
               : launch_chunk_t<bf16, 64, 128, 1, true>(a, st, nullptr, nullptr, &pg);
  return two ? launch_chunk_t<bf16, 64, 64, 2, true>(a, st, nullptr, nullptr, &pg)
             : launch_chunk_t<bf16, 64, 64, 1, true>(a, st, nullptr, nullptr, &pg);
}

hipError_t launch_chunk_fwd(const ChunkArgs &a, hipStream_t st) {
  if (!fast_chunk_supported(a.dtype, a.dk, a.dv, a.chunk)) {
    const GenExtra none{0, 0.f, nullptr, nullptr};
    return launch_chunk_general(a, none, st);
  }
  return launch_fast(a, st, nullptr);
}

// ---------------------------------------------------------------------------
// the segment-parallel forward (kla_seg.hip has the bookkeeping kernels)
// ---------------------------------------------------------------------------
// Workgroups the library's own choice of segments aims at: one per CU of an MI355X.
constexpr int kSegTargetGroups = 256;

static int seq_chunks_host(const ChunkArgs &a, const int32_t *cu_host, int n) {
  const long long len = a.cu_seqlens ? (long long)cu_host[n + 1] - cu_host[n] : a.T;
  return (int)((len + a.chunk - 1) / a.chunk);
}

long long chunk_seg_count(const ChunkArgs &a, const int32_t *cu_host, int L) {
  auto segs = [&](long long nch) { return std::max(1LL, (nch + L - 1) / L); };
  if (!a.cu_seqlens) return (long long)a.num_seqs * segs(((long long)a.T + a.chunk - 1) / a.chunk);
  long long total = 0;
  for (int n = 0; n < a.num_seqs; ++n) total += segs(seq_chunks_host(a, cu_host, n));
  return total;
}

bool chunk_seg_supported(int dtype, int dk, int dv, int chunk) { return fast_chunk_supported(dtype, dk, dv, chunk); }

namespace {
struct SegLayout {
  long long nseg;
  size_t first, e, d, m, fix, end;
};
size_t up256(size_t x) { return (x + 255) / 256 * 256; }
SegLayout seg_layout(const ChunkArgs &a, const int32_t *cu_host, int L) {
  SegLayout l;
  const size_t esz = a.dtype == 0 ? 2 : 4;
  l.nseg = chunk_seg_count(a, cu_host, L);
  const size_t nsh = (size_t)l.nseg * a.H;
  l.first = up256(chunk_workspace_bytes(a));
  l.e = l.first + up256(((size_t)a.num_seqs + 1) * 4);
  l.d = l.e + up256((size_t)a.B * a.H * a.T * a.dk * esz);
  l.m = l.d + up256(nsh * a.dk * a.dv * 4);
  l.fix = l.m + up256(nsh * a.dk * a.dk * 4);
  l.end = l.fix + up256(nsh * a.dk * a.dv * 4);
  return l;
}
}  // namespace

size_t chunk_seg_workspace_bytes(const ChunkArgs &a, const int32_t *cu_host, int L) {
  return L > 0 ? seg_layout(a, cu_host, L).end : chunk_workspace_bytes(a);
}

// The library's choice: segments only where the plain scan leaves CUs idle (fewer
// than one two-tile workgroup per CU) on long sequences, bf16 with 64-column tiles.
// The smallest segment length whose grid (v's tiles for every segment, the identity
// tiles for the later ones) still fits one round of workgroups, if that cuts the
// longest sequence into at least three segments (a 64-column step costs about 1.75
// two-column-tile steps, and the correction pass costs about a tenth of the scan).
int chunk_auto_seg_chunks(const ChunkArgs &a, const int32_t *cu_host) {
  if (a.dtype != 0 || a.chunk != 64 || (a.dk != 64 && a.dk != 128) || a.dv % 64 != 0) return 0;
  if (a.num_seqs <= 0 || (a.cu_seqlens && !cu_host)) return 0;
  if ((long long)a.num_seqs * a.H * (a.dv / 32) >= kSegTargetGroups) return 0;
  int nch_max = 0;
  for (int n = 0; n < (a.cu_seqlens ? a.num_seqs : 1); ++n) nch_max = std::max(nch_max, seq_chunks_host(a, cu_host, n));
  if (nch_max < 96) return 0;
  for (int G = 8; G >= 3; --G) {
    const int L = (nch_max + G - 1) / G;
    long long groups = 0;
    for (int n = 0; n < a.num_seqs; ++n) {
      const long long nch = a.cu_seqlens ? seq_chunks_host(a, cu_host, n) : nch_max;
      const long long S = std::max(1LL, (nch + L - 1) / L);
      groups += (long long)a.H * (S * (a.dv / 64) + (S - 1) * (a.dk / 64));
    }
    if (groups <= kSegTargetGroups) return L;
  }
  return 0;
}

template <typename E, int C, int DK>
static hipError_t seg_scan_t(const ChunkArgs &a, const SegArgs &sa, hipStream_t st) {
  if constexpr (std::is_same<E, bf16>::value) {
    if (a.dv % 64 == 0) return launch_chunk_t<E, C, DK, 4>(a, st, nullptr, nullptr, nullptr, nullptr, &sa);
    if (a.dv % 32 == 0) return launch_chunk_t<E, C, DK, 2>(a, st, nullptr, nullptr, nullptr, nullptr, &sa);
  }
  return launch_chunk_t<E, C, DK, 1>(a, st, nullptr, nullptr, nullptr, nullptr, &sa);
}

hipError_t launch_chunk_fwd_seg(const ChunkArgs &a, const int32_t *cu_host, int L, hipStream_t st) {
  if (!chunk_seg_supported(a.dtype, a.dk, a.dv, a.chunk) || L <= 0) return hipErrorInvalidValue;
  const SegLayout lay = seg_layout(a, cu_host, L);
  char *ws = static_cast<char *>(a.workspace);
  int *seg_first = reinterpret_cast<int *>(ws + lay.first);
  SegFixParams f;
  f.cu = a.cu_seqlens;
  f.seg_first = seg_first;
  f.nseq = a.num_seqs;
  f.H = a.H;
  f.T = a.T;
  f.C = a.chunk;
  f.dk = a.dk;
  f.dv = a.dv;
  f.dtype = a.dtype;
  f.seg_chunks = L;
  f.seg_max_chunks = 0;
  for (int n = 0; n < (a.cu_seqlens ? a.num_seqs : 1); ++n)
    f.seg_max_chunks = std::max(f.seg_max_chunks, seq_chunks_host(a, cu_host, n));
  f.nseg = lay.nseg;
  f.seg_d = reinterpret_cast<float *>(ws + lay.d);
  f.seg_m = reinterpret_cast<float *>(ws + lay.m);
  f.sfin = a.final_state;
  f.sfix = ws + lay.fix;
  f.eout = ws + lay.e;
  f.o = a.o;
  if (a.num_seqs == 0) return hipSuccess;
  hipError_t e = launch_seg_table(f, seg_first, st);
  if (e != hipSuccess) return e;
  const SegArgs sa{seg_first, L, lay.nseg, ws + lay.e, reinterpret_cast<float *>(ws + lay.d),
                   reinterpret_cast<float *>(ws + lay.m)};
  ChunkArgs b = a;
  b.final_state = nullptr;  // the end states go to seg_d; the combine writes the final state
  if (a.dtype == 0) {
    e = a.dk == 128 ? seg_scan_t<bf16, 64, 128>(b, sa, st) : seg_scan_t<bf16, 64, 64>(b, sa, st);
  } else if (a.chunk == 16) {
    switch (a.dk) {
      case 16: e = seg_scan_t<float, 16, 16>(b, sa, st); break;
      case 32: e = seg_scan_t<float, 16, 32>(b, sa, st); break;
      case 64: e = seg_scan_t<float, 16, 64>(b, sa, st); break;
      default: e = seg_scan_t<float, 16, 128>(b, sa, st); break;
    }
  } else {
    e = a.dk == 16 ? seg_scan_t<float, 64, 16>(b, sa, st) : seg_scan_t<float, 64, 32>(b, sa, st);
  }
  if (e != hipSuccess) return e;
  return launch_seg_finish(f, st);
}

template <typename E, int C, int DK, int NCT>
static hipError_t launch_rev_t(const ChunkArgs &a, const float *dsfin, const void *dout, float *ds0, void *dstates,
                               hipStream_t st) {
  using Sh = RevShape<E, C, DK, NCT>;
  ChunkParams p{};
  p.q = a.q;
  p.k = a.k;
  p.v = dout;
  p.g = a.g;
  p.eta = a.eta;
  p.eps = a.eps;
  p.s0 = dsfin;
  p.o = nullptr;
  p.sfin = ds0;
  p.cu = a.cu_seqlens;
  p.ws = static_cast<char *>(a.workspace);
  p.H = a.H;
  p.T = a.T;
  p.dv = a.dv;
  p.n_tiles = a.dv / Sh::DVT;
  p.nseq = a.num_seqs;
  p.beta_direct = a.beta_direct;
  p.nslot = slots_per_head(a.cu_seqlens != nullptr, a.B, a.T, a.num_seqs, C);
  p.ngroups = a.num_seqs * a.H;
  p.states = static_cast<char *>(dstates);
  p.order = nullptr;
  if (p.ngroups == 0) return hipSuccess;
  // the packed-sequence order the states pass wrote into the same workspace
  if (a.cu_seqlens && a.num_seqs > 1 && a.num_seqs <= kMaxOrdered && (long long)a.B * a.T > 0)
    p.order = reinterpret_cast<const int *>(static_cast<char *>(a.workspace) + order_offset_t<E, C>(a));
  const long long nblk = ((long long)p.ngroups + 7) / 8 * 8 * p.n_tiles;
  hipLaunchKernelGGL((kla_chunk_rev_kernel<E, C, DK, NCT>), dim3((unsigned)nblk), dim3(Sh::NT), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_chunk_rev(const ChunkArgs &a, const float *dsfin, const void *dout, float *ds0, void *dstates,
                            hipStream_t st, bool four) {
  if (!fast_chunk_supported(a.dtype, a.dk, a.dv, a.chunk)) return hipErrorInvalidValue;
  if (a.dtype == 0) {
    if (four && a.dv % 64 == 0) {
      if (a.dk == 128) return launch_rev_t<bf16, 64, 128, 4>(a, dsfin, dout, ds0, dstates, st);
      if (a.dk == 64) return launch_rev_t<bf16, 64, 64, 4>(a, dsfin, dout, ds0, dstates, st);
    }
    const bool two = use_two_column_tiles(a);
    if (a.dk == 128)
      return two ? launch_rev_t<bf16, 64, 128, 2>(a, dsfin, dout, ds0, dstates, st)
                 : launch_rev_t<bf16, 64, 128, 1>(a, dsfin, dout, ds0, dstates, st);
    if (a.dk == 64)
      return two ? launch_rev_t<bf16, 64, 64, 2>(a, dsfin, dout, ds0, dstates, st)
                 : launch_rev_t<bf16, 64, 64, 1>(a, dsfin, dout, ds0, dstates, st);
    return hipErrorInvalidValue;
  }
  if (a.chunk == 16) {
    switch (a.dk) {
      case 16: return launch_rev_t<float, 16, 16, 1>(a, dsfin, dout, ds0, dstates, st);
      case 32: return launch_rev_t<float, 16, 32, 1>(a, dsfin, dout, ds0, dstates, st);
      case 64: return launch_rev_t<float, 16, 64, 1>(a, dsfin, dout, ds0, dstates, st);
      case 128: return launch_rev_t<float, 16, 128, 1>(a, dsfin, dout, ds0, dstates, st);
    }
  } else if (a.chunk == 64) {
    switch (a.dk) {
      case 16: return launch_rev_t<float, 64, 16, 1>(a, dsfin, dout, ds0, dstates, st);
      case 32: return launch_rev_t<float, 64, 32, 1>(a, dsfin, dout, ds0, dstates, st);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_states(const ChunkArgs &a, void *states, hipStream_t st, void *timg, bool four,
                               hipEvent_t after_prep) {
  if (!fast_chunk_supported(a.dtype, a.dk, a.dv, a.chunk)) return hipErrorInvalidValue;
  return launch_fast(a, st, static_cast<char *>(states), static_cast<char *>(timg), four, after_prep);
}

// The backward's two state passes (the chunk-start states and the adjoint scan) depend
// only on the prep's workspace, not on each other.  With 64-column slices both fit one
// round of workgroups side by side (one per CU each), which runs them concurrently at the
// higher per-CU throughput of the wider slices.
bool bwd_scans_concurrent(const ChunkArgs &a, int cus) {
  return a.dtype == 0 && a.chunk == 64 && (a.dk == 64 || a.dk == 128) && a.dv % 64 == 0 &&
         2LL * a.num_seqs * a.H * (a.dv / 64) <= cus;
}

// ---------------------------------------------------------------------------
// Fixed scratch for the allocation-free entry point (kla_chunk_fwd_noalloc)
// ---------------------------------------------------------------------------
// The prep -> scan hand-over above needs a device workspace.  Callers that
// cannot allocate get it from this file-scope buffer instead: one copy per GPU,
// created when the code object is loaded on that GPU and held until the
// process ends.  Its contents need no initialisation: every slot the scan
// reads is written by the prep kernel of the same call, and the sequence
// order by the ranking kernel.  Calls that overlap in time on one GPU share
// it and therefore race.
constexpr size_t kStaticScratchBytes = KLA_NOALLOC_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

size_t static_scratch_bytes() { return kStaticScratchBytes; }

hipError_t static_scratch(void **ptr) {
  // In host code `scratch` names a host-side stand-in, not the device copy:
  // the device address comes from hipGetSymbolAddress, looked up once per
  // device with that device current, and only that address is used.
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace kla
