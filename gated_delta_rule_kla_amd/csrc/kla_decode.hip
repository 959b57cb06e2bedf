// kla_decode.hip -- single-token KLA decode step for gfx950.
//
// One recurrent step per (sequence, head):
//   alpha = exp(g), beta = eta / (||k||^2 + eps)  (or beta = eta as given: the
//   gated delta rule, whose learned coefficient the Kaczmarz step replaces)
//   y_k = S^T k, y_q = S^T q           (one pass over the old state)
//   e   = v - alpha y_k
//   o   = alpha y_q + beta (k.q) e     (= S_new^T q without a second pass)
//   S   = alpha S + beta k e^T         (written back in place)
// This is the update of "Resumen Técnico: Atención Lineal Kaczmarz (KLA)"
// (gist.science/es/paper/2605.08587), §"La Regla de Actualización KLA",
// with the decayed state alpha S and the readout o = S_new^T q.
//
// The step is HBM-bound (0.75 flop per byte): the fp32 state is read once and
// written once with 16-byte accesses and held in VGPRs in between.  One
// workgroup owns one (sequence, head) state of DK x DV floats; each thread
// holds a float4 column slice of RPT rows.  Threads of one row group cover one
// full row, so each load/store instruction of a wave touches whole contiguous
// rows.  Partial dot products are reduced across row groups with lane
// shuffles inside a wave and through LDS across waves.
//
// With PG the same step is PGDN's ("Preconditioned DeltaNet", §2.C-2.D): the key
// accumulator A += k (.) k (fp32, [N, H, dk], updated in place), the write key
// w = p(A) (.) k, beta = eta (given) or eta / (k.w + eps), and
//   o = alpha y_q + beta (w.q) e,   S = alpha S + beta w e^T
// (the residual is still read with k).
#include "kla_common.h"
#include "kla_internal.h"

namespace kla {

constexpr int decode_threads(int dk, int dv) {
  return dk * dv / 32 < 64 ? 64 : (dk * dv / 32 > 1024 ? 1024 : dk * dv / 32);
}

template <int DK, int DV>
struct DecodeShape {
  static constexpr int TPR = DV / 4;                        // threads per row
  static constexpr int NT = decode_threads(DK, DV);         // ~32 state floats per thread
  static constexpr int RG = NT / TPR;                       // row groups
  static constexpr int RPT = DK / RG;                       // rows per thread
  static constexpr int NW = NT / 64;                        // waves
  static_assert(TPR <= 64 && RG * TPR == NT && RPT * RG == DK, "decode tiling");
};

template <typename E, int DK, int DV, bool PG = false>
__global__ __launch_bounds__(decode_threads(DK, DV)) void kla_decode_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const E *__restrict__ g, const E *__restrict__ eta, float eps, int beta_direct, float *__restrict__ state,
    E *__restrict__ o, float *__restrict__ acc = nullptr, float band_c = 0.f) {
  using Sh = DecodeShape<DK, DV>;
  constexpr int TPR = Sh::TPR, RG = Sh::RG, RPT = Sh::RPT, NW = Sh::NW;
  constexpr int NRED = 10;  // y_k[4], y_q[4], k.w, w.q  (w = k outside PGDN)

  __shared__ float s_k[DK];
  __shared__ float s_q[DK];
  __shared__ float s_w[PG ? DK : 1];
  __shared__ float s_m[NW];
  __shared__ float s_red[NW > 1 ? NW : 1][TPR][NRED];

  const size_t nh = blockIdx.x;
  const int t = threadIdx.x;
  const int cg = t % TPR;  // column group: columns 4cg .. 4cg+3
  const int rg = t / TPR;  // row group: rows rg + RG p

  for (int i = t; i < DK; i += Sh::NT) {
    s_k[i] = Elem<E>::to_f32(k[nh * DK + i]);
    s_q[i] = Elem<E>::to_f32(q[nh * DK + i]);
  }

  // PGDN: the accumulator and key loads go out before the state's, so that the
  // accumulator update, its mean and the write key are formed while the state is in
  // flight (a wait for a load also waits for every load issued before it)
  constexpr int NA = PG ? (DK + Sh::NT - 1) / Sh::NT : 1;
  float av[NA], kk[NA];
  if constexpr (PG) {
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int i = t + Sh::NT * j;
      kk[j] = i < DK ? Elem<E>::to_f32(k[nh * DK + i]) : 0.f;
      av[j] = i < DK ? acc[nh * DK + i] : 0.f;
    }
  }

  float *S = state + nh * (size_t)(DK * DV);
  f32x4 s[RPT];
#pragma unroll
  for (int p = 0; p < RPT; ++p)
    s[p] = *reinterpret_cast<const f32x4 *>(S + (size_t)(rg + RG * p) * DV + 4 * cg);

  float vv[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) vv[c] = Elem<E>::to_f32(v[nh * DV + 4 * cg + c]);
  const float alpha = __expf(Elem<E>::to_f32(g[nh]));
  const float et = Elem<E>::to_f32(eta[nh]);

  if constexpr (PG) {
    // the accumulator, its mean over the coordinates, and the write key
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      av[j] = fmaf(kk[j], kk[j], av[j]);  // zero past DK
      part += av[j];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
    if ((t & 63) == 0) s_m[t >> 6] = part;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += s_m[w];
    const float log_m = pgdn_log2_mean(tot * (1.f / DK));
    const PgdnK pk = pgdn_k(band_c);
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int i = t + Sh::NT * j;
      if (i < DK) {
        s_w[i] = pgdn_precond(av[j], log_m, pk) * kk[j];
        acc[nh * DK + i] = av[j];
      }
    }
  }
  __syncthreads();

  float red[NRED];
#pragma unroll
  for (int i = 0; i < NRED; ++i) red[i] = 0.f;
#pragma unroll
  for (int p = 0; p < RPT; ++p) {
    const float kr = s_k[rg + RG * p], qr = s_q[rg + RG * p];
    const float wr = PG ? s_w[rg + RG * p] : kr;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      red[c] = fmaf(s[p][c], kr, red[c]);
      red[4 + c] = fmaf(s[p][c], qr, red[4 + c]);
    }
    red[8] = fmaf(kr, wr, red[8]);
    red[9] = fmaf(wr, qr, red[9]);
  }
  // reduce over the row groups inside the wave (lanes TPR apart)
#pragma unroll
  for (int off = TPR; off < 64; off <<= 1) {
#pragma unroll
    for (int i = 0; i < NRED; ++i) red[i] += __shfl_xor(red[i], off);
  }
  if constexpr (NW > 1) {
    const int lane = t & 63, w = t >> 6;
    if (lane < TPR) {
#pragma unroll
      for (int i = 0; i < NRED; ++i) s_red[w][lane][i] = red[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NRED; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) acc += s_red[ww][cg][i];
      red[i] = acc;
    }
  }

  const float beta = beta_direct ? et : et / (red[8] + eps);
  const float bkq = beta * red[9];
  float e[4], oo[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    e[c] = vv[c] - alpha * red[c];
    oo[c] = alpha * red[4 + c] + bkq * e[c];
  }
#pragma unroll
  for (int p = 0; p < RPT; ++p) {
    const float bk = beta * (PG ? s_w[rg + RG * p] : s_k[rg + RG * p]);
    f32x4 n;
#pragma unroll
    for (int c = 0; c < 4; ++c) n[c] = fmaf(alpha, s[p][c], bk * e[c]);
    *reinterpret_cast<f32x4 *>(S + (size_t)(rg + RG * p) * DV + 4 * cg) = n;
  }
  if (rg == 0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) o[nh * DV + 4 * cg + c] = Elem<E>::from_f32(oo[c]);
  }
}

template <typename E, int DK, int DV>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t st, float *acc = nullptr,
                                  float band_c = 0.f) {
  const unsigned nblk = (unsigned)((size_t)a.N * a.H);
  if (acc)
    hipLaunchKernelGGL((kla_decode_kernel<E, DK, DV, true>), dim3(nblk), dim3(DecodeShape<DK, DV>::NT), 0,
                       st, (const E *)a.q, (const E *)a.k, (const E *)a.v, (const E *)a.g,
                       (const E *)a.eta, a.eps, a.beta_direct, a.state, (E *)a.o, acc, band_c);
  else
    hipLaunchKernelGGL((kla_decode_kernel<E, DK, DV, false>), dim3(nblk), dim3(DecodeShape<DK, DV>::NT), 0,
                       st, (const E *)a.q, (const E *)a.k, (const E *)a.v, (const E *)a.g,
                       (const E *)a.eta, a.eps, a.beta_direct, a.state, (E *)a.o, nullptr, 0.f);
  return hipGetLastError();
}

static int dim_index(int d) {
  switch (d) {
    case 16: return 0;
    case 32: return 1;
    case 64: return 2;
    case 128: return 3;
    case 256: return 4;
    default: return -1;
  }
}

bool decode_supported(int dtype, int dk, int dv) {
  return (dtype == 0 || dtype == 1) && dim_index(dk) >= 0 && dim_index(dv) >= 0;
}

template <typename E, int DK>
static hipError_t dispatch_dv(const DecodeArgs &a, hipStream_t st, float *acc, float band_c) {
  switch (a.dv) {
    case 16: return launch_decode_t<E, DK, 16>(a, st, acc, band_c);
    case 32: return launch_decode_t<E, DK, 32>(a, st, acc, band_c);
    case 64: return launch_decode_t<E, DK, 64>(a, st, acc, band_c);
    case 128: return launch_decode_t<E, DK, 128>(a, st, acc, band_c);
    case 256: return launch_decode_t<E, DK, 256>(a, st, acc, band_c);
  }
  return hipErrorInvalidValue;
}

template <typename E>
static hipError_t dispatch_dk(const DecodeArgs &a, hipStream_t st, float *acc, float band_c) {
  switch (a.dk) {
    case 16: return dispatch_dv<E, 16>(a, st, acc, band_c);
    case 32: return dispatch_dv<E, 32>(a, st, acc, band_c);
    case 64: return dispatch_dv<E, 64>(a, st, acc, band_c);
    case 128: return dispatch_dv<E, 128>(a, st, acc, band_c);
    case 256: return dispatch_dv<E, 256>(a, st, acc, band_c);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t st) {
  if (a.dtype == 0) return dispatch_dk<bf16>(a, st, nullptr, 0.f);
  return dispatch_dk<float>(a, st, nullptr, 0.f);
}

// PGDN's step on the same kernel (the shapes decode_supported lists)
hipError_t launch_decode_pgdn(const DecodeArgs &a, float band_c, float *acc, hipStream_t st) {
  if (!acc) return hipErrorInvalidValue;
  if (a.dtype == 0) return dispatch_dk<bf16>(a, st, acc, band_c);
  return dispatch_dk<float>(a, st, acc, band_c);
}

}  // namespace kla
