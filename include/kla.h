/*
 * kla.h -- C ABI of the MI355X (gfx950) Kaczmarz Linear Attention operator.
 *
 * The operator.  Per sequence and head, with q_t, k_t in R^dk, v_t in R^dv and
 * state S_t in R^{dk x dv}:
 *
 *     alpha_t = exp(g_t)                           (g = log-decay, g <= 0)
 *     beta_t  = eta_t / (||k_t||_2^2 + eps)         Kaczmarz step
 *     e_t     = v_t - (alpha_t S_{t-1})^T k_t       residual against the decayed state
 *     S_t     = alpha_t S_{t-1} + beta_t k_t e_t^T
 *     o_t     = S_t^T q_t
 *
 * Source: "Resumen Técnico: Atención Lineal Kaczmarz (KLA)",
 * gist.science/es/paper/2605.08587 -- §"Derivación Teórica" (the write is the
 * projection of the decayed state onto {S : S^T k_t = v_t}), §"La Regla de
 * Actualización KLA" (beta_t and the update), §"Implementación" (state shape
 * dk x dv; the gates and the chunkwise block solver of Gated DeltaNet are kept,
 * only B = Diag(beta) changes).  The decay form exp(g_t) and the readout
 * o_t = S_t^T q_t (post-update state, no 1/sqrt(dk) scale) are the plainest
 * reading of the pages, which only name "decay gates" and the recurrent state.
 *
 * Conventions common to every entry point
 *   - Every data pointer is DEVICE memory (allocated by the caller, e.g. with
 *     PyTorch) unless its comment says "host".  The library allocates no
 *     device memory and keeps no state between calls: scratch memory a call
 *     needs (kla_chunk_fwd's workspace) is passed in by the caller.
 *   - Tensors are dense and contiguous, row-major, in the layouts stated per
 *     argument.  All data pointers must be 16-byte aligned (cu_seqlens:
 *     4-byte).
 *   - q, k, v, g, eta and o share one element type (kla_dtype_t); states are
 *     always fp32.  Accumulation is fp32.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls only enqueue work and return; kernel faults surface at the
 *     caller's next synchronisation.  Calls on different streams are
 *     independent and thread-safe.
 *   - Errors: a negative kla_status_t.  All argument validation is done on
 *     the host BEFORE any HIP call, so it also runs on a machine without a
 *     GPU; a failing HIP launch returns KLA_ERR_HIP.  Nothing is printed and
 *     no exception crosses the ABI.  On error nothing has been enqueued.
 */
#ifndef KLA_H
#define KLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KLA_DT_BF16 = 0, /* bfloat16 inputs/outputs: the production path, bf16 MFMA   */
    KLA_DT_F32 = 1   /* fp32 inputs/outputs: the debug build, fp32 MFMA           */
} kla_dtype_t;

typedef enum {
    KLA_OK = 0,
    KLA_ERR_NULL = -1,        /* a required pointer is NULL                      */
    KLA_ERR_SHAPE = -2,       /* a size is negative/zero or inconsistent         */
    KLA_ERR_DTYPE = -3,       /* unknown kla_dtype_t                             */
    KLA_ERR_UNSUPPORTED = -4, /* valid but not compiled: see supported shapes    */
    KLA_ERR_SEQLENS = -5,     /* cu_seqlens not 0 = c0 <= c1 <= ... <= cN = T    */
    KLA_ERR_EPS = -6,         /* eps < 0, NaN or infinite                        */
    KLA_ERR_WORKSPACE = -7,   /* workspace NULL or below kla_chunk_workspace_bytes */
    KLA_ERR_ALIGN = -8,       /* a data pointer is not 16-byte aligned           */
    KLA_ERR_HIP = -9,         /* the HIP runtime rejected a launch               */
    KLA_ERR_SCRATCH = -10,    /* kla_chunk_fwd_noalloc: more scratch than its fixed buffer */
    KLA_ERR_PARAM = -11       /* PGDN: gain not a kla_gain_t, or band not finite and >= 1 */
} kla_status_t;

/* The update coefficient ("gain") of the preconditioned variant (kla_pgdn_*). */
typedef enum {
    KLA_GAIN_GIVEN = 0,    /* coef is beta_t itself (Gated DeltaNet's learned coefficient)  */
    KLA_GAIN_KACZMARZ = 1  /* coef is eta_t; beta_t = eta_t / (k_t . w_t + eps)             */
} kla_gain_t;

/*
 * kla_chunk_fwd -- chunkwise-parallel prefill (the block solver).
 *
 * Computes o_t for every token and the final state of every sequence, using
 * per chunk of `chunk` tokens: B = Diag(beta), the unit-lower-triangular solve
 * T = (I + strictly-lower(B K K^T, decay-weighted))^-1, T applied to the chunk,
 * a sequential scan of the state over chunks, and the causal intra-chunk
 * output (§"Implementación" above: the block solver with only B changed).
 * The result equals the token recurrence up to rounding and does not depend
 * on `chunk`.
 *
 *   q, k      [B, H, T, dk]  dtype
 *   v         [B, H, T, dv]  dtype
 *   g, eta    [B, H, T]      dtype; g is the log-decay (alpha = exp(g)),
 *                            eta the relaxation gate (used as given)
 *   eps       fp32 scalar >= 0 (finite)
 *   initial_state  [N, H, dk, dv] fp32 (dv contiguous), or NULL = zeros
 *   o         [B, H, T, dv]  dtype, written for every token
 *   final_state    [N, H, dk, dv] fp32, or NULL = not written.  May alias
 *                  initial_state (each tile is read before it is written);
 *                  no other aliasing is allowed.
 *   cu_seqlens     device int32 [N + 1] or NULL.  NULL: N = B and batch row b
 *                  is sequence b.  Otherwise B must be 1 and sequence n is
 *                  tokens [cu[n], cu[n+1]) of that row (packed varlen);
 *                  empty sequences are allowed (their final state = initial).
 *   cu_seqlens_host  host mirror of cu_seqlens (required iff cu_seqlens is
 *                  given): validated here.  The kernels also clamp every range
 *                  to [0, T], so a device array that disagrees with the mirror
 *                  cannot cause an out-of-bounds access.
 *   num_seqs  N (must equal B when cu_seqlens is NULL)
 *   workspace, workspace_bytes  device scratch of at least
 *                  kla_chunk_workspace_bytes(...) bytes for the same arguments
 *                  (16-byte aligned; may be NULL when that size is 0).  Owned
 *                  by the caller; its contents need no initialisation and are
 *                  meaningless after the call.  Calls that overlap in time
 *                  must not share a workspace.
 *
 * Two kernels run on `stream`: a prep kernel computes, for every (chunk,
 * head) in parallel, the S-independent part of the block solver (beta, the
 * decay weights, K K^T, T and T' = T Diag(beta)) into the workspace; the
 * scan kernel then walks each sequence's chunks with the state in registers,
 * and forms the decayed causal scores of Q K^T and the output.
 *
 * Supported: either dtype, chunk in {16, 64}, dk in {16, 32, 64, 128}, dv a
 * multiple of 16 in [16, 256].  Anything else returns KLA_ERR_UNSUPPORTED.
 * H is at most 65,536 (KLA_ERR_SHAPE above: heads index a launch grid's second
 * dimension); the same holds for every chunked entry point below.
 * The pipelined prep + scan kernels run BF16 with chunk 64 and dk in {64, 128},
 * and F32 with chunk 16 (any dk) or chunk 64 with dk in {16, 32}; the other
 * combinations run a general kernel (one workgroup per sequence, head and 16
 * state columns, fp32 end to end, no workspace: kla_chunk_workspace_bytes
 * returns 0 for them), which is correct for every shape but not tuned.
 */
kla_status_t kla_chunk_fwd(const void *q, const void *k, const void *v,
                           const void *g, const void *eta, float eps,
                           const float *initial_state, void *o, float *final_state,
                           const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                           int num_seqs, int B, int H, int T, int dk, int dv, int chunk,
                           kla_dtype_t dtype, void *workspace, size_t workspace_bytes,
                           void *stream);

/*
 * kla_chunk_fwd_noalloc -- kla_chunk_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments without the workspace, the same
 * kernels and results.  The workspace comes from a fixed buffer inside the
 * library, one per GPU, of KLA_NOALLOC_SCRATCH_BYTES (64 MiB), held from the
 * library's first use on that GPU until the process ends.  The call allocates nothing (no hipMalloc, no allocating library
 * routine); its first call on a device looks the buffer's address up once.
 *
 *   Returns KLA_ERR_SCRATCH, before any HIP call, when the call needs more
 *   than that buffer: kla_chunk_workspace_bytes(...) for the same arguments
 *   must not exceed it (B=4 H=16 T=4096 dk=dv=128 bf16 needs 28.3 MB).
 *   Every call on one GPU shares the buffer: calls that overlap in time on
 *   the same GPU (different streams, different host threads) race and give
 *   wrong results.  Other status codes as kla_chunk_fwd.
 */
kla_status_t kla_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                                   const void *g, const void *eta, float eps,
                                   const float *initial_state, void *o, float *final_state,
                                   const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                                   int num_seqs, int B, int H, int T, int dk, int dv, int chunk,
                                   kla_dtype_t dtype, void *stream);

/*
 * kla_chunk_fwd_workspace_bytes -- an upper bound on the device workspace
 * kla_chunk_fwd (and kla_gdn_chunk_fwd) needs for these sizes, valid for
 * either element type and for both the dense (num_seqs == B) and the packed
 * (cu_seqlens) layout, since neither is an argument here.  Host-only, no HIP
 * call.  Returns 0 for sizes kla_chunk_fwd would reject for both element
 * types, and when no workspace is needed (no tokens).  Callers that know the
 * dtype and cu_seqlens may use the exact kla_chunk_workspace_bytes below.
 * For packed sequences it covers the unsegmented need (and the segmented one of
 * a single long sequence): with less than a call's segmented need, kla_chunk_fwd
 * runs that call unsegmented (see kla_chunk_fwd_seg).
 */
size_t kla_chunk_fwd_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, int num_seqs);

/*
 * kla_chunk_workspace_bytes -- device workspace kla_chunk_fwd needs for these
 * arguments (the same meaning as there; host-only, no HIP call).  6,912
 * bytes per (64-token chunk, head) in bf16, plus the segments' buffers where
 * kla_chunk_fwd cuts sequences into segments (kla_chunk_fwd_seg below).
 * kla_gdn_chunk_fwd needs the same.  Returns 0 when no workspace is
 * needed (no tokens) and also for arguments kla_chunk_fwd would reject.
 */
size_t kla_chunk_workspace_bytes(const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                                 int num_seqs, int B, int H, int T, int dk, int dv, int chunk,
                                 kla_dtype_t dtype);

/*
 * kla_chunk_fwd_seg -- kla_chunk_fwd with the sequences cut into segments that
 * are scanned side by side (the segment-parallel scan), for grids where few long
 * sequences leave most CUs idle.
 *
 * The chunk update of the state is affine, S' = M_c S + D_c, and so is each chunk's
 * output in its start state (§"Implementación": the chunkwise block solver).
 * Every sequence is cut into segments of `seg_chunks` chunks (the last one may be
 * shorter; a sequence of at most seg_chunks chunks stays whole), and all segments
 * are scanned at once: a sequence's first segment from its initial state, every
 * later one from zero, together with dk extra state columns that start from the
 * identity with v = 0 -- their end state is the segment's transfer map M (the
 * product of its M_c) and their outputs E give how the segment's outputs depend on
 * its start state.  A combine kernel then chains the segments in order in fp32
 * (S_start of segment s+1 = M_s S_start(s) + D_s, the last one the final state)
 * and a correction kernel adds E S_start to every later segment's outputs.  The
 * result equals kla_chunk_fwd's up to rounding.
 *
 *   seg_chunks  0: one segment per sequence (exactly kla_chunk_fwd's kernels);
 *               n > 0: segments of n chunks; negative: KLA_ERR_SHAPE.
 *   workspace   at least kla_chunk_seg_workspace_bytes(..., seg_chunks) bytes:
 *               kla_chunk_fwd's, then per call (N + 1) ints of segment table,
 *               E ([B, H, T, dk] in dtype), and per (segment, head) dk x dv
 *               (end state) + dk x dk (transfer map) + dk x dv (start state)
 *               fp32.
 *   Other arguments, ownership and errors as kla_chunk_fwd.  seg_chunks > 0 on a
 *   combination outside the pipelined kernels' (BF16 chunk 64 dk 64/128, F32
 *   chunk 16 or chunk 64 with dk 16/32) returns KLA_ERR_UNSUPPORTED.
 *
 * kla_chunk_fwd (and kla_gdn_chunk_fwd) choose segments themselves -- BF16, chunk
 * 64, dk 64 or 128, dv a multiple of 64, fewer than 256 workgroups of 32 state
 * columns (N * H * dv / 32 < 256) and at least 96 chunks in the longest sequence:
 * the shortest segments whose scan grid still fits 256 workgroups, if that cuts
 * the longest sequence in three or more -- and only when the workspace they are
 * given holds the segments' buffers (kla_chunk_workspace_bytes includes them);
 * with a smaller workspace of at least the unsegmented size they run unsegmented.
 * kla_chunk_fwd_noalloc does the same against its fixed buffer.
 */
kla_status_t kla_chunk_fwd_seg(const void *q, const void *k, const void *v,
                               const void *g, const void *eta, float eps,
                               const float *initial_state, void *o, float *final_state,
                               const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                               int num_seqs, int B, int H, int T, int dk, int dv, int chunk,
                               kla_dtype_t dtype, int seg_chunks, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * kla_chunk_seg_workspace_bytes -- device workspace kla_chunk_fwd_seg needs for
 * these arguments (host-only, no HIP call); 0 for arguments it would reject.
 */
size_t kla_chunk_seg_workspace_bytes(const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                                     int num_seqs, int B, int H, int T, int dk, int dv, int chunk,
                                     kla_dtype_t dtype, int seg_chunks);

/*
 * kla_decode_step -- one recurrent step for N sequences x H heads.
 *
 * The token update of §"La Regla de Actualización KLA" applied once per
 * (sequence, head); the state is read once from HBM and written once, and
 * o = S_new^T q is formed from the same pass as alpha S_old^T q +
 * beta (k.q) e.
 *
 *   q, k    [N, H, dk]  dtype
 *   v       [N, H, dv]  dtype
 *   g, eta  [N, H]      dtype
 *   eps     fp32 scalar >= 0 (finite)
 *   state   [N, H, dk, dv] fp32, updated IN PLACE
 *   o       [N, H, dv]  dtype
 *
 * Supported: dk, dv in {16, 32, 64, 128, 256}, either dtype.
 */
kla_status_t kla_decode_step(const void *q, const void *k, const void *v,
                             const void *g, const void *eta, float eps,
                             float *state, void *o,
                             int N, int H, int dk, int dv,
                             kla_dtype_t dtype, void *stream);

/*
 * kla_gdn_chunk_fwd, kla_gdn_decode_step -- the same two operations for the
 * gated delta rule (Gated DeltaNet), the model KLA modifies: KLA keeps
 * GDN's state, gates, recurrence and block-parallel algorithm and only
 * replaces its learned scalar update coefficient with the Kaczmarz step
 * eta / (||k||^2 + eps) (§"Declaración del Problema", §"Metodología: Atención
 * Lineal Kaczmarz", §"Implementación").  Here that coefficient is given:
 *
 *   beta    [B, H, T] (chunk) or [N, H] (decode), dtype: the update
 *           coefficient beta_t itself, used as S = alpha S + beta_t k e^T
 *
 * in place of eta and eps; every other argument, layout, status code and
 * supported shape is that of kla_chunk_fwd / kla_decode_step (the same
 * kernels run; kla_chunk_workspace_bytes sizes the workspace).  With
 * beta_t = eta_t / (||k_t||^2 + eps) the results equal KLA's.
 */
kla_status_t kla_gdn_chunk_fwd(const void *q, const void *k, const void *v,
                               const void *g, const void *beta,
                               const float *initial_state, void *o, float *final_state,
                               const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                               int num_seqs, int B, int H, int T, int dk, int dv, int chunk,
                               kla_dtype_t dtype, void *workspace, size_t workspace_bytes,
                               void *stream);

kla_status_t kla_gdn_decode_step(const void *q, const void *k, const void *v,
                                 const void *g, const void *beta,
                                 float *state, void *o,
                                 int N, int H, int dk, int dv,
                                 kla_dtype_t dtype, void *stream);

/*
 * kla_chunk_bwd -- gradients of kla_chunk_fwd.
 *
 * KLA is trained with Gated DeltaNet's block-parallel algorithm, only the
 * diagonal coefficient matrix Diag(beta) of the block solver changing
 * (§"Implementación"); this is the reverse mode of that block solver.  For a
 * scalar loss L with upstream gradients dout = dL/do and dfinal_state =
 * dL/dS_final, it returns dL/dq, dL/dk (including the path through ||k||^2 in
 * beta), dL/dv, dL/dg, dL/deta and dL/dinitial_state.
 *
 *   q, k, v, g, eta, eps, initial_state, cu_seqlens, cu_seqlens_host,
 *   num_seqs, B, H, T, dk, dv, chunk, dtype: the forward call's arguments
 *   dout            [B, H, T, dv]   dtype
 *   dfinal_state    [N, H, dk, dv]  fp32, or NULL (zero)
 *   dq, dk_, dv_    shaped and typed as q, k, v (written)
 *   dg, deta        [B, H, T]       fp32 (written)
 *   dinitial_state  [N, H, dk, dv]  fp32 (written), or NULL (not computed)
 *   workspace       kla_chunk_bwd_workspace_bytes(...) bytes of device memory
 *                   (16-byte aligned), owned by the caller, no initialisation
 *                   needed; holds per (chunk, head) T = (I + A)^-1 (BF16: as
 *                   its packed transposed image; F32: with the causal scores,
 *                   the decayed Gram matrix and the coefficient and decay
 *                   vectors), the chunk-start state and the chunk-end state
 *                   gradient (in `dtype`), then the forward's own workspace.
 *
 * Every pointer is 16-byte aligned device memory; gradient buffers must not
 * alias the inputs.  Positions of the gradient tensors that belong to no
 * sequence are not written.  Status codes and validation as kla_chunk_fwd
 * (all checks on the host before any HIP call); the supported shapes are
 * those of kla_chunk_fwd's pipelined kernels (BF16: chunk 64, dk in {64, 128};
 * F32: chunk 16 with dk in {16, 32, 64, 128}, chunk 64 with dk in {16, 32};
 * dv a multiple of 16 in [16, 256]); others return KLA_ERR_UNSUPPORTED.
 * Kernels run on `stream`: the forward's prep and scan kernels storing the
 * chunk-start states (BF16: the prep also writes the T image), a reverse scan
 * of the state gradients, and a parallel per-(chunk, head) gradient kernel
 * (F32: after a per-(chunk, head) prep of its own).  BF16 calls whose two
 * scans fit side by side on the GPU (2 * num_seqs * H * dv / 64 workgroups at
 * most one per CU, dv a multiple of 64) run the reverse scan on a stream of
 * the library's own (one per device, created on first use, default priority,
 * kept until the process ends), ordered after the prep on `stream` and before
 * the gradient kernel by two events: all work still completes in `stream`'s
 * order, and the caller's stream semantics (and graph capture of `stream`)
 * are unchanged.  Enqueues from several host threads are serialised around
 * that fork and join.
 */
kla_status_t kla_chunk_bwd(const void *q, const void *k, const void *v,
                           const void *g, const void *eta, float eps,
                           const float *initial_state, const void *dout, const float *dfinal_state,
                           void *dq, void *dk_, void *dv_, float *dg, float *deta,
                           float *dinitial_state,
                           const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                           int num_seqs, int B, int H, int T, int dk, int dv, int chunk,
                           kla_dtype_t dtype, void *workspace, size_t workspace_bytes,
                           void *stream);

/*
 * kla_gdn_chunk_bwd -- gradients of kla_gdn_chunk_fwd: as kla_chunk_bwd with
 * beta [B, H, T] given in place of eta and eps; dbeta [B, H, T] fp32 is dL/dbeta.
 */
kla_status_t kla_gdn_chunk_bwd(const void *q, const void *k, const void *v,
                               const void *g, const void *beta,
                               const float *initial_state, const void *dout, const float *dfinal_state,
                               void *dq, void *dk_, void *dv_, float *dg, float *dbeta,
                               float *dinitial_state,
                               const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                               int num_seqs, int B, int H, int T, int dk, int dv, int chunk,
                               kla_dtype_t dtype, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * kla_chunk_bwd_workspace_bytes -- device workspace kla_chunk_bwd and
 * kla_gdn_chunk_bwd need (host-only): per (chunk, head) 6,144 bytes (BF16, the
 * packed T image) or 3 C^2 e + 16 C bytes (F32), plus 2 dk dv e bytes, e = 2
 * for bf16 and 4 for fp32 (rounded up per region), plus
 * kla_chunk_workspace_bytes(...) for the forward kernels that recompute the
 * chunk-start states.  0 when no workspace is needed or for arguments
 * kla_chunk_bwd would reject.
 */
size_t kla_chunk_bwd_workspace_bytes(const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                                     int num_seqs, int B, int H, int T, int dk, int dv, int chunk,
                                     kla_dtype_t dtype);

/*
 * kla_pgdn_chunk_fwd -- chunkwise prefill of the preconditioned gated delta
 * rule (PGDN), "Preconditioned DeltaNet" (gist.science/es/paper/2604.21100):
 * §2.C accumulates the keys' diagonal second moments A_t = A_{t-1} + k_t (.) k_t
 * and preconditions with P_t = Diag(A_t)^-1 squashed into [1/band, band];
 * §2.A applies it to the write key (w_t = p_t (.) k_t); §2.D gives the gated
 * variant and its block-parallel form.  Per token:
 *
 *     A_t  = A_{t-1} + k_t (.) k_t                     (no decay; includes token t)
 *     p_t  = exp(c tanh(r / c)),  r_i = ln((mean_j A_t,j + 1e-30) / (A_t,i + 1e-30)),
 *            c = ln(band)  (band = 1: p_t = 1, the gated delta rule / KLA)
 *     w_t  = p_t (.) k_t
 *     beta = coef_t (KLA_GAIN_GIVEN)  or  coef_t / (k_t . w_t + eps) (KLA_GAIN_KACZMARZ)
 *     e_t  = v_t - (alpha_t S_{t-1})^T k_t,  S_t = alpha_t S_{t-1} + beta w_t e_t^T,
 *     o_t  = S_t^T q_t,  alpha_t = exp(g_t)
 *
 * The page fixes the accumulator, the inverse, the band and the log-space
 * squash; the normalisation by the mean over coordinates, the tanh form and
 * the Kaczmarz gain are this library's reading of it.
 *
 *   q, k, v, g, cu_seqlens, cu_seqlens_host, num_seqs, B, H, T, dk, dv,
 *   chunk, dtype, initial_state, o, final_state: as kla_chunk_fwd
 *   coef          [B, H, T] dtype: beta_t (KLA_GAIN_GIVEN) or eta_t (KLA_GAIN_KACZMARZ)
 *   eps           >= 0, finite (used by KLA_GAIN_KACZMARZ only)
 *   band          the squash's bound x: finite, >= 1
 *   initial_acc   [N, H, dk] fp32 accumulator before the first token, or NULL (zeros)
 *   final_acc     [N, H, dk] fp32, or NULL (not written); may alias initial_acc
 *
 *   workspace     kla_pgdn_chunk_workspace_bytes(...) bytes of device memory
 *                 (16-byte aligned, no initialisation needed; NULL when that is 0)
 *
 * Supported: either dtype, chunk in {16, 64}, dk in {16, 32, 64, 128}, dv a
 * multiple of 16 in [16, 256].  BF16 with chunk 64 and dk in {64, 128} runs the
 * pipelined prep and scan kernels (after two small passes that form the key
 * accumulator at every chunk's start); the prep also forms the write keys into
 * the workspace.  Every other supported shape runs the general kernel and needs
 * no workspace.  KLA_ERR_PARAM for a bad gain or band; KLA_ERR_WORKSPACE for a
 * missing or short workspace; other status codes as kla_chunk_fwd.
 */
kla_status_t kla_pgdn_chunk_fwd(const void *q, const void *k, const void *v,
                                const void *g, const void *coef, float eps,
                                kla_gain_t gain, float band,
                                const float *initial_state, const float *initial_acc,
                                void *o, float *final_state, float *final_acc,
                                const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                                int num_seqs, int B, int H, int T, int dk, int dv, int chunk,
                                kla_dtype_t dtype, void *workspace, size_t workspace_bytes,
                                void *stream);

/*
 * kla_pgdn_chunk_workspace_bytes -- device workspace kla_pgdn_chunk_fwd needs
 * (host-only): kla_chunk_workspace_bytes(...) plus, per (chunk, head), dk fp32
 * (the key accumulator at the chunk's start) and chunk x dk bf16 (the write
 * keys), each region rounded up to 256 bytes.  0 for shapes that run the
 * general kernel, with no tokens, or for arguments kla_pgdn_chunk_fwd would
 * reject.
 */
size_t kla_pgdn_chunk_workspace_bytes(const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                                      int num_seqs, int B, int H, int T, int dk, int dv, int chunk,
                                      kla_dtype_t dtype);

/*
 * kla_pgdn_decode_step -- one PGDN token for N sequences x H heads (the
 * per-token rule above): q, k [N, H, dk], v [N, H, dv], g, coef [N, H] (dtype);
 * state [N, H, dk, dv] fp32 and acc [N, H, dk] fp32 updated IN PLACE;
 * o [N, H, dv] dtype.  Supported: dk in {16, 32, 64, 128}, dv in [1, 256],
 * either dtype.  Status codes as kla_pgdn_chunk_fwd.
 */
kla_status_t kla_pgdn_decode_step(const void *q, const void *k, const void *v,
                                  const void *g, const void *coef, float eps,
                                  kla_gain_t gain, float band, float *state, float *acc,
                                  void *o, int N, int H, int dk, int dv,
                                  kla_dtype_t dtype, void *stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *kla_status_str(kla_status_t s);

/* ABI version of this header (incremented on any incompatible change). */
int kla_abi_version(void);

#define KLA_ABI_VERSION 9

/* Size of kla_chunk_fwd_noalloc's fixed per-GPU scratch buffer, in bytes. */
#define KLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

#ifdef __cplusplus
}
#endif

#endif /* KLA_H */
