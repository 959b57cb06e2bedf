"""fp64 CPU oracle of the preconditioned gated delta rule (PGDN).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module; only the test-suite, the smoke check and the benchmark's CPU-baseline
leg do.  It shares no code with the HIP path.

Source: [PDN] "Preconditioned DeltaNet: Curvature-aware Sequence Modeling for
Linear Recurrences", technical summary at gist.science/es/paper/2604.21100:

  * §2.A: under an exact preconditioner (the inverse of the keys' Gram matrix)
    the recurrence recovers the least-squares solution; applied to the write
    key ("ATK", apply-to-key) for DeltaNet-type rules.
  * §2.C: the diagonal approximation.  Only the diagonal second moments of the
    keys are accumulated, A_t = A_{t-1} + k_t (.) k_t, and the preconditioner is
    P_t = Diag(A_t)^-1, squashed in log space into a bounded band [1/x, x]
    (x about 1.5) for numerical stability.
  * §2.D: the decayed variant PGDN (Decay, Gain, Preconditioner, Solve) with a
    chunkwise-parallel form.

Readings where the page is silent (each also listed in the design notes):

  * P1 the accumulator starts at A_0 (zero unless given), includes the current
    token, and does not decay (the page's formula has no gate in it);
  * P2 the preconditioner is taken relative to its own mean over the dk key
    coordinates: the unsquashed log value of coordinate i is
        r_i = log((mean_j A_t,j + delta) / (A_t,i + delta)),
    i.e. Diag(A_t)^-1 up to one positive scalar per token (without some such
    normalisation the running sum drives every entry to the band's lower edge
    within a few hundred tokens); delta = 1e-30 only guards 0/0;
  * P3 the squash is p_i = exp(c tanh(r_i / c)) with c = ln x: the identity
    near r = 0, odd in log space, saturating at [1/x, x]; x = 1 gives p = 1;
  * P4 ATK: the write key is w_t = p_t (.) k_t; the residual is still read with
    k_t (e_t = v_t - (alpha_t S_{t-1})^T k_t), the read-out with q_t;
  * P5 the gain ("G" of the taxonomy) is either the given beta_t (Gated
    DeltaNet's learned coefficient: PGDN proper), or the Kaczmarz step in the
    preconditioned metric, beta_t = eta_t / (k_t^T w_t + eps) (the KLA
    coefficient of "Resumen Técnico: Atención Lineal Kaczmarz (KLA)",
    §"La Regla de Actualización KLA", with the write key preconditioned).
    With the second gain, eta = 1 and eps = 0 the write again interpolates:
    S_t^T k_t = v_t, the change being least-norm in the P^-1-weighted norm.

The decay and the read-out follow the KLA oracle's readings: S~ = exp(g_t) S,
o_t = S_t^T q_t (post-update state).

Parity status: pinned by tests/test_oracle_pgdn.py (reduction to the gated
delta rule at x = 1 and for isotropic keys, closed-form accumulator and
preconditioner, band and symmetry of the squash, interpolation and weighted
least-norm change with the Kaczmarz gain, chunk form with distinct read and
write keys equal to the recurrence, planted mutants).  What P1-P3 choose is a
reading, not a value the page fixes: a different normalisation or squash
would give different numbers, and no pin can tell which the page's authors
used ("parity unpinned" for that choice itself).
"""

from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np
import scipy.linalg

__all__ = ["GAIN_GIVEN", "GAIN_KACZMARZ", "PGDN_DELTA", "pgdn_preconditioner", "pgdn_recurrence",
           "pgdn_forward", "pgdn_decode_step", "pgdn_chunkwise"]

GAIN_GIVEN = 0       # beta_t given (Gated DeltaNet's learned coefficient)
GAIN_KACZMARZ = 1    # beta_t = eta_t / (k_t^T w_t + eps)
PGDN_DELTA = float(np.float32(1e-30))


def _squash(A: np.ndarray, band: float) -> np.ndarray:
    """p = exp(c tanh(r / c)), r = log((mean A + delta) / (A + delta)), c = ln band
    (readings P2, P3); A [..., dk] >= 0."""
    if band == 1.0:
        return np.ones_like(A)
    c = np.log(band)
    r = np.log((A.mean(axis=-1, keepdims=True) + PGDN_DELTA) / (A + PGDN_DELTA))
    return np.exp(c * np.tanh(r / c))


def pgdn_preconditioner(k: np.ndarray, band: float, A0: Optional[np.ndarray] = None):
    """Per-token preconditioner of one sequence and head.

    k [L, dk]; A0 [dk] or None (zeros).  Returns (p [L, dk], A_L [dk]) where
    p_t is the squashed diagonal preconditioner for token t, formed from the
    accumulator A_t = A_{t-1} + k_t (.) k_t that includes token t ([PDN] §2.C)."""
    k = np.asarray(k, dtype=np.float64)
    L, dk = k.shape
    A = np.zeros(dk) if A0 is None else np.array(A0, dtype=np.float64, copy=True)
    p = np.empty((L, dk))
    for t in range(L):
        A = A + k[t] * k[t]
        p[t] = _squash(A, band)
    return p, A


def pgdn_recurrence(q, k, v, g, coef, eps, gain, band, S0=None, A0=None):
    """Token-by-token PGDN for ONE sequence and ONE head, fp64.

    q, k [L, dk]; v [L, dv]; g, coef [L] (coef = beta with GAIN_GIVEN, eta with
    GAIN_KACZMARZ); S0 [dk, dv] or None; A0 [dk] or None.  Each step:
        A   = A + k_t (.) k_t;   p = squash(A);   w = p (.) k_t
        beta = coef_t            (GAIN_GIVEN)   or   coef_t / (k_t . w + eps)
        S~  = exp(g_t) S;  e = v_t - S~^T k_t;  S = S~ + beta w e^T;  o_t = S^T q_t
    Returns (o [L, dv], S_L, A_L)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    coef = np.asarray(coef, dtype=np.float64)
    L, dk = k.shape
    S = np.zeros((dk, v.shape[1])) if S0 is None else np.array(S0, dtype=np.float64, copy=True)
    A = np.zeros(dk) if A0 is None else np.array(A0, dtype=np.float64, copy=True)
    o = np.empty((L, v.shape[1]))
    for t in range(L):
        kt = k[t]
        A = A + kt * kt
        w = _squash(A, band) * kt
        beta = coef[t] if gain == GAIN_GIVEN else coef[t] / (kt @ w + eps)
        S_dec = np.exp(g[t]) * S
        e = v[t] - S_dec.T @ kt
        S = S_dec + beta * np.outer(w, e)
        o[t] = S.T @ q[t]
    return o, S, A


def pgdn_forward(q, k, v, g, coef, eps, gain, band, initial_state=None, initial_acc=None,
                 cu_seqlens: Optional[Sequence[int]] = None, heads: Optional[Sequence[int]] = None):
    """PGDN over a batch in the [B, H, T, d] layout, fp64 (layouts and varlen as
    kla_forward).  initial_state [N, H, dk, dv], initial_acc [N, H, dk] (zeros
    when None).  Returns (o [B, H, T, dv], final states [N, H, dk, dv], final
    accumulators [N, H, dk])."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    g, coef = np.asarray(g, np.float64), np.asarray(coef, np.float64)
    B, H, T, dk = k.shape
    dv = v.shape[3]
    if cu_seqlens is None:
        segs = [(b, 0, T) for b in range(B)]
    else:
        cu = [int(c) for c in cu_seqlens]
        segs = [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    N = len(segs)
    o = np.full((B, H, T, dv), np.nan)
    S_fin = np.full((N, H, dk, dv), np.nan)
    A_fin = np.full((N, H, dk), np.nan)
    for n, (b, t0, t1) in enumerate(segs):
        for h in (range(H) if heads is None else heads):
            S0 = None if initial_state is None else initial_state[n, h]
            A0 = None if initial_acc is None else initial_acc[n, h]
            o[b, h, t0:t1], S_fin[n, h], A_fin[n, h] = pgdn_recurrence(
                q[b, h, t0:t1], k[b, h, t0:t1], v[b, h, t0:t1], g[b, h, t0:t1], coef[b, h, t0:t1], eps,
                gain, band, S0, A0)
    return o, S_fin, A_fin


def pgdn_decode_step(q, k, v, g, coef, eps, gain, band, state, acc):
    """One PGDN step for N sequences x H heads: q, k [N, H, dk]; v [N, H, dv];
    g, coef [N, H]; state [N, H, dk, dv]; acc [N, H, dk].  Returns (o [N, H, dv],
    new state, new accumulator)."""
    N, H, dk = np.asarray(k).shape
    o = np.empty((N, H, np.asarray(v).shape[2]))
    S_new = np.empty(np.asarray(state).shape)
    A_new = np.empty((N, H, dk))
    for n in range(N):
        for h in range(H):
            oo, S_new[n, h], A_new[n, h] = pgdn_recurrence(
                np.asarray(q)[n, h][None], np.asarray(k)[n, h][None], np.asarray(v)[n, h][None],
                np.asarray(g)[n, h][None], np.asarray(coef)[n, h][None], eps, gain, band,
                np.asarray(state)[n, h], np.asarray(acc)[n, h])
            o[n, h] = oo[0]
    return o, S_new, A_new


def pgdn_chunkwise(q, k, w, v, g, beta, S0, chunk: int):
    """The block-parallel form ([PDN] §2.D) for ONE sequence and head, fp64,
    with read keys k and write keys w given ([L, dk] each) and the coefficients
    beta [L] given.  Per chunk of C tokens with start state S (unrolling the
    update over the chunk; gamma = running sum of g, Gam = exp(gamma)):

        A  = strictly-lower(Diag(beta) K W^T), entry (r, s) weighted by exp(gamma_r - gamma_s)
        T  = (I + A)^-1
        Ut = T Diag(beta) (V - Diag(Gam) K S)          (row r = beta_r e_r)
        O  = Diag(Gam) Q S + (Q W^T masked r >= s, weighted exp(gamma_r - gamma_s)) Ut
        S  <- Gam_C S + W^T Diag(exp(gamma_C - gamma)) Ut

    The read key enters where the state is read (K S, the rows of A), the
    write key where the state is written (W^T Ut, the columns of A and of the
    scores).  Returns (o [L, dv], S_L)."""
    q, k, w, v = (np.asarray(a, dtype=np.float64) for a in (q, k, w, v))
    g, beta = np.asarray(g, np.float64), np.asarray(beta, np.float64)
    L, dk = k.shape
    S = np.zeros((dk, v.shape[1])) if S0 is None else np.array(S0, dtype=np.float64, copy=True)
    o = np.empty((L, v.shape[1]))
    for c0 in range(0, L, chunk):
        c1 = min(c0 + chunk, L)
        n = c1 - c0
        K, Wk, Q, V, b = k[c0:c1], w[c0:c1], q[c0:c1], v[c0:c1], beta[c0:c1]
        gamma = np.cumsum(g[c0:c1])
        low = np.tril(np.ones((n, n), dtype=bool))
        decay = np.where(low, np.exp(np.where(low, gamma[:, None] - gamma[None, :], 0.0)), 0.0)
        A = np.tril(b[:, None] * (K @ Wk.T) * decay, -1)
        T = scipy.linalg.solve_triangular(np.eye(n) + A, np.eye(n), lower=True, unit_diagonal=True)
        Ut = T @ (b[:, None] * (V - np.exp(gamma)[:, None] * (K @ S)))
        o[c0:c1] = np.exp(gamma)[:, None] * (Q @ S) + ((Q @ Wk.T) * decay) @ Ut
        S = np.exp(gamma[-1]) * S + Wk.T @ (np.exp(gamma[-1] - gamma)[:, None] * Ut)
    return o, S
