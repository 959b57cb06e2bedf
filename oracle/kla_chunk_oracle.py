"""fp64 CPU chunkwise form of KLA (the block solver), for one sequence/head.

TEST INFRASTRUCTURE ONLY (see oracle/kla_oracle.py).  It is the reference for
the *algebra* the GPU prefill uses, and it is itself pinned to the
token-by-token recurrence (which is the method's definition) to ~1e-12.

Source: [KLA] "Resumen Técnico: Atención Lineal Kaczmarz (KLA)",
gist.science/es/paper/2605.08587, §"Implementación": KLA keeps Gated DeltaNet's
chunkwise-parallel training algorithm and only changes the diagonal
coefficient matrix B = Diag(beta_1..beta_C) inside the chunk solver.

The chunk algebra itself is not printed on the pages; it is the exact
reformulation of the recurrence over a chunk of C tokens with start state S0
(derived by unrolling the update; local index r = 1..C):

    gamma_r = sum_{j<=r} g_j        Gam_r = exp(gamma_r)
    beta_r  = eta_r / (||k_r||^2 + eps)
    A       = strictly-lower part of Diag(beta) K K^T, each (r, s) entry
              weighted by exp(gamma_r - gamma_s)
    T       = (I + A)^{-1}                     (unit lower triangular)
    W       = T Diag(beta * Gam) K,  U = T Diag(beta) V
    Ut      = U - W S0                         (Ut_r = beta_r e_r)
    O       = Diag(Gam) Q S0 + (Q K^T masked r >= s, weighted exp(gamma_r - gamma_s)) Ut
    S_C     = Gam_C S0 + K^T Diag(exp(gamma_C - gamma)) Ut

Every exponent used is of a non-positive number (r >= s), so the mask is
applied before the exponential.
"""

from __future__ import annotations

from typing import Optional

import numpy as np
import scipy.linalg

__all__ = ["kla_chunkwise"]


def kla_chunkwise(
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    g: np.ndarray,
    eta: np.ndarray,
    eps: float,
    S0: Optional[np.ndarray],
    chunk: int,
    return_chunks: bool = False,
    beta_given: Optional[np.ndarray] = None,
):
    """Chunkwise KLA for ONE sequence and ONE head in fp64.

    q, k: [L, dk]; v: [L, dv]; g, eta: [L]; S0: [dk, dv] or None.  The last
    chunk may be shorter than ``chunk``.  Returns (o [L, dv], S_L) and, with
    ``return_chunks``, a list of per-chunk dicts (beta, gamma, A, T, W, U, Ut,
    P) for inspecting intermediates.  With ``beta_given`` ([L]) the diagonal
    coefficients are taken as given (the gated delta rule, whose block solver
    KLA keeps, [KLA] §"Implementación") and eta, eps are not used.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    eta = np.asarray(eta, dtype=np.float64)
    L, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64, copy=True)
    o = np.empty((L, dv))
    dumps = []
    for c0 in range(0, L, chunk):
        c1 = min(c0 + chunk, L)
        n = c1 - c0
        K, Q, V = k[c0:c1], q[c0:c1], v[c0:c1]
        if beta_given is None:
            beta = eta[c0:c1] / (np.sum(K * K, axis=1) + eps)
        else:
            beta = np.asarray(beta_given, dtype=np.float64)[c0:c1]
        gamma = np.cumsum(g[c0:c1])
        Gam = np.exp(gamma)
        lower_incl = np.tril(np.ones((n, n), dtype=bool))
        diff = np.where(lower_incl, gamma[:, None] - gamma[None, :], 0.0)
        decay = np.where(lower_incl, np.exp(diff), 0.0)          # exp(gamma_r - gamma_s), r >= s
        A = np.tril(beta[:, None] * (K @ K.T) * decay, -1)
        T = scipy.linalg.solve_triangular(np.eye(n) + A, np.eye(n), lower=True,
                                          unit_diagonal=True)
        W = T @ ((beta * Gam)[:, None] * K)
        U = T @ (beta[:, None] * V)
        Ut = U - W @ S
        P = (Q @ K.T) * decay
        o[c0:c1] = Gam[:, None] * (Q @ S) + P @ Ut
        S = Gam[-1] * S + K.T @ (np.exp(gamma[-1] - gamma)[:, None] * Ut)
        if return_chunks:
            dumps.append(dict(beta=beta, gamma=gamma, A=A, T=T, W=W, U=U, Ut=Ut, P=P))
    if return_chunks:
        return o, S, dumps
    return o, S
