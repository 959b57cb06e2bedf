"""fp64 CPU oracle of the gradients of the KLA recurrence (reverse mode).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module; only the test-suite, the smoke check and the benchmark's CPU-baseline
leg do.  It shares no code with the HIP path.

What it computes: for the forward map of kla_oracle.kla_forward (or gdn_forward)
and upstream gradients dO = dL/do and dS_T = dL/dS_final, the gradients of that
scalar L with respect to q, k, v, g, eta (or beta) and the initial state, by the
chain rule applied to each token step in reverse order.

Source: "Resumen Técnico: Atención Lineal Kaczmarz (KLA)", gist.science/es/paper/2605.08587.
§"Implementación" states that KLA keeps Gated DeltaNet's parallel chunk *training*
algorithm, so the method is trained through this recurrence; the step
differentiated here is the one of §"La Regla de Actualización KLA" (with the
decay read as S~ = exp(g_t) S, the readout o_t = S_t^T q_t, as in kla_oracle).

One token step and its adjoint (dS is dL/dS_t on entry, dL/dS_{t-1} on exit):

    forward                          reverse
    alpha = exp(g)                   dS   += q do^T                (o = S_t^T q)
    n     = k.k                      dq    = S_t do
    beta  = eta / (n + eps)          dbeta = k^T dS e ;  dk = beta dS e ;  de = beta dS^T k
    S~    = alpha S_{t-1}            dv    = de ;  dS~ = dS - k de^T ;  dk -= S~ de
    e     = v - S~^T k               dalpha = <S_{t-1}, dS~> ;  dg = alpha dalpha
    S_t   = S~ + beta k e^T          dS    = alpha dS~
    o     = S_t^T q                  deta  = dbeta / (n + eps) ;  dk -= 2 eta dbeta/(n+eps)^2 k

In the gated-delta-rule mode beta is an input and its gradient is dbeta.

Parity status: pinned by element-wise central finite differences of the forward
oracle, hand-derived closed forms (one token from a zero state, pure decay) and
structural invariants; see tests/test_oracle_backward.py.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

__all__ = ["kla_backward", "gdn_backward"]

_CKPT = 64  # tokens between stored states in the reverse sweep


def _heads_backward(q, k, v, g, coef, eps, S0, dO, dST, beta_given):
    """Reverse sweep for one sequence, vectorised over a leading head axis.

    q, k: [H, L, dk]; v, dO: [H, L, dv]; g, coef: [H, L]; S0, dST: [H, dk, dv].
    coef is eta (KLA) or beta (beta_given).  Returns dq, dk, dv, dg, dcoef, dS0.
    The forward states are kept every _CKPT tokens and recomputed in between.
    """
    H, L, dk = k.shape
    dv = v.shape[2]
    nrm = np.einsum("hti,hti->ht", k, k)
    beta = coef if beta_given else coef / (nrm + eps)
    alpha = np.exp(g)

    def step(S, t):
        S_dec = alpha[:, t, None, None] * S
        e = v[:, t] - np.einsum("hij,hi->hj", S_dec, k[:, t])
        return S_dec + beta[:, t, None, None] * k[:, t, :, None] * e[:, None, :]

    ckpt = {}
    S = S0.copy()
    for t in range(L):
        if t % _CKPT == 0:
            ckpt[t] = S.copy()
        S = step(S, t)

    gq, gk, gv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    gg, gcoef = np.zeros((H, L)), np.zeros((H, L))
    dS = dST.copy()
    if L == 0:  # an empty sequence passes its state (and the state's gradient) through
        return gq, gk, gv, gg, gcoef, dS
    for c0 in range(((L - 1) // _CKPT) * _CKPT, -1, -_CKPT):
        c1 = min(c0 + _CKPT, L)
        states = [ckpt[c0]]                      # S_{c0-1+1} .. S_{c1}: states[j] = state before token c0+j
        for t in range(c0, c1):
            states.append(step(states[-1], t))
        for t in range(c1 - 1, c0 - 1, -1):
            S_prev, S_t = states[t - c0], states[t - c0 + 1]
            kt, qt, dot = k[:, t], q[:, t], dO[:, t]
            dS += qt[:, :, None] * dot[:, None, :]
            gq[:, t] = np.einsum("hij,hj->hi", S_t, dot)
            S_dec = alpha[:, t, None, None] * S_prev
            e = v[:, t] - np.einsum("hij,hi->hj", S_dec, kt)
            dSe = np.einsum("hij,hj->hi", dS, e)            # dS e   [H, dk]
            dbeta = np.einsum("hi,hi->h", kt, dSe)
            b = beta[:, t]
            dkt = b[:, None] * dSe
            de = b[:, None] * np.einsum("hij,hi->hj", dS, kt)
            gv[:, t] = de
            dS_dec = dS - kt[:, :, None] * de[:, None, :]
            dkt -= np.einsum("hij,hj->hi", S_dec, de)
            dalpha = np.einsum("hij,hij->h", S_prev, dS_dec)
            gg[:, t] = alpha[:, t] * dalpha
            dS = alpha[:, t, None, None] * dS_dec
            if beta_given:
                gcoef[:, t] = dbeta
            else:
                den = nrm[:, t] + eps
                gcoef[:, t] = dbeta / den
                dkt -= (2.0 * coef[:, t] * dbeta / den ** 2)[:, None] * kt
            gk[:, t] = dkt
    return gq, gk, gv, gg, gcoef, dS


def _backward(q, k, v, g, coef, eps, do, dS_final, initial_state, cu_seqlens, heads, beta_given):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    coef = np.asarray(coef, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, T, dk = k.shape
    dv = v.shape[3]
    if cu_seqlens is None:
        segs = [(b, 0, T) for b in range(B)]
    else:
        if B != 1:
            raise ValueError("packed sequences need B == 1")
        cu = [int(x) for x in cu_seqlens]
        segs = [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    hs = list(range(H)) if heads is None else [int(h) for h in heads]
    out = [np.full(q.shape, np.nan), np.full(k.shape, np.nan), np.full(v.shape, np.nan),
           np.full(g.shape, np.nan), np.full(coef.shape, np.nan)]
    dS0 = np.full((len(segs), H, dk, dv), np.nan)
    for n, (b, t0, t1) in enumerate(segs):
        S0 = (np.zeros((len(hs), dk, dv)) if initial_state is None
              else np.array(np.asarray(initial_state, dtype=np.float64)[n, hs], copy=True))
        dST = (np.zeros((len(hs), dk, dv)) if dS_final is None
               else np.array(np.asarray(dS_final, dtype=np.float64)[n, hs], copy=True))
        sl = (b, hs, slice(t0, t1))
        res = _heads_backward(q[sl], k[sl], v[sl], g[sl], coef[sl], eps, S0, do[sl], dST, beta_given)
        for dst, r in zip(out, res[:5]):
            dst[sl] = r
        dS0[n, hs] = res[5]
    return tuple(out) + (dS0,)


def kla_backward(q, k, v, g, eta, eps, do, dS_final=None, initial_state=None,
                 cu_seqlens: Optional[Sequence[int]] = None, heads: Optional[Sequence[int]] = None):
    """Gradients of L = <o, do> + <S_final, dS_final> through kla_forward, fp64.

    Layouts as kla_forward: q, k [B, H, T, dk]; v, do [B, H, T, dv]; g, eta
    [B, H, T]; initial_state, dS_final [N, H, dk, dv] or None (zeros).
    Returns (dq, dk, dv, dg, deta, dS0) with the shapes of (q, k, v, g, eta,
    initial_state).  ``heads`` restricts the work to a subset of heads (the
    others are NaN)."""
    return _backward(q, k, v, g, eta, eps, do, dS_final, initial_state, cu_seqlens, heads, False)


def gdn_backward(q, k, v, g, beta, do, dS_final=None, initial_state=None,
                 cu_seqlens: Optional[Sequence[int]] = None, heads: Optional[Sequence[int]] = None):
    """As kla_backward for the gated delta rule (beta [B, H, T] given); returns
    (dq, dk, dv, dg, dbeta, dS0)."""
    return _backward(q, k, v, g, beta, None, do, dS_final, initial_state, cu_seqlens, heads, True)
