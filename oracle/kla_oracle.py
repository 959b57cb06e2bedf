"""fp64 CPU oracle of the Kaczmarz Linear Attention (KLA) recurrence.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module; only the test-suite, the smoke check and the benchmark's CPU-baseline
leg do.  It shares no code with the HIP path.

What it computes is the plain definition of the method, token by token, in
float64 (numpy), taking every input exactly as the GPU receives it (bf16/fp32
values widened without change; eps as the same fp32 value).

Sources (cited by page title and section):

[KLA] "Resumen Técnico: Atención Lineal Kaczmarz (KLA)", gist.science/es/paper/2605.08587
      (same text in German at gist.science/de/paper/2605.08587 and French at
      gist.science/fr/paper/2605.08587).

  * §"Derivación Teórica": the write of token t is the state closest (in
    Frobenius norm) to the *decayed* previous state S~_{t-1} that satisfies
    S^T k_t = v_t; its solution is the orthogonal projection, step 1/||k_t||^2.
  * §"La Regla de Actualización KLA": beta_t = eta_t / (||k_t||_2^2 + eps),
    S_t = S~_{t-1} + beta_t k_t e_t^T with e_t = v_t - S~_{t-1}^T k_t.
  * §"Implementación": state S in R^{dk x dv}; decay and update gates kept
    from Gated DeltaNet.

Readings where the pages are silent (each listed in the design notes):

  * decay: S~_{t-1} = exp(g_t) * S_{t-1} with g_t one log-decay scalar per
    (token, head) -- the Gated-DeltaNet decay gate the pages say is kept;
  * output: o_t = S_t^T q_t with the post-update state, no 1/sqrt(dk) scale;
  * keys are used as given (no normalisation inside the operator);
  * chunking/varlen: a sequence starts from its own initial state (zero when
    absent) and carries its state only within itself.

Parity status: every function here is pinned by tests that do not retype its
formula (interpolation, least-norm projection, line search, finite-difference
gradient, Kaczmarz limit, closed forms, invariants); see tests/test_oracle_pins.py.
"""

from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = ["kla_recurrence", "kla_forward", "kla_decode_step", "gdn_recurrence", "gdn_forward",
           "gdn_decode_step"]


def kla_recurrence(
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    g: np.ndarray,
    eta: np.ndarray,
    eps: float,
    S0: Optional[np.ndarray] = None,
    return_states: bool = False,
):
    """Token-by-token KLA for ONE sequence and ONE head, in fp64.

    q, k: [L, dk]; v: [L, dv]; g, eta: [L]; S0: [dk, dv] or None (zeros).
    Returns (o [L, dv], S_L [dk, dv]) and, with ``return_states``, also all
    states [L + 1, dk, dv] (S_0 .. S_L).

    Each step follows [KLA] §"La Regla de Actualización KLA" with the decay of
    §"Derivación Teórica" read as S~ = exp(g_t) S:
        alpha = exp(g_t)
        beta  = eta_t / (k_t . k_t + eps)
        S~    = alpha S
        e     = v_t - S~^T k_t
        S     = S~ + beta k_t e^T
        o_t   = S^T q_t
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
    states = [S.copy()] if return_states else None
    for t in range(L):
        kt = k[t]
        alpha = np.exp(g[t])
        beta = eta[t] / (kt @ kt + eps)
        S_dec = alpha * S
        e = v[t] - S_dec.T @ kt
        S = S_dec + beta * np.outer(kt, e)
        o[t] = S.T @ q[t]
        if return_states:
            states.append(S.copy())
    if return_states:
        return o, S, np.stack(states)
    return o, S


def _run_heads(q, k, v, g, eta, eps, S, beta_given=None):
    """The same recurrence vectorised over a leading head axis (in place on S).

    q, k: [H, L, dk]; v: [H, L, dv]; g, eta: [H, L]; S: [H, dk, dv] fp64.
    With ``beta_given`` ([H, L]) the update coefficient is taken as given
    (the gated delta rule) and eta, eps are not used.
    Returns o [H, L, dv].
    """
    H, L, _ = k.shape
    o = np.empty((H, L, v.shape[2]))
    for t in range(L):
        kt = k[:, t, :]                                     # [H, dk]
        alpha = np.exp(g[:, t])                             # [H]
        if beta_given is None:
            beta = eta[:, t] / (np.einsum("hi,hi->h", kt, kt) + eps)
        else:
            beta = beta_given[:, t]
        S *= alpha[:, None, None]                           # S~ = alpha S
        e = v[:, t, :] - np.einsum("hij,hi->hj", S, kt)     # e = v - S~^T k
        S += beta[:, None, None] * kt[:, :, None] * e[:, None, :]
        o[:, t, :] = np.einsum("hij,hi->hj", S, q[:, t, :])  # o = S^T q
    return o


def _forward(q, k, v, g, coef, eps, initial_state, cu_seqlens, heads, beta_given):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    coef = np.asarray(coef, dtype=np.float64)
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
    o = np.full((B, H, T, dv), np.nan)
    S_fin = np.full((len(segs), H, dk, dv), np.nan)
    for n, (b, t0, t1) in enumerate(segs):
        if initial_state is None:
            S = np.zeros((len(hs), dk, dv))
        else:
            S = np.array(np.asarray(initial_state, dtype=np.float64)[n, hs], copy=True)
        c = coef[b, hs, t0:t1]
        o[b, hs, t0:t1] = _run_heads(q[b, hs, t0:t1], k[b, hs, t0:t1], v[b, hs, t0:t1],
                                     g[b, hs, t0:t1], None if beta_given else c, eps, S,
                                     beta_given=c if beta_given else None)
        S_fin[n, hs] = S
    return o, S_fin


def kla_forward(
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    g: np.ndarray,
    eta: np.ndarray,
    eps: float,
    initial_state: Optional[np.ndarray] = None,
    cu_seqlens: Optional[Sequence[int]] = None,
    heads: Optional[Sequence[int]] = None,
) -> Tuple[np.ndarray, np.ndarray]:
    """KLA over a batch in the [B, H, T, d] layout, fp64.

    Without ``cu_seqlens`` each batch row is one sequence (N = B).  With it,
    B must be 1 and sequence n is tokens [cu[n], cu[n+1]) of that row.  Every
    sequence starts from ``initial_state[n]`` ([N, H, dk, dv]) or zeros.

    ``heads`` restricts the computation to a subset of heads (outputs for the
    other heads are left as NaN); used to sample large workloads.

    Returns (o [B, H, T, dv], final states [N, H, dk, dv]).
    """
    return _forward(q, k, v, g, eta, eps, initial_state, cu_seqlens, heads, beta_given=False)


def gdn_forward(
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    g: np.ndarray,
    beta: np.ndarray,
    initial_state: Optional[np.ndarray] = None,
    cu_seqlens: Optional[Sequence[int]] = None,
    heads: Optional[Sequence[int]] = None,
) -> Tuple[np.ndarray, np.ndarray]:
    """The gated delta rule (Gated DeltaNet) over a batch, fp64: the KLA
    recurrence with the update coefficient beta_t [B, H, T] given instead of
    eta_t / (||k_t||^2 + eps).  [KLA] §"Declaración del Problema" and
    §"Metodología: Atención Lineal Kaczmarz": KLA is GDN with that learned
    coefficient replaced by the Kaczmarz step; state, gates and recurrence are
    kept (§"Implementación").  Arguments and results as kla_forward."""
    return _forward(q, k, v, g, beta, None, initial_state, cu_seqlens, heads, beta_given=True)


def kla_decode_step(
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    g: np.ndarray,
    eta: np.ndarray,
    eps: float,
    state: np.ndarray,
) -> Tuple[np.ndarray, np.ndarray]:
    """One recurrent step for N sequences x H heads, fp64.

    q, k: [N, H, dk]; v: [N, H, dv]; g, eta: [N, H]; state: [N, H, dk, dv].
    Returns (o [N, H, dv], new state).  The step is the token update of
    [KLA] §"La Regla de Actualización KLA" applied once per (sequence, head).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, H, dk = k.shape
    S = np.array(state, dtype=np.float64, copy=True).reshape(N * H, dk, -1)
    o = _run_heads(q.reshape(N * H, 1, dk), k.reshape(N * H, 1, dk),
                   v.reshape(N * H, 1, -1), np.asarray(g, np.float64).reshape(N * H, 1),
                   np.asarray(eta, np.float64).reshape(N * H, 1), eps, S)
    return o.reshape(N, H, -1), S.reshape(N, H, dk, -1)


def gdn_decode_step(
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    g: np.ndarray,
    beta: np.ndarray,
    state: np.ndarray,
) -> Tuple[np.ndarray, np.ndarray]:
    """One gated-delta-rule step for N sequences x H heads, fp64 (beta [N, H]
    given); as kla_decode_step otherwise."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, H, dk = k.shape
    S = np.array(state, dtype=np.float64, copy=True).reshape(N * H, dk, -1)
    o = _run_heads(q.reshape(N * H, 1, dk), k.reshape(N * H, 1, dk),
                   v.reshape(N * H, 1, -1), np.asarray(g, np.float64).reshape(N * H, 1),
                   None, None, S, beta_given=np.asarray(beta, np.float64).reshape(N * H, 1))
    return o.reshape(N, H, -1), S.reshape(N, H, dk, -1)


def gdn_recurrence(q, k, v, g, beta, S0=None):
    """Token-by-token gated delta rule for ONE sequence and ONE head, fp64:
    q, k [L, dk]; v [L, dv]; g, beta [L]; S0 [dk, dv] or None.  Each step:
    S~ = exp(g_t) S, e = v_t - S~^T k_t, S = S~ + beta_t k_t e^T, o_t = S^T q_t.
    Returns (o [L, dv], S_L)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    L, dk = k.shape
    S = np.zeros((dk, v.shape[1])) if S0 is None else np.array(S0, dtype=np.float64, copy=True)
    o = np.empty((L, v.shape[1]))
    for t in range(L):
        S_dec = np.exp(g[t]) * S
        e = v[t] - S_dec.T @ k[t]
        S = S_dec + beta[t] * np.outer(k[t], e)
        o[t] = S.T @ q[t]
    return o, S
