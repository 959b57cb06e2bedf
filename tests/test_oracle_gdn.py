"""Pins of the oracle's gated-delta-rule (Gated DeltaNet) mode: the KLA
recurrence with the update coefficient beta_t given instead of
eta_t / (||k_t||^2 + eps).

[KLA] "Resumen Técnico: Atención Lineal Kaczmarz (KLA)", gist.science/es/paper/2605.08587:
  §"Declaración del Problema"      GDN writes the residual with a learned scalar coefficient
  §"Metodología: Atención Lineal Kaczmarz"  KLA replaces that scalar with the Kaczmarz step
  §"Implementación"                state, gates, recurrence and block-parallel algorithm kept

Each pin checks a property computed independently of the update formula: a
hand-derived closed form, the projection property of the step 1/||k||^2, the
block (chunk) algebra, and the reduction to KLA when beta is KLA's step.
"""

import numpy as np
import pytest

from oracle import gdn_decode_step, gdn_forward, gdn_recurrence, kla_chunkwise, kla_forward

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _seq(seed, L, dk, dv):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((L, dk))
    k = rng.standard_normal((L, dk)) * np.exp(0.5 * rng.standard_normal(L))[:, None]
    v = rng.standard_normal((L, dv))
    g = -np.logaddexp(0.0, rng.standard_normal(L))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(L)))
    S0 = 0.3 * rng.standard_normal((dk, dv))
    return q, k, v, g, beta, S0


def test_single_token_closed_form():
    # S0 = 0: S_1 = beta k v^T and o_1 = beta (k.q) v (the decay acts on a zero state)
    q, k, v, g, beta, _ = _seq(1, 1, 5, 3)
    o, S = gdn_recurrence(q, k, v, g, beta)
    np.testing.assert_allclose(S, beta[0] * np.outer(k[0], v[0]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(o[0], beta[0] * (k[0] @ q[0]) * v[0], rtol=0, atol=1e-14)


def test_scalar_case_by_hand():
    # dk = dv = 1, three tokens: s <- a s + b k (v - a s k), o = s q, written out by hand
    q = np.array([[0.5], [-1.5], [2.0]])
    k = np.array([[2.0], [0.5], [-1.0]])
    v = np.array([[1.0], [3.0], [-2.0]])
    g = np.log(np.array([0.5, 0.8, 1.0]))
    beta = np.array([0.25, 2.0, 0.5])
    s, outs = 0.4, []
    for t, (a, b) in enumerate(zip([0.5, 0.8, 1.0], beta)):
        sd = a * s
        s = sd + b * k[t, 0] * (v[t, 0] - sd * k[t, 0])
        outs.append(s * q[t, 0])
    o, S = gdn_recurrence(q, k, v, g, beta, S0=np.array([[0.4]]))
    np.testing.assert_allclose(o[:, 0], outs, rtol=0, atol=1e-15)
    assert abs(S[0, 0] - s) <= 1e-15


def test_zero_beta_is_pure_decay():
    q, k, v, g, _, S0 = _seq(2, 9, 4, 3)
    o, S = gdn_recurrence(q, k, v, g, np.zeros(9), S0)
    np.testing.assert_allclose(S, np.exp(g.sum()) * S0, rtol=1e-14, atol=0)
    decays = np.exp(np.cumsum(g))
    np.testing.assert_allclose(o, np.stack([decays[t] * S0.T @ q[t] for t in range(9)]), rtol=1e-13, atol=0)


def test_kaczmarz_coefficient_interpolates():
    # beta_t = 1 / ||k_t||^2 is the orthogonal projection: every write stores v_t exactly
    q, k, v, g, _, S0 = _seq(3, 12, 6, 4)
    beta = 1.0 / np.sum(k * k, axis=1)
    S = S0.copy()
    for t in range(12):
        _, S = gdn_recurrence(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], beta[t:t + 1], S)
        np.testing.assert_allclose(S.T @ k[t], v[t], rtol=0, atol=1e-10 * np.abs(v[t]).max())


@pytest.mark.parametrize("C", [1, 3, 16, 64])
def test_block_form_equals_recurrence(C):
    q, k, v, g, beta, S0 = _seq(4, 150, 8, 6)
    o_r, S_r = gdn_recurrence(q, k, v, g, beta, S0)
    o_c, S_c = kla_chunkwise(q, k, v, g, None, None, S0, C, beta_given=beta)
    np.testing.assert_allclose(o_c, o_r, rtol=0, atol=1e-12 * np.abs(o_r).max())
    np.testing.assert_allclose(S_c, S_r, rtol=0, atol=1e-12 * np.abs(S_r).max())


def test_reduces_to_kla_with_the_kaczmarz_step():
    rng = np.random.default_rng(5)
    B, H, T, dk, dv = 2, 3, 20, 8, 5
    q, k, v = (rng.standard_normal((B, H, T, d)) for d in (dk, dk, dv))
    g = -np.logaddexp(0.0, rng.standard_normal((B, H, T)))
    eta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, H, T))))
    eps = 1e-3
    beta = eta / (np.sum(k * k, axis=-1) + eps)
    o_k, S_k = kla_forward(q, k, v, g, eta, eps)
    o_g, S_g = gdn_forward(q, k, v, g, beta)
    np.testing.assert_allclose(o_g, o_k, rtol=0, atol=1e-13 * np.abs(o_k).max())
    np.testing.assert_allclose(S_g, S_k, rtol=0, atol=1e-13 * np.abs(S_k).max())


def test_batch_driver_matches_per_sequence_recurrence_and_decode():
    rng = np.random.default_rng(6)
    H, dk, dv = 2, 4, 3
    cu = [0, 7, 7, 19]
    T = cu[-1]
    q, k, v = (rng.standard_normal((1, H, T, d)) for d in (dk, dk, dv))
    g = -np.logaddexp(0.0, rng.standard_normal((1, H, T)))
    beta = rng.uniform(0.0, 1.0, (1, H, T))
    S0 = rng.standard_normal((3, H, dk, dv))
    o, S = gdn_forward(q, k, v, g, beta, initial_state=S0, cu_seqlens=cu)
    for n in range(3):
        for h in range(H):
            t0, t1 = cu[n], cu[n + 1]
            o_r, S_r = gdn_recurrence(q[0, h, t0:t1], k[0, h, t0:t1], v[0, h, t0:t1], g[0, h, t0:t1],
                                      beta[0, h, t0:t1], S0[n, h])
            np.testing.assert_allclose(o[0, h, t0:t1], o_r, rtol=0, atol=1e-13)
            np.testing.assert_allclose(S[n, h], S_r, rtol=0, atol=1e-13)
    # decode steps over sequence 2 reproduce its prefill
    st = S0[2][None].copy()
    for t in range(cu[2], cu[3]):
        od, st = gdn_decode_step(q[:, :, t], k[:, :, t], v[:, :, t], g[:, :, t], beta[:, :, t], st)
        np.testing.assert_allclose(od[0], o[0, :, t], rtol=0, atol=1e-13)
    np.testing.assert_allclose(st[0], S[2], rtol=0, atol=1e-13)
