"""Pins of the fp64 oracle to facts the pages and mathematics fix.

None of these re-types the oracle's update formula and compares it with
itself: each checks a property that is computed independently (a dense
least-norm solve, a numerical line search, finite-difference gradients, the
textbook limit of Kaczmarz's cyclic projections, hand-derived examples,
invariants).  Sources, by page title and section:

[KLA] "Resumen Técnico: Atención Lineal Kaczmarz (KLA)", gist.science/es/paper/2605.08587
  §"Derivación Teórica"            write = projection of the decayed state onto
                                   {S : S^T k = v}; step 1/||k||^2
  §"La Regla de Actualización KLA" beta = eta/(||k||^2 + eps), S = S~ + beta k e^T,
                                   e = v - S~^T k
  §"Propiedades Clave"             with eta = 1, eps = 0: orthogonal projection
                                   (least-norm change), exact line search of the
                                   per-token loss, normalised gradient step

Every pin is written as a function of the recurrence under test, so the last
test can plant plausible mistakes in copies of the oracle (on the CPU) and
check that each mutant fails at least one pin.
"""

import math

import numpy as np
import pytest
import scipy.optimize

from oracle import kla_recurrence

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _keys(rng, L, dk, spread=1.0):
    k = rng.standard_normal((L, dk))
    return k * np.exp(spread * rng.standard_normal(L))[:, None]


def _case(seed, L, dk, dv, *, g_scale=1.0, eta=None, spread=1.0, s0=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((L, dk))
    k = _keys(rng, L, dk, spread)
    v = rng.standard_normal((L, dv))
    g = -g_scale * np.log1p(np.exp(rng.standard_normal(L)))
    if eta is None:
        eta = 1.0 / (1.0 + np.exp(-rng.standard_normal(L)))
    else:
        eta = np.full(L, float(eta))
    S0 = rng.standard_normal((dk, dv)) if s0 else None
    return q, k, v, g, eta, S0


# --------------------------------------------------------------------------
# pins, each a function of the recurrence ``rec``
# --------------------------------------------------------------------------

def pin_interpolation(rec):
    """eta = 1, eps = 0: every write satisfies S_t^T k_t = v_t ([KLA] §Derivación Teórica)."""
    q, k, v, g, eta, S0 = _case(1, 40, 6, 4, eta=1.0, spread=1.5)
    _, _, states = rec(q, k, v, g, eta, 0.0, S0, return_states=True)
    for t in range(len(k)):
        r = states[t + 1].T @ k[t] - v[t]
        assert np.max(np.abs(r)) <= 1e-10 * np.max(np.abs(v[t])), (t, r)


def _least_norm_change(k, e):
    """Least-Frobenius-norm D with D^T k = e, by a dense pseudo-inverse solve."""
    dk, dv = k.size, e.size
    M = np.zeros((dv, dk * dv))          # (D^T k)_j = sum_i D[i, j] k_i, D row-major
    for j in range(dv):
        M[j, j::dv] = k
    return (np.linalg.pinv(M) @ e).reshape(dk, dv)


def pin_least_norm(rec):
    """eta = 1, eps = 0: S_t - S~ is the least-norm solution of D^T k_t = e_t
    ([KLA] §Propiedades Clave, orthogonal projection).  Undecayed (g = 0) so
    that S~ = S_{t-1} needs no reading of the decay."""
    q, k, v, g, eta, S0 = _case(2, 8, 3, 2, eta=1.0)
    g = np.zeros_like(g)
    _, _, st = rec(q, k, v, g, eta, 0.0, S0, return_states=True)
    for t in range(len(k)):
        e = v[t] - st[t].T @ k[t]
        D = _least_norm_change(k[t], e)
        np.testing.assert_allclose(st[t + 1] - st[t], D, rtol=0, atol=1e-12 * max(1, np.abs(D).max()))


def pin_least_norm_decayed(rec):
    """Same as pin_least_norm around the decayed state exp(g_t) S_{t-1}."""
    q, k, v, g, eta, S0 = _case(3, 8, 3, 2, eta=1.0)
    _, _, st = rec(q, k, v, g, eta, 0.0, S0, return_states=True)
    for t in range(len(k)):
        S_dec = math.exp(g[t]) * st[t]
        D = _least_norm_change(k[t], v[t] - S_dec.T @ k[t])
        np.testing.assert_allclose(st[t + 1] - S_dec, D, rtol=0, atol=1e-12 * max(1, np.abs(D).max()))


def pin_line_search(rec):
    """eta = 1, eps = 0: the step along k e^T is the exact minimiser of the
    per-token loss 0.5 ||S^T k - v||^2 ([KLA] §Propiedades Clave, exact line
    search); the minimiser is found numerically (Brent)."""
    q, k, v, g, eta, S0 = _case(4, 12, 5, 3, eta=1.0, spread=1.5)
    g = np.zeros_like(g)
    _, _, st = rec(q, k, v, g, eta, 0.0, S0, return_states=True)
    for t in range(len(k)):
        S_dec, kt, vt = st[t], k[t], v[t]
        d = np.outer(kt, vt - S_dec.T @ kt)                 # update direction
        f = lambda b: 0.5 * np.sum(((S_dec + b * d).T @ kt - vt) ** 2)
        hi = 10.0 / (kt @ kt)
        res = scipy.optimize.minimize_scalar(f, bracket=(0.0, hi), tol=1e-14)
        b_star = res.x
        dS = st[t + 1] - S_dec
        b_eff = np.sum(dS * d) / np.sum(d * d)
        assert np.max(np.abs(dS - b_eff * d)) <= 1e-12 * np.max(np.abs(dS))  # along d
        assert abs(b_eff - b_star) <= 1e-7 * b_star, (t, b_eff, b_star)


def pin_normalised_gradient(rec):
    """General eta, eps: S_t - S~ = -(eta/(||k||^2+eps)) grad l(S~) with
    l(S) = 0.5 ||S^T k - v||^2, the gradient taken by central differences
    ([KLA] §Propiedades Clave, normalised SGD step)."""
    q, k, v, g, eta, S0 = _case(5, 6, 4, 3)
    g = np.zeros_like(g)
    eps = 0.25
    _, _, st = rec(q, k, v, g, eta, eps, S0, return_states=True)
    h = 1e-5
    for t in range(len(k)):
        S_dec, kt, vt = st[t], k[t], v[t]
        loss = lambda S: 0.5 * np.sum((S.T @ kt - vt) ** 2)
        grad = np.zeros_like(S_dec)
        for i in range(S_dec.shape[0]):
            for j in range(S_dec.shape[1]):
                E = np.zeros_like(S_dec)
                E[i, j] = h
                grad[i, j] = (loss(S_dec + E) - loss(S_dec - E)) / (2 * h)
        step = eta[t] / (kt @ kt + eps)
        np.testing.assert_allclose(st[t + 1] - S_dec, -step * grad, rtol=1e-6, atol=1e-8)


def pin_kaczmarz_limit(rec):
    """g = 0, eta = 1, eps = 0, cycling m <= dk independent keys: the state
    converges to the projection of S0 onto {S : K S = V}, i.e.
    S0 + pinv(K) (V - K S0) -- the textbook limit of Kaczmarz's method
    ([KLA] §Derivación Teórica names Kaczmarz projection)."""
    rng = np.random.default_rng(6)
    dk, dv, m, sweeps = 5, 3, 3, 400
    K = rng.standard_normal((m, dk)) * np.array([0.3, 1.0, 4.0])[:, None]
    V = rng.standard_normal((m, dv))
    S0 = rng.standard_normal((dk, dv))
    k = np.tile(K, (sweeps, 1))
    v = np.tile(V, (sweeps, 1))
    L = len(k)
    _, S = rec(np.zeros((L, dk)), k, v, np.zeros(L), np.ones(L), 0.0, S0)
    S_star = S0 + np.linalg.pinv(K) @ (V - K @ S0)
    np.testing.assert_allclose(S, S_star, rtol=0, atol=1e-10 * np.abs(S_star).max())


def pin_orthogonal_keys(rec):
    """Mutually orthogonal keys, g = 0, eta = 1, eps = 0: the writes do not
    interfere, S_T = S0 + sum_s k_s (v_s - S0^T k_s)^T / ||k_s||^2, and every
    pair is recalled exactly."""
    rng = np.random.default_rng(7)
    dk, dv, m = 6, 4, 5
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, m)))
    k = (Qm * np.array([0.2, 1.0, 3.0, 0.7, 10.0])).T
    v = rng.standard_normal((m, dv))
    S0 = rng.standard_normal((dk, dv))
    _, S = rec(np.zeros((m, dk)), k, v, np.zeros(m), np.ones(m), 0.0, S0)
    expect = S0.copy()
    for s in range(m):
        expect += np.outer(k[s], v[s] - S0.T @ k[s]) / (k[s] @ k[s])
    np.testing.assert_allclose(S, expect, rtol=0, atol=1e-12 * np.abs(expect).max())
    for s in range(m):
        np.testing.assert_allclose(S.T @ k[s], v[s], rtol=0, atol=1e-12)


def pin_pure_decay(rec):
    """eta = 0: nothing is written and the state only decays,
    S_t = exp(g_1 + ... + g_t) S0, o_t = S_t^T q_t."""
    q, k, v, g, eta, S0 = _case(8, 10, 4, 3)
    o, S = rec(q, k, v, g, np.zeros_like(eta), 1e-6, S0)
    gam = np.cumsum(g)
    np.testing.assert_allclose(S, math.exp(gam[-1]) * S0, rtol=1e-13, atol=0)
    for t in range(len(k)):
        np.testing.assert_allclose(o[t], math.exp(gam[t]) * S0.T @ q[t], rtol=1e-12, atol=1e-300)


def pin_hand_examples(rec):
    """Two small cases worked out by hand in exact binary fractions.

    Scalar (dk = dv = 1), S0 = 0:
      t1: k=2, v=1, q=1, g=0, eta=1, eps=0: beta=1/4, e=1, s=1/2, o=1/2
      t2: k=1, v=3, q=2, g=ln(1/2), eta=1/2, eps=0: beta=1/2, s~=1/4, e=11/4,
          s=1/4+11/8=13/8, o=13/4
      t3: k=-2, v=1, q=-1, g=0, eta=1, eps=4: beta=1/8, e=1+13/4=17/4,
          s=13/8-17/16=9/16, o=-9/16
    2x2, S0 = I:
      t1: k=(1,1), v=(0,2), q=(1,0), g=0, eta=1, eps=0: beta=1/2, e=(-1,1),
          S=[[1/2,1/2],[-1/2,3/2]], o=(1/2,1/2)
      t2: k=(0,2), v=(1,1), q=(0,1), g=ln(1/2), eta=1, eps=4: beta=1/8,
          S~=[[1/4,1/4],[-1/4,3/4]], S~^T k=(-1/2,3/2), e=(3/2,-1/2),
          S=[[1/4,1/4],[1/8,5/8]], o=(1/8,5/8)
    """
    o, S = rec(np.array([[1.0], [2.0], [-1.0]]), np.array([[2.0], [1.0], [-2.0]]),
               np.array([[1.0], [3.0], [1.0]]), np.array([0.0, math.log(0.5), 0.0]),
               np.array([1.0, 0.5, 1.0]), 0.0, np.zeros((1, 1)))
    # the third token has its own eps; run it as a continuation
    o3, S3 = rec(np.array([[-1.0]]), np.array([[-2.0]]), np.array([[1.0]]),
                 np.array([0.0]), np.array([1.0]), 4.0,
                 rec(np.array([[1.0], [2.0]]), np.array([[2.0], [1.0]]),
                     np.array([[1.0], [3.0]]), np.array([0.0, math.log(0.5)]),
                     np.array([1.0, 0.5]), 0.0, np.zeros((1, 1)))[1])
    np.testing.assert_allclose(o[:2, 0], [0.5, 3.25], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o3[0, 0], -9 / 16, rtol=0, atol=1e-15)
    np.testing.assert_allclose(S3[0, 0], 9 / 16, rtol=0, atol=1e-15)

    o_a, S_a = rec(np.array([[1.0, 0.0]]), np.array([[1.0, 1.0]]), np.array([[0.0, 2.0]]),
                   np.array([0.0]), np.array([1.0]), 0.0, np.eye(2))
    np.testing.assert_allclose(S_a, [[0.5, 0.5], [-0.5, 1.5]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o_a[0], [0.5, 0.5], rtol=0, atol=1e-15)
    o_b, S_b = rec(np.array([[0.0, 1.0]]), np.array([[0.0, 2.0]]), np.array([[1.0, 1.0]]),
                   np.array([math.log(0.5)]), np.array([1.0]), 4.0, S_a)
    np.testing.assert_allclose(S_b, [[0.25, 0.25], [0.125, 0.625]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o_b[0], [0.125, 0.625], rtol=0, atol=1e-15)


def pin_scale_invariance(rec):
    """eps = 0: scaling each pair (k_t, v_t) by its own c_t > 0 leaves every
    state unchanged -- the key-norm normalisation the method is about."""
    q, k, v, g, eta, S0 = _case(9, 30, 5, 3)
    c = np.exp(2.0 * np.random.default_rng(10).standard_normal(len(k)))
    o1, S1 = rec(q, k, v, g, eta, 0.0, S0)
    o2, S2 = rec(q, c[:, None] * k, c[:, None] * v, g, eta, 0.0, S0)
    np.testing.assert_allclose(S2, S1, rtol=0, atol=1e-12 * np.abs(S1).max())
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12 * np.abs(o1).max())


def pin_column_separability(rec):
    """Column j of S and o depends only on column j of v and S0."""
    q, k, v, g, eta, S0 = _case(11, 25, 4, 5)
    o, S = rec(q, k, v, g, eta, 1e-3, S0)
    for j in range(v.shape[1]):
        oj, Sj = rec(q, k, v[:, j:j + 1], g, eta, 1e-3, S0[:, j:j + 1])
        np.testing.assert_allclose(oj[:, 0], o[:, j], rtol=0, atol=1e-13 * np.abs(o).max())
        np.testing.assert_allclose(Sj[:, 0], S[:, j], rtol=0, atol=1e-13 * np.abs(S).max())


def pin_linearity(rec):
    """For fixed (q, k, g, eta) the outputs are linear in (v, S0) jointly."""
    q, k, v1, g, eta, S01 = _case(12, 25, 4, 3)
    rng = np.random.default_rng(13)
    v2, S02, a = rng.standard_normal(v1.shape), rng.standard_normal(S01.shape), -1.7
    o1, S1 = rec(q, k, v1, g, eta, 1e-3, S01)
    o2, S2 = rec(q, k, v2, g, eta, 1e-3, S02)
    o3, S3 = rec(q, k, v1 + a * v2, g, eta, 1e-3, S01 + a * S02)
    np.testing.assert_allclose(o3, o1 + a * o2, rtol=0, atol=1e-12 * np.abs(o3).max())
    np.testing.assert_allclose(S3, S1 + a * S2, rtol=0, atol=1e-12 * np.abs(S3).max())


def pin_boundedness(rec):
    """eta in [0, 2], eps >= 0: ||I - beta k k^T||_2 <= 1, hence
    ||S_t||_2 <= exp(g_t) ||S_{t-1}||_2 + eta_t ||v_t|| / ||k_t|| at every t."""
    rng = np.random.default_rng(14)
    L, dk, dv = 300, 6, 4
    q, k, v = rng.standard_normal((L, dk)), _keys(rng, L, dk, 2.0), rng.standard_normal((L, dv))
    g = -0.05 * np.log1p(np.exp(rng.standard_normal(L)))
    eta = rng.uniform(0.0, 2.0, L)
    _, _, st = rec(q, k, v, g, eta, 1e-6, np.zeros((dk, dv)), return_states=True)
    for t in range(L):
        lhs = np.linalg.norm(st[t + 1], 2)
        rhs = math.exp(g[t]) * np.linalg.norm(st[t], 2) + eta[t] * np.linalg.norm(v[t]) / np.linalg.norm(k[t])
        assert lhs <= rhs * (1 + 1e-12), (t, lhs, rhs)


ALL_PINS = [
    pin_interpolation, pin_least_norm, pin_least_norm_decayed, pin_line_search,
    pin_normalised_gradient, pin_kaczmarz_limit, pin_orthogonal_keys, pin_pure_decay,
    pin_hand_examples, pin_scale_invariance, pin_column_separability, pin_linearity,
    pin_boundedness,
]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(kla_recurrence)


# --------------------------------------------------------------------------
# planted mistakes (CPU only): each mutant of the recurrence must fail a pin
# --------------------------------------------------------------------------

def _mutant(kind):
    def rec(q, k, v, g, eta, eps, S0=None, return_states=False):
        L, dk = k.shape
        dv = v.shape[1]
        S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=float)
        o = np.empty((L, dv))
        states = [S.copy()]
        for t in range(L):
            kt = k[t]
            alpha = math.exp(-g[t]) if kind == "decay_sign" else math.exp(g[t])
            nrm = kt @ kt
            if kind == "norm_not_squared":
                nrm = math.sqrt(nrm)
            beta = eta[t] / (nrm + (0.0 if kind == "no_eps" else eps))
            S_dec = alpha * S
            e = v[t] - (S if kind == "residual_undecayed" else S_dec).T @ kt
            if kind == "decay_after_write":
                S_new = alpha * (S + beta * np.outer(kt, v[t] - S.T @ kt))
            elif kind == "sign":
                S_new = S_dec - beta * np.outer(kt, e)
            elif kind == "transposed_outer":
                S_new = S_dec + beta * np.outer(e, kt) if dk == dv else S_dec + beta * np.outer(kt, e)
            else:
                S_new = S_dec + beta * np.outer(kt, e)
            o[t] = (S if kind == "output_pre_update" else S_new).T @ q[t]
            if kind == "output_untransposed" and dk == dv:
                o[t] = S_new @ q[t]
            S = S_new
            states.append(S.copy())
        if return_states:
            return o, S, np.stack(states)
        return o, S
    return rec


MUTANTS = ["decay_sign", "norm_not_squared", "no_eps", "residual_undecayed",
           "decay_after_write", "sign", "transposed_outer", "output_pre_update",
           "output_untransposed"]


def test_unmutated_copy_passes_every_pin():
    rec = _mutant("none")
    for pin in ALL_PINS:
        pin(rec)


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_is_caught(kind):
    rec = _mutant(kind)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(rec)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {kind} passed every pin"
