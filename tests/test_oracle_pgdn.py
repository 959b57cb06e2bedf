"""Pins of the PGDN oracle (preconditioned gated delta rule), CPU only.

[PDN] "Preconditioned DeltaNet: Curvature-aware Sequence Modeling for Linear
Recurrences", gist.science/es/paper/2604.21100:
  §2.A  an exact preconditioner applied to the write key ("ATK") recovers the
        least-squares solution
  §2.C  diagonal second moments A_t = A_{t-1} + k_t (.) k_t, P_t = Diag(A_t)^-1,
        squashed in log space into [1/x, x]
  §2.D  PGDN: the decayed (gated) variant, block-parallel form
[KLA] "Resumen Técnico: Atención Lineal Kaczmarz (KLA)", gist.science/es/paper/2605.08587,
  §"La Regla de Actualización KLA" (the Kaczmarz gain, with the preconditioned
  write key here) and §"Derivación Teórica" (with eta = 1, eps = 0 the write is
  a projection: S^T k = v, the change least-norm).

None of the pins retypes the update.  They check: the reduction to the
(separately coded) gated delta rule and KLA oracles where the preconditioner
is the identity (band x = 1, and keys whose coordinates all have one
magnitude); the accumulator's closed form (a plain sum of squares) and its
order independence; properties of the preconditioner observed through single
steps of the recurrence (scale-free, 1 at the mean, inverse order, inside the
band, odd in log space); interpolation and the P^-1-weighted least-norm change
under the Kaczmarz gain (brute-force weighted least-norm solve); the block
form with distinct read and write keys against the recurrence; the batch,
varlen, split/resume and decode drivers.  Every pin is a function of the
recurrence under test, so planted mistakes in copies of it must each fail one.
"""

import math

import numpy as np
import pytest

from oracle import gdn_recurrence, kla_recurrence
from oracle.pgdn_oracle import (GAIN_GIVEN, GAIN_KACZMARZ, PGDN_DELTA, pgdn_chunkwise, pgdn_decode_step,
                                pgdn_forward, pgdn_preconditioner, pgdn_recurrence)

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

BAND = 1.5


def _case(seed, L, dk, dv, *, spread=0.5, coef=None, g_scale=1.0, s0=True, scales=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((L, dk))
    k = rng.standard_normal((L, dk)) * np.exp(spread * rng.standard_normal(L))[:, None]
    if scales is not None:                      # per-coordinate key scales
        k = k * scales[None, :]
    v = rng.standard_normal((L, dv))
    g = -g_scale * np.log1p(np.exp(rng.standard_normal(L)))
    c = 1.0 / (1.0 + np.exp(-rng.standard_normal(L))) if coef is None else np.full(L, float(coef))
    S0 = 0.3 * rng.standard_normal((dk, dv)) if s0 else None
    return q, k, v, g, c, S0


def _states(rec, q, k, v, g, c, eps, gain, band, S0, A0=None):
    """Run token by token, returning the states S_0 .. S_L and accumulators."""
    S = np.zeros((k.shape[1], v.shape[1])) if S0 is None else S0.copy()
    A = np.zeros(k.shape[1]) if A0 is None else A0.copy()
    Ss, As = [S], [A]
    for t in range(len(k)):
        _, S, A = rec(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], c[t:t + 1], eps, gain, band, S, A)
        Ss.append(S)
        As.append(A)
    return Ss, As


def _observed_p(rec, kt, A_prev, band):
    """The preconditioner a step applies, observed from outside: one step from
    a zero state with beta = 1, no decay and v = e_0 writes S = w e_0^T, so
    w = S[:, 0] and p = w / k."""
    dk = kt.shape[0]
    v = np.zeros((1, 3))
    v[0, 0] = 1.0
    _, S, _ = rec(np.zeros((1, dk)), kt[None], v, np.zeros(1), np.ones(1), 0.0, GAIN_GIVEN, band,
                  np.zeros((dk, 3)), A_prev)
    return S[:, 0] / kt


# ---------------------------------------------------------------- pins ----

def pin_band_one_is_gdn_and_kla(rec):
    """x = 1 makes P = I: PGDN with the given gain is the gated delta rule, with
    the Kaczmarz gain it is KLA (both oracles are coded separately)."""
    q, k, v, g, c, S0 = _case(1, 37, 6, 4)
    o, S, _ = rec(q, k, v, g, c, 0.0, GAIN_GIVEN, 1.0, S0)
    o_r, S_r = gdn_recurrence(q, k, v, g, c, S0)
    np.testing.assert_allclose(o, o_r, rtol=0, atol=1e-12 * np.abs(o_r).max())
    np.testing.assert_allclose(S, S_r, rtol=0, atol=1e-12 * np.abs(S_r).max())
    o, S, _ = rec(q, k, v, g, c, 1e-3, GAIN_KACZMARZ, 1.0, S0)
    o_r, S_r = kla_recurrence(q, k, v, g, c, 1e-3, S0)
    np.testing.assert_allclose(o, o_r, rtol=0, atol=1e-12 * np.abs(o_r).max())
    np.testing.assert_allclose(S, S_r, rtol=0, atol=1e-12 * np.abs(S_r).max())


def pin_isotropic_keys_are_gdn(rec):
    """Keys whose coordinates all have the same magnitude keep every diagonal
    second moment equal, so the (scale-free) preconditioner is the identity at
    any band: the gated delta rule and KLA again."""
    rng = np.random.default_rng(2)
    L, dk, dv = 30, 8, 3
    q = rng.standard_normal((L, dk))
    k = np.sign(rng.standard_normal((L, dk))) * np.exp(rng.standard_normal(L))[:, None]
    v = rng.standard_normal((L, dv))
    g = -np.log1p(np.exp(rng.standard_normal(L)))
    c = 1.0 / (1.0 + np.exp(-rng.standard_normal(L)))
    S0 = rng.standard_normal((dk, dv))
    o, S, _ = rec(q, k, v, g, c, 0.0, GAIN_GIVEN, 3.0, S0)
    o_r, S_r = gdn_recurrence(q, k, v, g, c, S0)
    np.testing.assert_allclose(o, o_r, rtol=0, atol=1e-12 * np.abs(o_r).max())
    o, S, _ = rec(q, k, v, g, c, 0.0, GAIN_KACZMARZ, 3.0, S0)
    o_r, S_r = kla_recurrence(q, k, v, g, c, 0.0, S0)
    np.testing.assert_allclose(S, S_r, rtol=0, atol=1e-12 * np.abs(S_r).max())


def pin_accumulator_is_the_sum_of_squares(rec):
    """A_L = A_0 + sum_t k_t (.) k_t ([PDN] §2.C), whatever the gates, and
    therefore independent of the order of the tokens."""
    q, k, v, g, c, S0 = _case(3, 25, 5, 2, spread=1.0)
    A0 = np.abs(np.random.default_rng(4).standard_normal(5))
    _, _, A = rec(q, k, v, g, c, 1e-6, GAIN_KACZMARZ, BAND, S0, A0)
    np.testing.assert_allclose(A, A0 + np.sum(k * k, axis=0), rtol=1e-13)
    perm = np.random.default_rng(5).permutation(len(k))
    _, _, Ap = rec(q[perm], k[perm], v[perm], g[perm], c[perm], 1e-6, GAIN_GIVEN, BAND, S0, A0)
    np.testing.assert_allclose(Ap, A, rtol=1e-13)


def pin_preconditioner_properties(rec):
    """Observed through single steps: p lies in [1/x, x]; it is 1 where A_i
    equals the mean of A; larger second moments get smaller weights (Diag(A)^-1
    up to scale); scaling every key by s leaves it unchanged; it is odd in log
    space (coordinates whose A_i / mean are reciprocal get reciprocal weights);
    and the current token is in the accumulator."""
    dk = 4
    # coordinate scales d: A_i = t d_i^2 for keys d (.) (+-1); mean(d^2) = 1, so
    # coordinates 0 and 1 (d^2 = 1/2, 3/2?) ... chosen so that d0^2 d3^2 = 1
    d2 = np.array([0.5, 1.0, 0.5, 2.0])
    d2 = d2 / d2.mean()                       # mean of the second moments is 1
    rng = np.random.default_rng(6)
    A = np.zeros(dk)
    for t in range(6):
        kt = np.sign(rng.standard_normal(dk)) * np.sqrt(d2) * (3.0 if t % 2 else 0.5)
        p = _observed_p(rec, kt, A, BAND)
        A = A + kt * kt
        assert np.all(p >= 1 / BAND - 1e-12) and np.all(p <= BAND + 1e-12), p
        rel = A / A.mean()
        order = np.argsort(rel)
        assert np.all(np.diff(p[order]) <= 1e-12), (rel, p)      # inverse order
        if t == 0:
            # the first token alone: p depends on k_0 (.) k_0, not on the empty accumulator
            assert np.max(np.abs(p - 1.0)) > 1e-3, p
        # scale-free: all keys and the accumulator scaled by s^2
        ps = _observed_p(rec, 7.0 * kt, 49.0 * (A - kt * kt), BAND)
        np.testing.assert_allclose(ps, p, rtol=1e-12)
    # 1 at the mean, reciprocal pairs: A / mean = (0.5, 1, 0.5, 2) / 1 -> p0 * p3 = 1, p1 = 1
    rel = A / A.mean()
    assert abs(rel[1] - 1.0) < 1e-12 and abs(rel[0] * rel[3] - 1.0) < 1e-12
    kt = np.sqrt(d2) * 1e-9                     # a negligible token keeps A's ratios
    p = _observed_p(rec, kt, A - kt * kt, BAND)
    assert abs(p[1] - 1.0) <= 1e-9 and abs(p[0] * p[3] - 1.0) <= 1e-9, p


def pin_preconditioner_saturates(rec):
    """Coordinates whose second moment is far below or above the mean get the
    band's edges x and 1/x (the bounded squash of [PDN] §2.C)."""
    kt = np.array([1e-6, 1.0, 1.0, 1e3])
    p = _observed_p(rec, kt, np.zeros(4), BAND)
    assert abs(p[0] - BAND) <= 1e-3 and abs(p[3] - 1 / BAND) <= 1e-3, p


def pin_interpolation_kaczmarz(rec):
    """Kaczmarz gain, eta = 1, eps = 0: every write satisfies S_t^T k_t = v_t
    (the projection of the KLA page, in the preconditioned metric)."""
    q, k, v, g, c, S0 = _case(7, 30, 6, 4, coef=1.0, spread=1.5, scales=np.exp(np.linspace(-1, 1, 6)))
    Ss, _ = _states(rec, q, k, v, g, c, 0.0, GAIN_KACZMARZ, BAND, S0)
    for t in range(len(k)):
        r = Ss[t + 1].T @ k[t] - v[t]
        assert np.max(np.abs(r)) <= 1e-10 * np.max(np.abs(v[t])), (t, r)


def pin_weighted_least_norm(rec):
    """Kaczmarz gain, eta = 1, eps = 0: the change S_t - S~ is the solution of
    min sum_i ||Delta_i||^2 / p_i subject to Delta^T k_t = e_t (the exact solve
    the diagonal preconditioner stands in for), found by a dense weighted
    least-norm solve on vec(Delta); p is the weight the step applies, observed
    with a separate step."""
    q, k, v, g, c, S0 = _case(8, 7, 3, 2, coef=1.0, scales=np.array([0.3, 1.0, 2.5]))
    Ss, As = _states(rec, q, k, v, g, c, 0.0, GAIN_KACZMARZ, BAND, S0)
    dk, dv = 3, 2
    for t in range(len(k)):
        p = _observed_p(rec, k[t], As[t], BAND)
        S_dec = math.exp(g[t]) * Ss[t]
        e = v[t] - S_dec.T @ k[t]
        # unknown x = vec(Delta) (row-major, dk x dv); constraints: for each column j,
        # sum_i Delta_ij k_i = e_j.  Substitute Delta = Diag(sqrt p) Y and take the
        # least-norm Y.
        M = np.zeros((dv, dk * dv))
        for j in range(dv):
            for i in range(dk):
                M[j, i * dv + j] = k[t, i] * math.sqrt(p[i])
        y = np.linalg.pinv(M) @ e
        D = np.sqrt(p)[:, None] * y.reshape(dk, dv)
        np.testing.assert_allclose(Ss[t + 1] - S_dec, D, rtol=0, atol=1e-12 * max(1.0, np.abs(D).max()))


def pin_given_gain_step(rec):
    """Given gain: a step from a zero state writes beta_t (p (.) k_t) v_t^T and
    reads out o = beta (q . (p (.) k)) v -- the write key is preconditioned, the
    read-out key is not (ATK, [PDN] §2.A)."""
    rng = np.random.default_rng(9)
    kt = rng.standard_normal(5) * np.array([0.2, 0.5, 1.0, 2.0, 4.0])
    qt, vt = rng.standard_normal(5), rng.standard_normal(3)
    p = _observed_p(rec, kt, np.zeros(5), BAND)
    o, S, _ = rec(qt[None], kt[None], vt[None], np.array([-0.3]), np.array([0.7]), 0.0, GAIN_GIVEN, BAND,
                  np.zeros((5, 3)), np.zeros(5))
    np.testing.assert_allclose(S, 0.7 * np.outer(p * kt, vt), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(o[0], 0.7 * (qt @ (p * kt)) * vt, rtol=1e-13, atol=1e-15)


def pin_residual_uses_read_key(rec):
    """With a non-zero start state the residual is read with k (not w): one
    given-gain step from S0 equals exp(g) S0 + beta w (v - exp(g) S0^T k)^T,
    w observed separately."""
    rng = np.random.default_rng(10)
    dk, dv = 4, 3
    kt = rng.standard_normal(dk) * np.array([0.3, 1.0, 1.0, 3.0])
    qt, vt = rng.standard_normal(dk), rng.standard_normal(dv)
    S0 = rng.standard_normal((dk, dv))
    A0 = np.abs(rng.standard_normal(dk))
    w = _observed_p(rec, kt, A0, BAND) * kt
    a, b = math.exp(-0.2), 0.6
    _, S, _ = rec(qt[None], kt[None], vt[None], np.array([-0.2]), np.array([b]), 0.0, GAIN_GIVEN, BAND,
                  S0, A0)
    np.testing.assert_allclose(S, a * S0 + b * np.outer(w, vt - a * S0.T @ kt), rtol=1e-12, atol=1e-14)


ALL_PINS = [pin_band_one_is_gdn_and_kla, pin_isotropic_keys_are_gdn, pin_accumulator_is_the_sum_of_squares,
            pin_preconditioner_properties, pin_preconditioner_saturates, pin_interpolation_kaczmarz,
            pin_weighted_least_norm, pin_given_gain_step, pin_residual_uses_read_key]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pgdn_oracle_pin(pin):
    pin(pgdn_recurrence)


# ----------------------------------------------- the block form, drivers ----

@pytest.mark.parametrize("chunk", [1, 3, 16, 64])
@pytest.mark.parametrize("gain", [GAIN_GIVEN, GAIN_KACZMARZ])
def test_block_form_with_distinct_keys_equals_recurrence(chunk, gain):
    """[PDN] §2.D: the chunkwise form with read keys K and write keys W = P K
    gives the recurrence's outputs and state (ragged last chunk included)."""
    q, k, v, g, c, S0 = _case(11, 150, 8, 5, spread=1.0, scales=np.exp(np.linspace(-1.5, 1.5, 8)))
    A0 = np.abs(np.random.default_rng(12).standard_normal(8))
    o_r, S_r, _ = pgdn_recurrence(q, k, v, g, c, 1e-4, gain, BAND, S0, A0)
    p, _ = pgdn_preconditioner(k, BAND, A0)
    w = p * k
    beta = c if gain == GAIN_GIVEN else c / (np.sum(k * w, axis=1) + 1e-4)
    o, S = pgdn_chunkwise(q, k, w, v, g, beta, S0, chunk)
    np.testing.assert_allclose(o, o_r, rtol=0, atol=1e-12 * np.abs(o_r).max())
    np.testing.assert_allclose(S, S_r, rtol=0, atol=1e-12 * np.abs(S_r).max())


def test_preconditioner_helper_matches_the_accumulator():
    k = _case(13, 40, 6, 2, spread=1.0)[1]
    A0 = np.abs(np.random.default_rng(14).standard_normal(6))
    p, A = pgdn_preconditioner(k, BAND, A0)
    np.testing.assert_allclose(A, A0 + np.sum(k * k, 0), rtol=1e-13)
    for t in (0, 17, 39):
        np.testing.assert_allclose(p[t], _observed_p(pgdn_recurrence, k[t], A0 + np.sum(k[:t] ** 2, 0), BAND),
                                   rtol=1e-12)


def test_drivers_varlen_split_and_decode():
    rng = np.random.default_rng(15)
    H, dk, dv = 2, 4, 3
    lens = [0, 5, 1, 9]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = rng.standard_normal((1, H, T, dk))
    k = rng.standard_normal((1, H, T, dk)) * np.array([0.5, 1, 1, 2])
    v = rng.standard_normal((1, H, T, dv))
    g = -np.log1p(np.exp(rng.standard_normal((1, H, T))))
    c = 1 / (1 + np.exp(-rng.standard_normal((1, H, T))))
    S0 = rng.standard_normal((4, H, dk, dv))
    A0 = np.abs(rng.standard_normal((4, H, dk)))
    for gain in (GAIN_GIVEN, GAIN_KACZMARZ):
        o, S, A = pgdn_forward(q, k, v, g, c, 1e-5, gain, BAND, S0, A0, cu_seqlens=cu)
        for n in range(4):
            for h in range(H):
                a, b = cu[n], cu[n + 1]
                o_r, S_r, A_r = pgdn_recurrence(q[0, h, a:b], k[0, h, a:b], v[0, h, a:b], g[0, h, a:b],
                                                c[0, h, a:b], 1e-5, gain, BAND, S0[n, h], A0[n, h])
                np.testing.assert_allclose(o[0, h, a:b], o_r, rtol=1e-14, atol=1e-14)
                np.testing.assert_allclose(S[n, h], S_r, rtol=1e-14, atol=1e-14)
                np.testing.assert_allclose(A[n, h], A_r, rtol=1e-14)
        # split / resume inside the last sequence: carrying (S, A) is exact
        a, b = cu[3], cu[4]
        o1, S1, A1 = pgdn_recurrence(q[0, 0, a:a + 4], k[0, 0, a:a + 4], v[0, 0, a:a + 4], g[0, 0, a:a + 4],
                                     c[0, 0, a:a + 4], 1e-5, gain, BAND, S0[3, 0], A0[3, 0])
        o2, S2, A2 = pgdn_recurrence(q[0, 0, a + 4:b], k[0, 0, a + 4:b], v[0, 0, a + 4:b], g[0, 0, a + 4:b],
                                     c[0, 0, a + 4:b], 1e-5, gain, BAND, S1, A1)
        np.testing.assert_allclose(np.concatenate([o1, o2]), o[0, 0, a:b], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(S2, S[3, 0], rtol=1e-13, atol=1e-14)
        # decode, one token at a time for all (sequence, head) pairs of a dense batch
        qq, kk, vv = q[:, :, 6:10], k[:, :, 6:10], v[:, :, 6:10]
        gg, cc = g[:, :, 6:10], c[:, :, 6:10]
        o_p, S_p, A_p = pgdn_forward(qq, kk, vv, gg, cc, 1e-5, gain, BAND, S0[:1], A0[:1])
        St, At = S0[:1].copy(), A0[:1].copy()
        for t in range(4):
            od, St, At = pgdn_decode_step(qq[:, :, t], kk[:, :, t], vv[:, :, t], gg[:, :, t], cc[:, :, t], 1e-5,
                                          gain, BAND, St, At)
            np.testing.assert_allclose(od, o_p[:, :, t], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(St, S_p, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(At, A_p, rtol=1e-13)


def test_delta_is_the_fp32_guard():
    assert PGDN_DELTA == float(np.float32(1e-30)) and PGDN_DELTA > 0


# ------------------------------------------- planted mistakes (CPU only) ----

def _mutant(kind):
    def rec(q, k, v, g, coef, eps, gain, band, S0=None, A0=None):
        L, dk = k.shape
        S = np.zeros((dk, v.shape[1])) if S0 is None else np.array(S0, dtype=float)
        A = np.zeros(dk) if A0 is None else np.array(A0, dtype=float)
        o = np.empty((L, v.shape[1]))
        for t in range(L):
            kt = k[t]
            alpha = math.exp(g[t])
            A_prev = A
            A = (alpha * A if kind == "acc_decays" else A) + kt * kt
            Ause = A_prev if kind == "acc_excludes_current" else A
            if band == 1.0:
                p = np.ones(dk)
            else:
                cc = math.log(band)
                if kind == "no_mean_normalisation":
                    r = -np.log(Ause + PGDN_DELTA)
                else:
                    r = np.log((Ause.mean() + PGDN_DELTA) / (Ause + PGDN_DELTA))
                p = np.exp((-1 if kind == "squash_sign" else 1) * cc * np.tanh(r / cc))
            w = kt / p if kind == "inverse_precond" else (kt if kind == "write_key_unpreconditioned" else p * kt)
            if gain == GAIN_GIVEN:
                beta = coef[t]
            else:
                beta = coef[t] / ((kt @ kt if kind == "gain_kk" else kt @ w) + eps)
            S_dec = alpha * S
            e = v[t] - S_dec.T @ (w if kind == "residual_with_w" else kt)
            S = S_dec + beta * np.outer(w, e)
            o[t] = S.T @ q[t]
        return o, S, A
    return rec


MUTANTS = ["write_key_unpreconditioned", "inverse_precond", "acc_excludes_current", "gain_kk",
           "residual_with_w", "squash_sign", "acc_decays", "no_mean_normalisation"]


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
