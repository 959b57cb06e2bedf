"""Pins of the fp64 backward oracle (oracle/kla_backward_oracle.py).

The gradient oracle is the chain rule applied to the token recurrence by hand.
Nothing here re-types it: the pins are

* element-wise central finite differences of the *forward* oracle (itself pinned
  in test_oracle_pins.py) for every input of small KLA and gated-delta-rule
  cases, including a sequence longer than the reverse sweep's checkpoint
  interval and packed sequences;
* closed forms derived by hand: one token from a zero state, and pure decay
  (eta = 0), where o_t = exp(sum_{s<=t} g_s) S0^T q_t;
* structure: packed sequences give the gradients of separate calls, and the
  gradients are linear in the upstream gradients.

The last test plants plausible mistakes (a dropped term, a wrong sign, the
wrong state) in copies of the oracle, on the CPU, and checks that each one fails
the finite-difference pin.

Source: "Resumen Técnico: Atención Lineal Kaczmarz (KLA)", gist.science/es/paper/2605.08587,
§"La Regla de Actualización KLA" (the step) and §"Implementación" (the method is trained
through the same recurrence as Gated DeltaNet).
"""

import inspect
import types

import numpy as np
import pytest

import oracle.kla_backward_oracle as kbo
from oracle import kla_forward, gdn_forward


def _case(seed, B, H, T, dk, dv, *, s0=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk)) * np.exp(0.5 * rng.standard_normal((B, H, T, 1)))
    v = rng.standard_normal((B, H, T, dv))
    g = -np.log1p(np.exp(rng.standard_normal((B, H, T))))
    eta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, H, T))))
    do = rng.standard_normal((B, H, T, dv))
    return q, k, v, g, eta, do, rng


def _loss(fwd, args, do, dS_T, S0, cu):
    o, S = fwd(*args, initial_state=S0, cu_seqlens=cu)
    val = float(np.sum(o * do))
    if dS_T is not None:
        val += float(np.sum(S * dS_T))
    return val


def _fd_check(fwd, bwd, q, k, v, g, coef, eps, do, dS_T, S0, cu, rtol=2e-6):
    """Compare every gradient element with a central difference of the loss."""
    extra = () if eps is None else (eps,)
    grads = bwd(q, k, v, g, coef, *extra, do, dS_T, S0, cu_seqlens=cu)
    inputs = [q, k, v, g, coef, S0]
    names = ["dq", "dk", "dv", "dg", "dcoef", "dS0"]
    for idx, (name, x, gx) in enumerate(zip(names, inputs, grads)):
        if x is None:
            continue
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            h = 1e-6 * max(1.0, abs(x[i]))
            xs = [a.copy() if a is not None else None for a in inputs]
            xs[idx][i] = x[i] + h
            lp = _loss(fwd, tuple(xs[:5]) + extra, do, dS_T, xs[5], cu)
            xs[idx][i] = x[i] - h
            lm = _loss(fwd, tuple(xs[:5]) + extra, do, dS_T, xs[5], cu)
            num[i] = (lp - lm) / (2 * h)
        scale = max(np.max(np.abs(num)), 1e-12)
        err = np.max(np.abs(gx - num)) / scale
        assert err <= rtol, (name, err)


def test_fd_kla_long_sequence_with_states():
    """Every gradient of a 70-token KLA sequence (past one 64-token checkpoint
    interval), with an initial state and an upstream state gradient."""
    q, k, v, g, eta, do, rng = _case(11, 1, 2, 70, 3, 2)
    S0 = rng.standard_normal((1, 2, 3, 2))
    dS_T = rng.standard_normal((1, 2, 3, 2))
    _fd_check(kla_forward, kbo.kla_backward, q, k, v, g, eta, 1e-3, do, dS_T, S0, None)


def test_fd_kla_batch_no_states():
    q, k, v, g, eta, do, _ = _case(12, 2, 1, 9, 4, 3)
    _fd_check(kla_forward, kbo.kla_backward, q, k, v, g, eta, 1e-6, do, None, None, None)


def test_fd_kla_packed_sequences():
    """Packed sequences, one of them empty (its state and gradient pass through)."""
    q, k, v, g, eta, do, rng = _case(13, 1, 1, 17, 3, 3)
    cu = [0, 5, 5, 6, 17]
    S0 = rng.standard_normal((4, 1, 3, 3))
    dS_T = rng.standard_normal((4, 1, 3, 3))
    _fd_check(kla_forward, kbo.kla_backward, q, k, v, g, eta, 1e-6, do, dS_T, S0, cu)


def test_fd_gated_delta_rule():
    q, k, v, g, _, do, rng = _case(14, 1, 2, 12, 3, 2)
    beta = rng.uniform(0.1, 1.5, size=g.shape)
    S0 = rng.standard_normal((1, 2, 3, 2))
    dS_T = rng.standard_normal((1, 2, 3, 2))
    _fd_check(gdn_forward, kbo.gdn_backward, q, k, v, g, beta, None, do, dS_T, S0, None)


def test_single_token_closed_form():
    """From S0 = 0 one token gives o = beta (k.q) v with beta = eta/(k.k + eps),
    so for L = <o, w>: dv = beta (k.q) w, dq = beta (w.v) k,
    deta = (k.q)(w.v)/(n + eps), dk = (w.v) eta (q/(n+eps) - 2 (k.q) k/(n+eps)^2)
    and dg = 0 (nothing to decay).  The loss is linear in S0, so its gradient
    there, exp(g) (q - beta (k.q) k) w^T, holds at S0 = 0 too."""
    rng = np.random.default_rng(5)
    dk, dv = 4, 3
    q = rng.standard_normal((1, 1, 1, dk))
    k = rng.standard_normal((1, 1, 1, dk))
    v = rng.standard_normal((1, 1, 1, dv))
    g = np.array([[[-0.3]]])
    eta = np.array([[[0.7]]])
    w = rng.standard_normal((1, 1, 1, dv))
    eps = 1e-2
    dq, dkk, dvv, dg, deta, dS0 = kbo.kla_backward(q, k, v, g, eta, eps, w)
    qv, kv, vv, wv = q[0, 0, 0], k[0, 0, 0], v[0, 0, 0], w[0, 0, 0]
    n = kv @ kv
    beta = 0.7 / (n + eps)
    kq, wv_v = kv @ qv, wv @ vv
    np.testing.assert_allclose(dvv[0, 0, 0], beta * kq * wv, rtol=1e-13)
    np.testing.assert_allclose(dq[0, 0, 0], beta * wv_v * kv, rtol=1e-13)
    np.testing.assert_allclose(deta[0, 0, 0], kq * wv_v / (n + eps), rtol=1e-13)
    np.testing.assert_allclose(dkk[0, 0, 0],
                               wv_v * 0.7 * (qv / (n + eps) - 2 * kq * kv / (n + eps) ** 2),
                               rtol=1e-12, atol=1e-14)
    assert abs(dg[0, 0, 0]) < 1e-15
    # S1 = a S0 + beta k (v - a S0^T k)^T, o = S1^T q, so
    # dL/dS0 = a (q - beta (k.q) k) w^T, with a = exp(g).
    a = np.exp(-0.3)
    np.testing.assert_allclose(dS0[0, 0], a * np.outer(qv - beta * kq * kv, wv), rtol=1e-12, atol=1e-15)


def test_pure_decay_closed_form():
    """eta = 0: S_t = exp(G_t) S0 with G_t = sum_{s<=t} g_s, o_t = S_t^T q_t.
    For L = sum_t <o_t, w_t>: dS0 = sum_t exp(G_t) q_t w_t^T,
    dg_s = sum_{t>=s} exp(G_t) q_t^T S0 w_t, dq_t = exp(G_t) S0 w_t, dv = 0."""
    rng = np.random.default_rng(6)
    T, dk, dv = 10, 3, 4
    q, k, v, g, _, w, _ = _case(7, 1, 1, T, dk, dv)
    eta = np.zeros((1, 1, T))
    S0 = rng.standard_normal((1, 1, dk, dv))
    dq, _, dvv, dg, _, dS0 = kbo.kla_backward(q, k, v, g, eta, 1e-6, w, None, S0)
    G = np.cumsum(g[0, 0])
    s0 = S0[0, 0]
    terms = np.array([np.exp(G[t]) * (q[0, 0, t] @ s0 @ w[0, 0, t]) for t in range(T)])
    np.testing.assert_allclose(dg[0, 0], np.cumsum(terms[::-1])[::-1], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dS0[0, 0], sum(np.exp(G[t]) * np.outer(q[0, 0, t], w[0, 0, t])
                                              for t in range(T)), rtol=1e-12)
    for t in range(T):
        np.testing.assert_allclose(dq[0, 0, t], np.exp(G[t]) * s0 @ w[0, 0, t], rtol=1e-12)
    assert np.max(np.abs(dvv)) == 0.0


def test_packed_equals_separate_calls():
    q, k, v, g, eta, do, rng = _case(21, 1, 2, 150, 4, 3)
    cu = [0, 64, 65, 150]
    S0 = rng.standard_normal((3, 2, 4, 3))
    dS_T = rng.standard_normal((3, 2, 4, 3))
    packed = kbo.kla_backward(q, k, v, g, eta, 1e-6, do, dS_T, S0, cu_seqlens=cu)
    for n in range(3):
        t0, t1 = cu[n], cu[n + 1]
        sl = (slice(None), slice(None), slice(t0, t1))
        sep = kbo.kla_backward(q[sl], k[sl], v[sl], g[sl], eta[sl], 1e-6, do[sl],
                               dS_T[n:n + 1], S0[n:n + 1])
        for a, b in zip(packed[:5], sep[:5]):
            np.testing.assert_array_equal(a[sl], b)
        np.testing.assert_array_equal(packed[5][n], sep[5][0])


def test_linear_in_upstream_gradients():
    q, k, v, g, eta, do, rng = _case(22, 1, 2, 20, 3, 3)
    S0 = rng.standard_normal((1, 2, 3, 3))
    d1, d2 = rng.standard_normal((1, 2, 3, 3)), rng.standard_normal((1, 2, 3, 3))
    do2 = rng.standard_normal(do.shape)
    a = kbo.kla_backward(q, k, v, g, eta, 1e-6, do, d1, S0)
    b = kbo.kla_backward(q, k, v, g, eta, 1e-6, do2, d2, S0)
    c = kbo.kla_backward(q, k, v, g, eta, 1e-6, 2 * do - do2, 2 * d1 - d2, S0)
    for x, y, z in zip(a, b, c):
        np.testing.assert_allclose(z, 2 * x - y, rtol=1e-9, atol=1e-11 * np.max(np.abs(x)))


_MUTANTS = [
    ("dS_dec = dS - kt[:, :, None] * de[:, None, :]", "dS_dec = dS + kt[:, :, None] * de[:, None, :]"),
    ("gg[:, t] = alpha[:, t] * dalpha", "gg[:, t] = dalpha"),
    ("dkt -= (2.0 * coef[:, t]", "dkt -= (1.0 * coef[:, t]"),
    ("gq[:, t] = np.einsum(\"hij,hj->hi\", S_t, dot)", "gq[:, t] = np.einsum(\"hij,hj->hi\", S_prev, dot)"),
    ("dkt -= np.einsum(\"hij,hj->hi\", S_dec, de)", "dkt -= np.einsum(\"hij,hj->hi\", S_prev, de)"),
    ("dS = alpha[:, t, None, None] * dS_dec", "dS = dS_dec"),
    ("dS += qt[:, :, None] * dot[:, None, :]", "dS += dot[:, None, :].sum() * qt[:, :, None]"),
    ("dalpha = np.einsum(\"hij,hij->h\", S_prev, dS_dec)", "dalpha = np.einsum(\"hij,hij->h\", S_prev, dS)"),
]


@pytest.mark.parametrize("old,new", _MUTANTS)
def test_mutants_fail_the_fd_pin(old, new):
    src = inspect.getsource(kbo)
    assert src.count(old) == 1, old
    mod = types.ModuleType("kbo_mutant")
    exec(compile(src.replace(old, new), "kbo_mutant", "exec"), mod.__dict__)
    q, k, v, g, eta, do, rng = _case(31, 1, 1, 6, 3, 2)
    S0 = rng.standard_normal((1, 1, 3, 2))
    dS_T = rng.standard_normal((1, 1, 3, 2))
    with pytest.raises(AssertionError):
        _fd_check(kla_forward, mod.kla_backward, q, k, v, g, eta, 1e-3, do, dS_T, S0, None)
