"""The oracle's chunkwise form and batch drivers against its recurrence.

The chunk solver is an exact reformulation of the token recurrence
([KLA] "Resumen Técnico: Atención Lineal Kaczmarz (KLA)",
gist.science/es/paper/2605.08587, §"Implementación": the block solver is kept
and only B = Diag(beta) changes), so it must agree to rounding.  The batch
drivers (fixed-length, packed varlen, decode) must agree with the
single-sequence recurrence they are built from.
"""

import numpy as np
import pytest
import torch

from gated_delta_rule_kla_amd import inputs
from oracle import kla_chunkwise, kla_decode_step, kla_forward, kla_recurrence


def _seq(seed, L, dk, dv, spread=1.0, g_scale=1.0, s0=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((L, dk))
    k = rng.standard_normal((L, dk)) * np.exp(spread * rng.standard_normal(L))[:, None]
    v = rng.standard_normal((L, dv))
    g = -g_scale * np.log1p(np.exp(rng.standard_normal(L)))
    eta = 1 / (1 + np.exp(-rng.standard_normal(L)))
    S0 = 0.5 * rng.standard_normal((dk, dv)) if s0 else None
    return q, k, v, g, eta, S0


@pytest.mark.parametrize("chunk", [1, 2, 3, 16, 64])
@pytest.mark.parametrize("L", [50, 64, 131])
def test_chunkwise_equals_recurrence(chunk, L):
    q, k, v, g, eta, S0 = _seq(100 + chunk + L, L, 8, 6, spread=1.0)
    o_r, S_r = kla_recurrence(q, k, v, g, eta, 1e-6, S0)
    o_c, S_c = kla_chunkwise(q, k, v, g, eta, 1e-6, S0, chunk)
    np.testing.assert_allclose(o_c, o_r, rtol=0, atol=1e-12 * np.abs(o_r).max())
    np.testing.assert_allclose(S_c, S_r, rtol=0, atol=1e-12 * np.abs(S_r).max())


def test_chunkwise_heavy_tailed_slow_decay():
    # the long-context workload's regime: key scale exp(N(0,1)), g = -0.1 softplus
    q, k, v, g, eta, S0 = _seq(7, 300, 16, 8, spread=1.0, g_scale=0.1, s0=False)
    eta = 1 / (1 + np.exp(-(np.random.default_rng(8).standard_normal(300) + 1.0)))
    o_r, S_r = kla_recurrence(q, k, v, g, eta, 1e-6)
    o_c, S_c = kla_chunkwise(q, k, v, g, eta, 1e-6, None, 64)
    np.testing.assert_allclose(o_c, o_r, rtol=0, atol=1e-11 * np.abs(o_r).max())
    np.testing.assert_allclose(S_c, S_r, rtol=0, atol=1e-11 * np.abs(S_r).max())


def test_chunk_intermediates():
    """Ut_r = beta_r e_r with e_r the residual of the recurrence at token r."""
    q, k, v, g, eta, S0 = _seq(9, 20, 5, 3)
    _, _, states = kla_recurrence(q, k, v, g, eta, 1e-6, S0, return_states=True)
    _, _, dumps = kla_chunkwise(q, k, v, g, eta, 1e-6, S0, 8, return_chunks=True)
    for c, d in enumerate(dumps):
        for r in range(len(d["beta"])):
            t = 8 * c + r
            e = v[t] - (np.exp(g[t]) * states[t]).T @ k[t]
            np.testing.assert_allclose(d["Ut"][r], d["beta"][r] * e, rtol=1e-11, atol=1e-13)
        n = len(d["beta"])
        np.testing.assert_allclose(np.diag(d["T"]), np.ones(n))
        assert np.all(np.triu(d["T"], 1) == 0)


def test_forward_fixed_length_matches_recurrence():
    x = inputs.make_prefill(B=2, H=3, T=70, dk=8, dv=4, dtype=torch.float32,
                            s0_std=0.3, seed=5)
    f = inputs.to_f64
    o, S = kla_forward(f(x.q), f(x.k), f(x.v), f(x.g), f(x.eta), x.eps, f(x.initial_state))
    for b in range(2):
        for h in range(3):
            o_r, S_r = kla_recurrence(f(x.q)[b, h], f(x.k)[b, h], f(x.v)[b, h], f(x.g)[b, h],
                                      f(x.eta)[b, h], x.eps, f(x.initial_state)[b, h])
            np.testing.assert_allclose(o[b, h], o_r, rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(S[b, h], S_r, rtol=1e-13, atol=1e-13)


def test_varlen_equals_separate_sequences():
    x = inputs.make_prefill(H=2, dk=8, dv=4, dtype=torch.float32, s0_std=0.2,
                            lengths=[5, 1, 17, 0, 33], seed=6)
    f = inputs.to_f64
    cu = x.cu_seqlens.tolist()
    o, S = kla_forward(f(x.q), f(x.k), f(x.v), f(x.g), f(x.eta), x.eps,
                       f(x.initial_state), cu_seqlens=cu)
    for n in range(len(cu) - 1):
        t0, t1 = cu[n], cu[n + 1]
        for h in range(2):
            o_r, S_r = kla_recurrence(f(x.q)[0, h, t0:t1], f(x.k)[0, h, t0:t1], f(x.v)[0, h, t0:t1],
                                      f(x.g)[0, h, t0:t1], f(x.eta)[0, h, t0:t1], x.eps,
                                      f(x.initial_state)[n, h])
            np.testing.assert_allclose(o[0, h, t0:t1], o_r, rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(S[n, h], S_r, rtol=1e-13, atol=1e-13)
    # the empty sequence hands its initial state straight through
    np.testing.assert_array_equal(S[3], f(x.initial_state)[3])


def test_split_and_resume():
    q, k, v, g, eta, S0 = _seq(21, 90, 6, 4)
    o, S = kla_recurrence(q, k, v, g, eta, 1e-6, S0)
    for cut in (1, 37, 64, 89):
        o1, S1 = kla_recurrence(q[:cut], k[:cut], v[:cut], g[:cut], eta[:cut], 1e-6, S0)
        o2, S2 = kla_chunkwise(q[cut:], k[cut:], v[cut:], g[cut:], eta[cut:], 1e-6, S1, 16)
        np.testing.assert_allclose(np.concatenate([o1, o2]), o, rtol=0, atol=1e-12 * np.abs(o).max())
        np.testing.assert_allclose(S2, S, rtol=0, atol=1e-12 * np.abs(S).max())


def test_decode_steps_equal_prefill():
    d = inputs.make_decode(N=3, H=2, dk=8, dv=4, steps=12, dtype=torch.float32, seed=8)
    f = inputs.to_f64
    S = f(d.state)
    outs = []
    for s in range(12):
        o, S = kla_decode_step(f(d.q)[s], f(d.k)[s], f(d.v)[s], f(d.g)[s], f(d.eta)[s], d.eps, S)
        outs.append(o)
    outs = np.stack(outs)            # [steps, N, H, dv]
    for n in range(3):
        for h in range(2):
            o_r, S_r = kla_recurrence(f(d.q)[:, n, h], f(d.k)[:, n, h], f(d.v)[:, n, h],
                                      f(d.g)[:, n, h], f(d.eta)[:, n, h], d.eps, f(d.state)[n, h])
            np.testing.assert_allclose(outs[:, n, h], o_r, rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(S[n, h], S_r, rtol=1e-13, atol=1e-13)


def test_heads_subset_matches_full():
    x = inputs.make_prefill(B=1, H=4, T=40, dk=8, dv=4, dtype=torch.float32, seed=9)
    f = inputs.to_f64
    o, S = kla_forward(f(x.q), f(x.k), f(x.v), f(x.g), f(x.eta), x.eps)
    o2, S2 = kla_forward(f(x.q), f(x.k), f(x.v), f(x.g), f(x.eta), x.eps, heads=[1, 3])
    np.testing.assert_array_equal(o2[:, [1, 3]], o[:, [1, 3]])
    assert np.isnan(o2[:, 0]).all()
