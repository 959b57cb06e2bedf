"""GPU parity of the general chunk kernel (the shapes the pipelined kernels are not
compiled for) and of the preconditioned variant (PGDN), through the C ABI,
against the fp64 oracles.

Criterion (per output tensor): max|gpu - ref| / max|ref| <= 2e-2 for bf16
inputs, <= 1e-4 for fp32 inputs.  Every element is compared; the shapes span
several chunks and a ragged tail.
"""

import numpy as np
import pytest
import torch

from gated_delta_rule_kla_amd import inputs, kla
from oracle import (GAIN_GIVEN, GAIN_KACZMARZ, gdn_forward, kla_forward, pgdn_decode_step, pgdn_forward)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = torch.device("cuda:0")
TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}
f = inputs.to_f64


def rel_err(got, ref):
    got, ref = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    assert np.isfinite(got).all(), "non-finite GPU output"
    return float(np.abs(got - ref).max() / np.abs(ref).max())


def _dev(x):
    return (None if t is None else t.to(DEV) for t in (x.q, x.k, x.v, x.g, x.eta, x.initial_state, x.cu_seqlens))


def run_kla(x, chunk):
    q, k, v, g, eta, s0, cu = _dev(x)
    o, S = kla.chunk_fwd(q, k, v, g, eta, x.eps, s0, cu, chunk=chunk, cu_seqlens_host=x.cu_seqlens)
    torch.cuda.synchronize()
    return o.cpu(), S.cpu()


def check_kla(x, chunk):
    o, S = run_kla(x, chunk)
    cu = None if x.cu_seqlens is None else x.cu_seqlens.tolist()
    o_r, S_r = kla_forward(f(x.q), f(x.k), f(x.v), f(x.g), f(x.eta), x.eps, f(x.initial_state), cu_seqlens=cu)
    tol = TOL[x.q.dtype]
    eo, es = rel_err(f(o), o_r), rel_err(f(S), S_r)
    print(f"{x.name} chunk {chunk}: err_o={eo:.3e} err_S={es:.3e} tol={tol}")
    assert eo <= tol and es <= tol, (eo, es)
    return o, S


# ------------------------------------------- shapes of the general kernel ----

@pytest.mark.parametrize("dtype,chunk,dk,dv,T", [
    (torch.bfloat16, 16, 128, 128, 277),   # bf16 chunk 16
    (torch.bfloat16, 16, 16, 16, 200),     # bf16 chunk 16, dk 16
    (torch.bfloat16, 64, 16, 16, 333),     # bf16 dk 16
    (torch.bfloat16, 64, 32, 256, 150),    # bf16 dk 32, wide values
    (torch.float32, 64, 128, 128, 290),    # fp32 chunk 64 at dk 128
    (torch.float32, 64, 64, 32, 100),
])
def test_general_shapes(dtype, chunk, dk, dv, T):
    x = inputs.make_prefill(B=2, H=2, T=T, dk=dk, dv=dv, chunk=chunk, dtype=dtype, s0_std=0.05,
                            seed=T + dk, name=f"general-{dtype}-c{chunk}-dk{dk}-dv{dv}")
    check_kla(x, chunk)


def test_general_varlen_and_empty_sequences():
    x = inputs.make_prefill(H=3, dk=128, dv=32, chunk=16, s0_std=0.05, lengths=[0, 1, 15, 16, 17, 70, 0],
                            seed=101, name="general-varlen")
    check_kla(x, 16)


def test_general_fp32_chunk64_dk128_heavy_tailed_keys():
    x = inputs.make_prefill(B=1, H=2, T=500, dk=128, dv=64, chunk=64, dtype=torch.float32, sigma_k=1.0,
                            g_scale=0.1, eta_mu=1.0, seed=102, name="general-fp32-heavy")
    check_kla(x, 64)


def test_bf16_chunk_size_invariance_16_vs_64():
    """The result does not depend on the chunk size: bf16 chunk 16 (general kernel)
    against chunk 64 (pipelined kernels) on the same inputs, to the bf16 tolerance."""
    x = inputs.make_prefill(B=2, H=2, T=300, dk=128, dv=128, chunk=64, s0_std=0.05, seed=103, name="inv-bf16")
    o64, S64 = run_kla(x, 64)
    o16, S16 = run_kla(x, 16)
    assert rel_err(f(o16), f(o64)) <= 2e-2 and rel_err(f(S16), f(S64)) <= 2e-2


def test_general_gdn_mode():
    x = inputs.unit_keys(inputs.make_prefill(B=1, H=2, T=150, dk=128, dv=64, chunk=16, s0_std=0.05, seed=104,
                                             name="general-gdn"))
    q, k, v, g, b, s0, _ = _dev(x)
    o, S = kla.gdn_chunk_fwd(q, k, v, g, b, s0, chunk=16)
    torch.cuda.synchronize()
    o_r, S_r = gdn_forward(f(x.q), f(x.k), f(x.v), f(x.g), f(x.eta), f(x.initial_state))
    assert rel_err(f(o.cpu()), o_r) <= 2e-2 and rel_err(f(S.cpu()), S_r) <= 2e-2


def test_general_edge_exact_projection_fp32():
    """eta = 1, eps = 0 on the general kernel (fp32, chunk 64, dk 128)."""
    import dataclasses
    x = inputs.make_prefill(B=1, H=2, T=200, dk=128, dv=32, chunk=64, dtype=torch.float32, sigma_k=1.0,
                            g_scale=0.05, s0_std=0.1, seed=105, name="general-proj")
    x = dataclasses.replace(x, eta=torch.ones_like(x.eta), eps=0.0)
    check_kla(x, 64)


# ------------------------------------------------------------------ PGDN ----

def _pgdn_inputs(seed, *, B=2, H=2, T=200, dk=64, dv=32, dtype=torch.bfloat16, lengths=None, unit=False):
    """Seeded inputs with per-coordinate key scales exp(-1 .. 1) (so the
    preconditioner has something to correct) and an initial accumulator.  With
    ``unit`` every scaled key is then normalised to length 1: with a given
    coefficient beta in (0, 1) that is the regime in which the gated delta rule
    is contractive (on keys of length ~10 it diverges, in the oracle too)."""
    import dataclasses
    x = inputs.make_prefill(B=B, H=H, T=T, dk=dk, dv=dv, chunk=64, dtype=dtype, s0_std=0.05, seed=seed,
                            lengths=lengths)
    rng = np.random.default_rng(seed + 1)
    sc = torch.from_numpy(np.exp(np.linspace(-1.0, 1.0, dk)))
    k = x.k.to(torch.float64) * sc
    if unit:
        k = k / torch.linalg.vector_norm(k, dim=-1, keepdim=True).clamp_min(1e-30)
    x = dataclasses.replace(x, k=k.to(dtype))
    N = x.num_seqs
    acc0 = torch.from_numpy(np.abs(rng.standard_normal((N, H, dk))).astype(np.float32) * 5.0)
    return x, acc0


def run_pgdn(x, acc0, gain, band, chunk):
    q, k, v, g, c, s0, cu = _dev(x)
    o, S, A = kla.pgdn_chunk_fwd(q, k, v, g, c, x.eps, gain, band, s0, None if acc0 is None else acc0.to(DEV), cu,
                                 chunk=chunk, cu_seqlens_host=x.cu_seqlens)
    torch.cuda.synchronize()
    return o.cpu(), S.cpu(), A.cpu()


def check_pgdn(x, acc0, gain, band, chunk):
    o, S, A = run_pgdn(x, acc0, gain, band, chunk)
    cu = None if x.cu_seqlens is None else x.cu_seqlens.tolist()
    gi = GAIN_GIVEN if gain == "given" else GAIN_KACZMARZ
    o_r, S_r, A_r = pgdn_forward(f(x.q), f(x.k), f(x.v), f(x.g), f(x.eta), x.eps, gi, band, f(x.initial_state),
                                 f(acc0), cu_seqlens=cu)
    tol = TOL[x.q.dtype]
    eo, es, ea = rel_err(f(o), o_r), rel_err(f(S), S_r), rel_err(f(A), A_r)
    print(f"pgdn {x.q.dtype} {gain} band {band} chunk {chunk}: err_o={eo:.3e} err_S={es:.3e} err_A={ea:.3e}")
    assert eo <= tol and es <= tol and ea <= 1e-4, (eo, es, ea)


@pytest.mark.parametrize("gain", ["given", "kaczmarz"])
@pytest.mark.parametrize("dtype,chunk,dk", [(torch.bfloat16, 64, 128), (torch.bfloat16, 64, 64), (torch.bfloat16, 16, 64),
                                             (torch.float32, 64, 32), (torch.float32, 16, 128)])
def test_pgdn_prefill(gain, dtype, chunk, dk):
    x, acc0 = _pgdn_inputs(200 + dk + chunk, dk=dk, dtype=dtype, unit=gain == "given")
    check_pgdn(x, acc0, gain, 1.5, chunk)


@pytest.mark.parametrize("gain", ["given", "kaczmarz"])
def test_pgdn_prefill_two_column_tiles(gain):
    """Enough (sequence, head) pairs for 32-column workgroups in the pipelined PGDN scan:
    B=8 x H=16 x dv=64, bf16, chunk 64, dk 128, ragged tail."""
    x, acc0 = _pgdn_inputs(230, B=8, H=16, T=130, dk=128, dv=64, unit=gain == "given")
    check_pgdn(x, acc0, gain, 1.5, 64)


def test_pgdn_prefill_varlen_no_initial_accumulator():
    x, _ = _pgdn_inputs(210, H=3, dk=128, dv=64, lengths=[0, 1, 63, 64, 65, 130, 0])
    check_pgdn(x, None, "kaczmarz", 2.0, 64)


def test_pgdn_band_one_is_the_gated_delta_rule():
    """band = 1: p = 1, so PGDN with the given gain is GDN (the pipelined kernels' GDN entry)."""
    x, acc0 = _pgdn_inputs(211, dk=128, dv=64, unit=True)
    o, S, _ = run_pgdn(x, acc0, "given", 1.0, 64)
    q, k, v, g, b, s0, _ = _dev(x)
    o_g, S_g = kla.gdn_chunk_fwd(q, k, v, g, b, s0, chunk=64)
    torch.cuda.synchronize()
    assert rel_err(f(o), f(o_g.cpu())) <= 2e-2 and rel_err(f(S), f(S_g.cpu())) <= 2e-2


def test_pgdn_exact_projection_fp32():
    """Kaczmarz gain with eta = 1, eps = 0: the preconditioned write still interpolates."""
    import dataclasses
    x, acc0 = _pgdn_inputs(212, B=1, dk=64, dv=32, dtype=torch.float32)
    x = dataclasses.replace(x, eta=torch.ones_like(x.eta), eps=0.0)
    check_pgdn(x, acc0, "kaczmarz", 1.5, 64)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("gain", ["given", "kaczmarz"])
def test_pgdn_decode(dtype, gain):
    d = inputs.make_decode(N=3, H=2, dk=128, dv=96, steps=5, dtype=dtype, seed=213)
    if gain == "given":
        d = inputs.unit_keys(d)
    rng = np.random.default_rng(214)
    acc = torch.from_numpy(np.abs(rng.standard_normal((3, 2, 128))).astype(np.float32))
    st, ac = d.state.to(DEV), acc.to(DEV)
    S_r, A_r = f(d.state), f(acc)
    gi = GAIN_GIVEN if gain == "given" else GAIN_KACZMARZ
    for s in range(5):
        o = kla.pgdn_decode_step(d.q[s].to(DEV), d.k[s].to(DEV), d.v[s].to(DEV), d.g[s].to(DEV), d.eta[s].to(DEV),
                                 d.eps, st, ac, gain=gain, band=1.5)
        o_r, S_r, A_r = pgdn_decode_step(f(d.q[s]), f(d.k[s]), f(d.v[s]), f(d.g[s]), f(d.eta[s]), d.eps, gi, 1.5,
                                         S_r, A_r)
        assert rel_err(f(o.cpu()), o_r) <= TOL[dtype]
    torch.cuda.synchronize()
    assert rel_err(f(st.cpu()), S_r) <= TOL[dtype] and rel_err(f(ac.cpu()), A_r) <= 1e-4


def test_pgdn_prefill_then_decode_continues():
    x, acc0 = _pgdn_inputs(215, dk=64, dv=32, T=150)
    T0 = 140
    head = inputs.PrefillInputs(*(t[:, :, :T0].contiguous() for t in (x.q, x.k, x.v, x.g, x.eta)), x.eps,
                                x.initial_state, None, 64)
    _, S, A = run_pgdn(head, acc0, "kaczmarz", 1.5, 64)
    st, ac = S.to(DEV), A.to(DEV)
    outs = []
    for t in range(T0, 150):
        sl = lambda z: z[:, :, t].contiguous().to(DEV)
        outs.append(kla.pgdn_decode_step(sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.eta), x.eps, st, ac,
                                         gain="kaczmarz", band=1.5).cpu())
    torch.cuda.synchronize()
    o_r, S_r, A_r = pgdn_forward(f(x.q), f(x.k), f(x.v), f(x.g), f(x.eta), x.eps, GAIN_KACZMARZ, 1.5,
                                 f(x.initial_state), f(acc0))
    assert rel_err(f(torch.stack(outs, 2)), o_r[:, :, T0:]) <= 2e-2
    assert rel_err(f(st.cpu()), S_r) <= 2e-2 and rel_err(f(ac.cpu()), A_r) <= 1e-4
