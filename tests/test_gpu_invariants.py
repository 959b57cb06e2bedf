"""GPU invariants of the prefill that hold whatever the oracle says (HIP path against itself).

* Split and resume: prefill of tokens [0, t) and then of [t, T) from the state it returned
  equals one prefill of [0, T), for a t that is not a multiple of the chunk (the second call's
  chunks start at t, so the two runs use different chunk boundaries).
* A packed batch equals one call per sequence: chunks start at each sequence's first token
  either way.
* State columns are independent: a call with dv columns equals calls on column slices of v and
  of the initial state, whatever column tiling each call's grid picks.

bf16 calls run bf16 MFMA products over fp32 state; results that take different rounding paths
(split and resume) are compared to the bf16 bar (2e-2 x max|.|), the others to 1e-5."""

import numpy as np
import pytest
import torch

from gated_delta_rule_kla_amd import inputs, kla

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = torch.device("cuda:0")
f = inputs.to_f64


def rel(a, b):
    a, b = f(a), f(b)
    assert np.isfinite(a).all() and np.isfinite(b).all()
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-30))


def fwd(q, k, v, g, eta, eps, s0=None, cu=None, cuh=None, chunk=64):
    o, S = kla.chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV), eta.to(DEV), eps,
                         None if s0 is None else s0.to(DEV), None if cu is None else cu.to(DEV),
                         chunk=chunk, cu_seqlens_host=cuh)
    torch.cuda.synchronize()
    return o.cpu(), S.cpu()


@pytest.mark.parametrize("dtype,chunk,dk,dv,t,tol", [
    (torch.bfloat16, 64, 128, 128, 100, 2e-2),
    (torch.bfloat16, 64, 64, 256, 333, 2e-2),
    (torch.float32, 16, 32, 16, 37, 1e-4),
])
def test_split_and_resume_mid_chunk(dtype, chunk, dk, dv, t, tol):
    x = inputs.make_prefill(B=2, H=3, T=500, dk=dk, dv=dv, chunk=chunk, dtype=dtype, s0_std=0.02, seed=7301,
                            name="split")
    print(f"case split t={t} {x.dims} chunk={chunk}", flush=True)
    a = lambda z: z[:, :, :t]
    b = lambda z: z[:, :, t:]
    o, S = fwd(x.q, x.k, x.v, x.g, x.eta, x.eps, x.initial_state, chunk=chunk)
    o1, S1 = fwd(a(x.q), a(x.k), a(x.v), a(x.g), a(x.eta), x.eps, x.initial_state, chunk=chunk)
    o2, S2 = fwd(b(x.q), b(x.k), b(x.v), b(x.g), b(x.eta), x.eps, S1, chunk=chunk)
    eo, es = rel(torch.cat([o1, o2], dim=2), o), rel(S2, S)
    print(f"  err_o={eo:.3e} err_S={es:.3e} (tol {tol})")
    assert eo <= tol and es <= tol, (eo, es)


def test_packed_batch_equals_one_call_per_sequence():
    lengths = [70, 0, 130, 64, 1, 257]
    x = inputs.make_prefill(H=4, dk=128, dv=128, chunk=64, s0_std=0.02, lengths=lengths, seed=7302,
                            name="packed")
    print(f"case packed lengths={lengths}", flush=True)
    o, S = fwd(x.q, x.k, x.v, x.g, x.eta, x.eps, x.initial_state, x.cu_seqlens, x.cu_seqlens)
    cu = x.cu_seqlens.tolist()
    for n in range(len(lengths)):
        t0, t1 = cu[n], cu[n + 1]
        s0 = x.initial_state[n:n + 1]
        if t1 == t0:
            assert torch.equal(S[n], s0[0]), n  # an empty sequence keeps its state
            continue
        sl = lambda z: z[:, :, t0:t1]
        on, Sn = fwd(sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.eta), x.eps, s0)
        eo, es = rel(on, o[:, :, t0:t1]), rel(Sn, S[n:n + 1])
        print(f"  sequence {n} ({t1 - t0} tokens): err_o={eo:.1e} err_S={es:.1e}")
        assert eo <= 1e-5 and es <= 1e-5, (n, eo, es)


@pytest.mark.parametrize("B,H,T,dv,split", [(1, 2, 300, 128, 64), (1, 16, 640, 256, 64), (2, 3, 200, 96, 32)])
def test_state_columns_are_independent(B, H, T, dv, split):
    x = inputs.make_prefill(B=B, H=H, T=T, dk=128, dv=dv, chunk=64, s0_std=0.02, seed=7303, name="columns")
    print(f"case columns {x.dims} split={split}", flush=True)
    o, S = fwd(x.q, x.k, x.v, x.g, x.eta, x.eps, x.initial_state)
    for c0 in range(0, dv, split):
        c = slice(c0, c0 + split)
        oc, Sc = fwd(x.q, x.k, x.v[..., c].contiguous(), x.g, x.eta, x.eps,
                     x.initial_state[..., c].contiguous())
        eo, es = rel(oc, o[..., c]), rel(Sc, S[..., c])
        print(f"  columns {c0}..{c0 + split - 1}: err_o={eo:.1e} err_S={es:.1e}")
        assert eo <= 1e-5 and es <= 1e-5, (c0, eo, es)
