"""The seeded input generator: determinism, shapes and the stated distributions."""

import math

import numpy as np
import torch

from gated_delta_rule_kla_amd import inputs


def test_deterministic_and_seed_sensitive():
    a = inputs.make_prefill(B=1, H=2, T=33, dk=16, dv=8, seed=3)
    b = inputs.make_prefill(B=1, H=2, T=33, dk=16, dv=8, seed=3)
    c = inputs.make_prefill(B=1, H=2, T=33, dk=16, dv=8, seed=4)
    for f in ("q", "k", "v", "g", "eta"):
        assert torch.equal(getattr(a, f), getattr(b, f))
    assert not torch.equal(a.q, c.q)


def test_shapes_dtypes_and_ranges():
    x = inputs.prefill_config(1, H=2, T=256, B=1)
    assert x.q.shape == (1, 2, 256, 128) and x.q.dtype == torch.bfloat16
    assert x.g.shape == (1, 2, 256)
    assert (x.g.float() < 0).all()                    # log-decay is negative
    assert ((x.eta.float() > 0) & (x.eta.float() < 1)).all()
    assert x.eps == float(np.float32(1e-6))
    assert x.initial_state is None and x.cu_seqlens is None


def test_key_norm_spread():
    # ln(norm) has std ~ sigma_k around ln(sqrt(dk))
    x = inputs.make_prefill(B=1, H=4, T=4096, dk=128, dv=16, sigma_k=1.0, seed=2,
                            dtype=torch.float32)
    ln = torch.log(x.k.norm(dim=-1)).flatten().numpy()
    assert abs(ln.std() - 1.0) < 0.05
    assert abs(ln.mean() - math.log(math.sqrt(128))) < 0.05


def test_varlen_config_lengths():
    x = inputs.prefill_config(4, H=1)
    cu = x.cu_seqlens.numpy()
    L = np.diff(cu)
    assert len(L) == 32 and L.min() >= 512 and L.max() <= 16384
    assert cu[0] == 0 and cu[-1] == x.q.shape[2]
    assert x.initial_state.shape == (32, 1, 128, 128)
    assert abs(float(x.initial_state.std()) - 0.02) < 0.001


def test_decode_inputs():
    d = inputs.make_decode(N=4, H=2, dk=16, dv=8, steps=5, seed=1)
    assert d.q.shape == (5, 4, 2, 16) and d.v.shape == (5, 4, 2, 8) and d.g.shape == (5, 4, 2)
    assert d.state.shape == (4, 2, 16, 8) and d.state.dtype == torch.float32
