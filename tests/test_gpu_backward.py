"""GPU parity of the backward pass (kla_chunk_bwd, kla_gdn_chunk_bwd) against
the fp64 gradient oracle, on the same seeded inputs and upstream gradients.

Criterion per gradient tensor, as for the forward: max|gpu - ref| / max|ref|
<= 2e-2 for bf16 inputs (fp32 accumulation; dq, dk, dv are returned in bf16),
<= 1e-4 for the fp32 debug build.  Small cases span several chunks and a
ragged tail and are compared element by element; the benchmark-size workload
is compared on a sampled head.
"""

import numpy as np
import pytest
import torch

from gated_delta_rule_kla_amd import inputs, kla
from oracle import gdn_backward, kla_backward

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = torch.device("cuda:0")
TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}
f = inputs.to_f64
NAMES = ("dq", "dk", "dv", "dg", "deta", "dS0")


def rel_err(got, ref):
    got, ref = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    assert np.isfinite(got).all(), "non-finite GPU output"
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def run_bwd(x, do, ds, gdn_beta=None, need_dinitial=True):
    s0 = None if x.initial_state is None else x.initial_state.to(DEV)
    cu = None if x.cu_seqlens is None else x.cu_seqlens.to(DEV)
    dsd = None if ds is None else ds.to(DEV)
    if gdn_beta is None:
        out = kla.chunk_bwd(x.q.to(DEV), x.k.to(DEV), x.v.to(DEV), x.g.to(DEV), x.eta.to(DEV), do.to(DEV),
                            x.eps, s0, dsd, cu, chunk=x.chunk, cu_seqlens_host=x.cu_seqlens,
                            need_dinitial=need_dinitial)
    else:
        out = kla.gdn_chunk_bwd(x.q.to(DEV), x.k.to(DEV), x.v.to(DEV), x.g.to(DEV), gdn_beta.to(DEV),
                                do.to(DEV), s0, dsd, cu, chunk=x.chunk, cu_seqlens_host=x.cu_seqlens,
                                need_dinitial=need_dinitial)
    torch.cuda.synchronize()
    return [None if t is None else t.cpu() for t in out]


def oracle_bwd(x, do, ds, gdn_beta=None, heads=None):
    cu = None if x.cu_seqlens is None else x.cu_seqlens.tolist()
    if gdn_beta is None:
        return kla_backward(f(x.q), f(x.k), f(x.v), f(x.g), f(x.eta), x.eps, f(do), f(ds),
                            f(x.initial_state), cu_seqlens=cu, heads=heads)
    return gdn_backward(f(x.q), f(x.k), f(x.v), f(x.g), f(gdn_beta), f(do), f(ds), f(x.initial_state),
                        cu_seqlens=cu, heads=heads)


def check_bwd(x, seed, gdn_beta=None, ds_std=1.0):
    do, ds = inputs.make_upstream(x, seed, ds_std=ds_std)
    got = run_bwd(x, do, ds, gdn_beta)
    ref = oracle_bwd(x, do, ds, gdn_beta)
    tol = TOL[x.q.dtype]
    errs = {}
    for name, a, b in zip(NAMES, got, ref):
        errs[name] = rel_err(f(a), b)
    print(f"{x.name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()) + f" tol={tol}")
    assert all(v <= tol for v in errs.values()), errs
    return got


def test_bwd_tiny_fp32_workload():
    """The tiny fp32 workload (B=1 H=1 T=256 dk=dv=16 chunk 16), with an initial state."""
    x = inputs.make_prefill(B=1, H=1, T=256, dk=16, dv=16, chunk=16, dtype=torch.float32, s0_std=0.5,
                            seed=1000, name="bwd-fp32-tiny")
    check_bwd(x, 1)


@pytest.mark.parametrize("dk,dv,T", [(32, 48, 333), (16, 16, 64), (32, 32, 1)])
def test_bwd_fp32_chunk64(dk, dv, T):
    x = inputs.make_prefill(B=2, H=2, T=T, dk=dk, dv=dv, chunk=64, dtype=torch.float32, s0_std=0.3,
                            seed=T + 7, name=f"bwd-fp32-c64-{dk}x{dv}-T{T}")
    check_bwd(x, T)


@pytest.mark.parametrize("dk", [16, 64, 128])
def test_bwd_fp32_chunk16(dk):
    x = inputs.make_prefill(B=1, H=3, T=100, dk=dk, dv=32, chunk=16, dtype=torch.float32, s0_std=0.1,
                            seed=dk + 3, name=f"bwd-fp32-c16-dk{dk}")
    check_bwd(x, dk)


@pytest.mark.parametrize("B,H,T,dk,dv", [
    (1, 2, 300, 128, 128),     # several chunks, ragged tail
    (1, 2, 273, 128, 256),     # wide values
    (2, 2, 129, 64, 64),       # dk 64
    (1, 1, 64, 128, 32),       # exactly one chunk
    (1, 1, 7, 128, 128),       # shorter than one chunk
    (1, 3, 200, 128, 48),      # dv not a multiple of 32: 16-column scan slices
    (2, 1, 90, 64, 16),        # a single 16-column slice, dk 64
])
def test_bwd_bf16(B, H, T, dk, dv):
    x = inputs.make_prefill(B=B, H=H, T=T, dk=dk, dv=dv, chunk=64, s0_std=0.02, seed=B * H + T + 1,
                            name=f"bwd-bf16-{B}x{H}x{T}-{dk}x{dv}")
    check_bwd(x, T + 1)


def test_bwd_bf16_heavy_tailed_keys_slow_decay():
    x = inputs.make_prefill(B=1, H=2, T=600, dk=128, dv=128, chunk=64, sigma_k=1.0, g_scale=0.1,
                            eta_mu=1.0, seed=21, name="bwd-heavy")
    check_bwd(x, 21)


def test_bwd_varlen_with_empty_and_tiny_sequences():
    x = inputs.make_prefill(H=3, dk=128, dv=128, chunk=64, s0_std=0.02,
                            lengths=[0, 1, 63, 64, 65, 200, 17, 0], seed=22, name="bwd-varlen")
    check_bwd(x, 22)


def test_bwd_varlen_fp32():
    x = inputs.make_prefill(H=2, dk=32, dv=16, chunk=16, dtype=torch.float32, s0_std=0.2,
                            lengths=[5, 0, 16, 33, 1], seed=23, name="bwd-varlen-fp32")
    check_bwd(x, 23)


def test_bwd_without_state_gradients():
    """No initial state, no upstream state gradient, dS0 not requested."""
    x = inputs.make_prefill(B=1, H=2, T=150, dk=128, dv=64, chunk=64, seed=24, name="bwd-nostate")
    do, _ = inputs.make_upstream(x, 24, ds_std=None)
    got = run_bwd(x, do, None, need_dinitial=False)
    ref = oracle_bwd(x, do, None)
    assert got[5] is None
    for name, a, b in zip(NAMES[:5], got[:5], ref[:5]):
        assert rel_err(f(a), b) <= TOL[torch.bfloat16], name


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_bwd_gated_delta_rule(dtype):
    """Unit-norm keys with beta = eta in (0, 1), where the gated delta rule is a contraction."""
    chunk = 64 if dtype == torch.bfloat16 else 16
    dk = 128 if dtype == torch.bfloat16 else 32
    x = inputs.unit_keys(inputs.make_prefill(B=1, H=2, T=200, dk=dk, dv=64, chunk=chunk, dtype=dtype,
                                             s0_std=0.05, seed=25, name=f"bwd-gdn-{dtype}"))
    check_bwd(x, 26, gdn_beta=x.eta)


def test_bwd_gdn_with_the_kaczmarz_step_matches_kla():
    """beta_t = eta_t / (||k_t||^2 + eps) through the gated-delta-rule backward gives KLA's dq, dv,
    dg and dS0, and dbeta / (||k||^2 + eps) = deta (fp32 debug build)."""
    x = inputs.make_prefill(B=1, H=2, T=200, dk=32, dv=16, chunk=16, dtype=torch.float32, s0_std=0.05,
                            seed=28, name="bwd-gdn-vs-kla")
    do, ds = inputs.make_upstream(x, 28)
    den = (x.k * x.k).sum(-1) + x.eps
    beta = (x.eta / den).to(torch.float32)
    a = run_bwd(x, do, ds)
    b = run_bwd(x, do, ds, gdn_beta=beta)
    for i in (0, 2, 3, 5):
        assert rel_err(f(b[i]), f(a[i])) <= 1e-4, NAMES[i]
    assert rel_err(f(b[4]) / f(den), f(a[4])) <= 1e-4


def test_bwd_large_grid_sequential_scans():
    """A grid too large for the two state passes to run side by side (2 x 8 sequences x 17 heads x
    2 slices of 64 columns > one workgroup per CU): they run one after the other on the caller's
    stream with 32-column slices.  Compared on three sampled heads of every sequence."""
    x = inputs.make_prefill(B=8, H=17, T=150, dk=128, dv=128, chunk=64, s0_std=0.02, seed=2917,
                            name="bwd-large-grid")
    do, ds = inputs.make_upstream(x, 2917)
    got = run_bwd(x, do, ds)
    heads = [0, 9, 16]
    ref = oracle_bwd(x, do, ds, heads=heads)
    for name, a, b in zip(NAMES, got, ref):
        e = rel_err(f(a)[:, heads], b[:, heads])
        assert e <= TOL[torch.bfloat16], (name, e)


def test_bwd_deterministic():
    x = inputs.make_prefill(B=1, H=2, T=200, dk=128, dv=128, chunk=64, s0_std=0.02, seed=27, name="det")
    do, ds = inputs.make_upstream(x, 27)
    a = run_bwd(x, do, ds)
    b = run_bwd(x, do, ds)
    for u, w in zip(a, b):
        assert torch.equal(u, w)


def test_bwd_full_workload_sampled_head():
    """The benchmark's backward workload B=4 H=16 T=4096 dk=dv=128 bf16, compared on head 5 of
    every batch row (the oracle computes one head on its own)."""
    x = inputs.prefill_config(1)
    do, ds = inputs.make_upstream(x, 101)
    got = run_bwd(x, do, ds)
    ref = oracle_bwd(x, do, ds, heads=[5])
    for name, a, b in zip(NAMES, got, ref):
        ga = f(a)[:, 5] if name != "dS0" else f(a)[:, 5]
        e = rel_err(ga, b[:, 5])
        print(f"full {name}: {e:.2e}")
        assert e <= TOL[torch.bfloat16], (name, e)
