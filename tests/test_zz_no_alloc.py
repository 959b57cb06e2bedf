"""kla_chunk_fwd_noalloc (the entry point with a fixed per-GPU scratch buffer
instead of a caller workspace) against kla_chunk_fwd, through the C ABI.

The two run the same kernels, so their outputs must agree bit for bit.  Calls
come in a row on one GPU, each later one smaller than the one before, so a
call that depended on what an earlier call left in the shared buffer would
show; the oracle checks the first call's result as well.  One call is cut into
segments (the segment-parallel scan's buffers also live in the scratch)."""

import numpy as np
import pytest
import torch

from gated_delta_rule_kla_amd import inputs, kla
from oracle import kla_forward

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = torch.device("cuda:0")
f = inputs.to_f64


def _both(x):
    q, k, v, g, eta = (t.to(DEV) for t in (x.q, x.k, x.v, x.g, x.eta))
    s0 = None if x.initial_state is None else x.initial_state.to(DEV)
    cu = None if x.cu_seqlens is None else x.cu_seqlens.to(DEV)
    B, H, T, dk, dv = x.dims
    N = x.num_seqs
    o_s = torch.empty((B, H, T, dv), dtype=q.dtype, device=DEV)
    S_s = torch.empty((N, H, dk, dv), dtype=torch.float32, device=DEV)
    kla.chunk_fwd(q, k, v, g, eta, x.eps, s0, cu, chunk=x.chunk, cu_seqlens_host=x.cu_seqlens,
                  out=o_s, final_state=S_s, workspace="static")
    o_w, S_w = kla.chunk_fwd(q, k, v, g, eta, x.eps, s0, cu, chunk=x.chunk, cu_seqlens_host=x.cu_seqlens)
    torch.cuda.synchronize()
    return o_s.cpu(), S_s.cpu(), o_w.cpu(), S_w.cpu()


def test_noalloc_matches_workspace_entry_point_on_calls_in_a_row():
    # few long sequences: the library cuts them into segments (about 10 MB of scratch)
    seg = inputs.make_prefill(B=1, H=2, T=6400, dk=128, dv=256, chunk=64, sigma_k=1.0, g_scale=0.1,
                              seed=95, name="segmented")
    assert kla.chunk_workspace_bytes(1, 2, 6400, 128, 256) > kla.chunk_workspace_bytes(1, 2, 6400, 128, 256,
                                                                                       seg_chunks=0)
    assert kla.chunk_workspace_bytes(1, 2, 6400, 128, 256) < kla.NOALLOC_SCRATCH_BYTES
    cases = [
        inputs.prefill_config(1),                                          # 28.3 MB of scratch
        seg,
        inputs.make_prefill(B=2, H=3, T=333, dk=128, dv=128, chunk=64, s0_std=0.05, seed=91, name="mid"),
        inputs.make_prefill(H=2, dk=128, dv=64, chunk=64, s0_std=0.05, lengths=[5, 0, 130, 64], seed=92,
                            name="varlen"),
        inputs.make_prefill(B=1, H=1, T=40, dk=32, dv=16, chunk=16, dtype=torch.float32, seed=93,
                            name="fp32-small"),
    ]
    for i, x in enumerate(cases):
        o_s, S_s, o_w, S_w = _both(x)
        assert torch.equal(o_s, o_w) and torch.equal(S_s, S_w), x.name
        if i == 0:
            # sampled heads of the large call against the oracle as well
            for b, h in [(0, 0), (3, 15)]:
                o_r, S_r = kla_forward(f(x.q[b:b + 1, h:h + 1]), f(x.k[b:b + 1, h:h + 1]),
                                       f(x.v[b:b + 1, h:h + 1]), f(x.g[b:b + 1, h:h + 1]),
                                       f(x.eta[b:b + 1, h:h + 1]), x.eps)
                eo = np.abs(f(o_s[b, h]) - o_r[0, 0]).max() / np.abs(o_r).max()
                es = np.abs(f(S_s[b, h]) - S_r[0, 0]).max() / np.abs(S_r).max()
                assert eo <= 2e-2 and es <= 2e-2, (eo, es)
        else:
            cu = None if x.cu_seqlens is None else x.cu_seqlens.tolist()
            o_r, S_r = kla_forward(f(x.q), f(x.k), f(x.v), f(x.g), f(x.eta), x.eps, f(x.initial_state),
                                   cu_seqlens=cu)
            tol = 2e-2 if x.q.dtype == torch.bfloat16 else 1e-4
            assert np.abs(f(o_s) - o_r).max() <= tol * np.abs(o_r).max(), x.name
            assert np.abs(f(S_s) - S_r).max() <= tol * np.abs(S_r).max(), x.name


def test_noalloc_refuses_a_call_larger_than_its_buffer():
    x = inputs.make_prefill(B=1, H=1, T=64, dk=128, dv=16, chunk=64, seed=94)
    big = 4 * 64 * 128 * 6912  # B=4 H=64 T=8192 needs this much; refused before any launch
    assert kla.chunk_workspace_bytes(4, 64, 8192, 128, 128) == big > kla.NOALLOC_SCRATCH_BYTES
    q = torch.empty((4, 64, 8192, 128), dtype=torch.bfloat16, device=DEV)
    gz = torch.empty((4, 64, 8192), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(kla.KlaError) as ei:
        kla.chunk_fwd(q, q, q, gz, gz, 1e-6, workspace="static")
    assert ei.value.status == -10
    del q, gz
    # the buffer still serves a call that fits
    o_s, S_s, o_w, S_w = _both(x)
    assert torch.equal(o_s, o_w) and torch.equal(S_s, S_w)
