"""GPU parity of the segment-parallel prefill (kla_chunk_fwd_seg) against the fp64 oracle.

Each case cuts sequences into segments of a few chunks, so that segment boundaries fall inside
sequences, next to ragged tails and empty sequences, and compares o and the final states
element by element with the oracle's token recurrence (the bf16 bar 2e-2 x max|ref|, the fp32
debug bar 1e-4), and with the same call unsegmented.  The paths covered: bf16 64-column tiles
with the MFMA correction (dk 128 and 64), bf16 16- and 32-column tiles with the fp32
correction, fp32 chunk 16 and chunk 64, packed batches with empty and one-token sequences,
initial states, a segment length that leaves one segment per sequence, the library's own
choice on a grid of few long sequences, the gated delta rule (update coefficient given) on the
same choice, and the unsegmented fallback for a workspace without room for the segments.
"""

import numpy as np
import pytest
import torch

from gated_delta_rule_kla_amd import inputs, kla
from oracle import kla_forward

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = torch.device("cuda:0")
TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}
f = inputs.to_f64


def rel_err(got, ref):
    got, ref = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    assert np.isfinite(got).all(), "non-finite GPU output"
    return float(np.abs(got - ref).max() / np.abs(ref).max())


def run(x, seg_chunks):
    s0 = None if x.initial_state is None else x.initial_state.to(DEV)
    cu = None if x.cu_seqlens is None else x.cu_seqlens.to(DEV)
    o, S = kla.chunk_fwd(x.q.to(DEV), x.k.to(DEV), x.v.to(DEV), x.g.to(DEV), x.eta.to(DEV), x.eps, s0, cu,
                         chunk=x.chunk, cu_seqlens_host=x.cu_seqlens, seg_chunks=seg_chunks)
    torch.cuda.synchronize()
    return o.cpu(), S.cpu()


def check(x, seg_chunks):
    print(f"case {x.name} seg_chunks={seg_chunks} dims={x.dims}", flush=True)
    o, S = run(x, seg_chunks)
    cu = None if x.cu_seqlens is None else x.cu_seqlens.tolist()
    o_r, S_r = kla_forward(f(x.q), f(x.k), f(x.v), f(x.g), f(x.eta), x.eps, f(x.initial_state), cu_seqlens=cu)
    tol = TOL[x.q.dtype]
    eo, es = rel_err(f(o), o_r), rel_err(f(S), S_r)
    o0, S0 = run(x, 0)
    do, ds = rel_err(f(o), f(o0)), rel_err(f(S), f(S0))
    print(f"  vs oracle err_o={eo:.3e} err_S={es:.3e}; vs unsegmented {do:.3e} {ds:.3e} (tol {tol})")
    assert eo <= tol and es <= tol, (eo, es)
    assert do <= tol and ds <= tol, (do, ds)


@pytest.mark.parametrize("seg_chunks", [1, 3, 4])
def test_seg_dense_bf16_four_tiles_dk128(seg_chunks):
    x = inputs.make_prefill(B=2, H=3, T=700, dk=128, dv=128, chunk=64, s0_std=0.02, seed=5101,
                            name="seg-dense-dk128")
    check(x, seg_chunks)


def test_seg_dense_bf16_dk64_dv256():
    x = inputs.make_prefill(B=1, H=2, T=1000, dk=64, dv=256, chunk=64, sigma_k=1.0, g_scale=0.1, eta_mu=1.0,
                            seed=5102, name="seg-dense-dk64-dv256")
    check(x, 5)


def test_seg_packed_bf16_with_empty_and_tiny_sequences():
    x = inputs.make_prefill(H=2, dk=128, dv=64, chunk=64, lengths=[70, 0, 130, 600, 64, 1, 333], s0_std=0.02,
                            seed=5103, name="seg-packed")
    check(x, 2)


def test_seg_packed_bf16_dk64():
    x = inputs.make_prefill(H=3, dk=64, dv=128, chunk=64, lengths=[500, 257, 0, 900], seed=5104,
                            name="seg-packed-dk64")
    check(x, 3)


@pytest.mark.parametrize("dv", [48, 96])
def test_seg_bf16_narrow_tiles(dv):
    # dv not a multiple of 64: 16- or 32-column tiles and the fp32 correction
    x = inputs.make_prefill(B=1, H=2, T=450, dk=128, dv=dv, chunk=64, s0_std=0.02, seed=5105,
                            name=f"seg-bf16-dv{dv}")
    check(x, 2)


def test_seg_fp32_chunk16():
    x = inputs.make_prefill(B=2, H=2, T=300, dk=32, dv=16, chunk=16, dtype=torch.float32, s0_std=0.02,
                            seed=5106, name="seg-fp32-c16")
    check(x, 4)


def test_seg_fp32_chunk64_packed():
    x = inputs.make_prefill(H=2, dk=16, dv=32, chunk=64, dtype=torch.float32, lengths=[200, 0, 390, 65],
                            s0_std=0.02, seed=5107, name="seg-fp32-c64-packed")
    check(x, 2)


def test_seg_longer_than_every_sequence_is_one_segment():
    x = inputs.make_prefill(B=2, H=2, T=300, dk=128, dv=128, chunk=64, s0_std=0.02, seed=5108,
                            name="seg-one-segment")
    check(x, 100)


def test_seg_library_choice_on_few_long_sequences():
    """B=1 H=4 T=8192 dk=128 dv=256: 16 two-tile workgroups would leave the GPU idle, so
    kla_chunk_fwd cuts the 128 chunks into segments itself (its workspace query includes their
    buffers); the result matches the unsegmented call and, on two heads, the oracle."""
    x = inputs.make_prefill(B=1, H=4, T=8192, dk=128, dv=256, chunk=64, sigma_k=1.0, g_scale=0.1, eta_mu=1.0,
                            seed=5109, name="seg-auto")
    plain = kla.chunk_workspace_bytes(1, 4, 8192, 128, 256, seg_chunks=0)
    assert kla.chunk_workspace_bytes(1, 4, 8192, 128, 256) > plain  # the library's choice segments
    print(f"case {x.name} (library's choice)", flush=True)
    o, S = run(x, None)
    o0, S0 = run(x, 0)
    assert rel_err(f(o), f(o0)) <= 2e-2 and rel_err(f(S), f(S0)) <= 2e-2
    for h in (0, 3):
        o_r, S_r = kla_forward(f(x.q[:, h:h + 1]), f(x.k[:, h:h + 1]), f(x.v[:, h:h + 1]), f(x.g[:, h:h + 1]),
                               f(x.eta[:, h:h + 1]), x.eps)
        eo, es = rel_err(f(o[:, h:h + 1]), o_r), rel_err(f(S[:, h:h + 1]), S_r)
        print(f"  head {h}: err_o={eo:.3e} err_S={es:.3e}")
        assert eo <= 2e-2 and es <= 2e-2, (h, eo, es)


def test_seg_gdn_mode_and_the_unsegmented_fallback():
    """kla_gdn_chunk_fwd takes the same choice of segments (B=1 H=4 T=8192 dv=256: eight
    segments of 16 chunks); given a workspace of only the unsegmented size it runs unsegmented
    instead.  Both agree, and two heads match the gated-delta-rule oracle."""
    from oracle import gdn_forward
    x = inputs.unit_keys(inputs.make_prefill(B=1, H=4, T=8192, dk=128, dv=256, chunk=64, g_scale=0.1,
                                             seed=5110, name="seg-gdn"))
    full = kla.chunk_workspace_bytes(1, 4, 8192, 128, 256)
    plain = kla.chunk_workspace_bytes(1, 4, 8192, 128, 256, seg_chunks=0)
    assert full > plain > 0
    args = [t.to(DEV) for t in (x.q, x.k, x.v, x.g, x.eta)]
    print(f"case {x.name}: segmented, then a workspace of {plain} bytes", flush=True)
    o1, S1 = kla.gdn_chunk_fwd(*args, workspace=torch.empty(full, dtype=torch.uint8, device=DEV))
    o0, S0 = kla.gdn_chunk_fwd(*args, workspace=torch.empty(plain, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    o1, S1, o0, S0 = o1.cpu(), S1.cpu(), o0.cpu(), S0.cpu()
    assert rel_err(f(o1), f(o0)) <= 2e-2 and rel_err(f(S1), f(S0)) <= 2e-2
    for h in (0, 3):
        o_r, S_r = gdn_forward(f(x.q[:, h:h + 1]), f(x.k[:, h:h + 1]), f(x.v[:, h:h + 1]), f(x.g[:, h:h + 1]),
                               f(x.eta[:, h:h + 1]))
        for o, S in ((o1, S1), (o0, S0)):
            eo, es = rel_err(f(o[:, h:h + 1]), o_r), rel_err(f(S[:, h:h + 1]), S_r)
            print(f"  head {h}: err_o={eo:.3e} err_S={es:.3e}")
            assert eo <= 2e-2 and es <= 2e-2, (h, eo, es)


def test_seg_dv192_six_wave_correction():
    # dv = 192: the MFMA correction with six waves of two column tiles
    x = inputs.make_prefill(B=2, H=2, T=520, dk=128, dv=192, chunk=64, s0_std=0.02, seed=5111,
                            name="seg-dv192")
    check(x, 3)


def test_seg_final_state_aliases_initial_state():
    """The final state may be written over the initial state: the scan reads it for the first
    segments, and only the combine kernel, which runs after the scan, writes the final state."""
    x = inputs.make_prefill(B=2, H=3, T=600, dk=128, dv=128, chunk=64, s0_std=0.05, seed=5112,
                            name="seg-alias")
    args = [t.to(DEV) for t in (x.q, x.k, x.v, x.g, x.eta)]
    s0 = x.initial_state.to(DEV)
    print(f"case {x.name}: in place", flush=True)
    o_ref, S_ref = kla.chunk_fwd(*args, x.eps, s0.clone(), seg_chunks=2)
    s_inout = s0.clone()
    o_in, S_in = kla.chunk_fwd(*args, x.eps, s_inout, final_state=s_inout, seg_chunks=2)
    torch.cuda.synchronize()
    assert S_in.data_ptr() == s_inout.data_ptr()
    assert torch.equal(o_in.cpu(), o_ref.cpu()) and torch.equal(S_in.cpu(), S_ref.cpu())


def test_seg_more_segment_heads_than_a_grid_row_holds():
    """fp32 chunk 16, H=64, one chunk per segment over 1,100 chunks: 70,400 (segment, head)
    pairs, more than the 65,536 a launch grid's second dimension holds.  The correction
    takes them along the first dimension; every head matches the unsegmented call, and two
    heads match the oracle."""
    x = inputs.make_prefill(B=1, H=64, T=17600, dk=16, dv=16, chunk=16, dtype=torch.float32, s0_std=0.02,
                            seed=5113, name="seg-many")
    print(f"case {x.name} seg_chunks=1 dims={x.dims}", flush=True)
    o, S = run(x, 1)
    o0, S0 = run(x, 0)
    do, ds = rel_err(f(o), f(o0)), rel_err(f(S), f(S0))
    print(f"  vs unsegmented {do:.3e} {ds:.3e}")
    assert do <= 1e-4 and ds <= 1e-4, (do, ds)
    for h in (0, 63):
        o_r, S_r = kla_forward(f(x.q[:, h:h + 1]), f(x.k[:, h:h + 1]), f(x.v[:, h:h + 1]), f(x.g[:, h:h + 1]),
                               f(x.eta[:, h:h + 1]), x.eps, f(x.initial_state[:, h:h + 1]))
        eo, es = rel_err(f(o[:, h:h + 1]), o_r), rel_err(f(S[:, h:h + 1]), S_r)
        print(f"  head {h}: err_o={eo:.3e} err_S={es:.3e}")
        assert eo <= 1e-4 and es <= 1e-4, (h, eo, es)
