"""Host logic of the segment-parallel prefill (kla_chunk_fwd_seg, kla_chunk_seg_workspace_bytes and
the library's own choice of segments in kla_chunk_fwd), and the algebra it rests on, checked on
the oracle.  No GPU: every kla_chunk_fwd_seg call here is rejected during validation."""

import ctypes

import numpy as np
import pytest

from gated_delta_rule_kla_amd import kla
from oracle import kla_forward

OK, E_NULL, E_SHAPE, E_UNSUP, E_WS = 0, -1, -2, -4, -7
FAKE = 0x7F0000000000


def up(x):
    return (x + 255) // 256 * 256


def _ws(seg=None, cu=None, cuh=None, N=2, B=2, H=4, T=100, dk=128, dv=128, chunk=64, dtype=0):
    L = kla.lib()
    if seg is None:
        return L.kla_chunk_workspace_bytes(cu, cuh, N, B, H, T, dk, dv, chunk, dtype)
    return L.kla_chunk_seg_workspace_bytes(cu, cuh, N, B, H, T, dk, dv, chunk, dtype, seg)


def _fwd_seg(seg, ws_bytes=1 << 40, q=FAKE, cu=None, cuh=None, N=2, B=2, H=4, T=100, dk=128, dv=128, chunk=64,
             dtype=0):
    return kla.lib().kla_chunk_fwd_seg(q, FAKE, FAKE, FAKE, FAKE, 1e-6, None, FAKE, FAKE, cu, cuh, N, B, H, T, dk,
                                       dv, chunk, dtype, seg, FAKE, ws_bytes, None)


def test_seg_workspace_layout():
    # kla_chunk_fwd's workspace, then (N + 1) ints, E [B, H, T, dk] in the element type, and per
    # (segment, head) the end state (dk x dv), the transfer map (dk x dk), the start state (dk x dv)
    base = _ws()
    assert _ws(seg=0) == base
    for L, nseg_per in [(1, 2), (2, 1), (5, 1)]:  # T=100: 2 chunks per sequence
        nsh = 2 * nseg_per * 4
        want = up(base) + up(3 * 4) + up(2 * 4 * 100 * 128 * 2) + 2 * up(nsh * 128 * 128 * 4) + up(
            nsh * 128 * 128 * 4)
        assert _ws(seg=L) == want, L
    # fp32 chunk 16: E in fp32
    base32 = _ws(dtype=1, chunk=16, dk=32, dv=16)
    nsh = 2 * 3 * 4  # 7 chunks in segments of 3
    assert _ws(seg=3, dtype=1, chunk=16, dk=32, dv=16) == (up(base32) + up(3 * 4) + up(2 * 4 * 100 * 32 * 4)
                                                           + up(nsh * 32 * 16 * 4) + up(nsh * 32 * 32 * 4)
                                                           + up(nsh * 32 * 16 * 4))
    # packed: an empty sequence is one (empty) segment
    arr = (ctypes.c_int32 * 4)(0, 0, 30, 300)  # 0, 1 and 5 chunks
    basep = _ws(cu=FAKE, cuh=ctypes.addressof(arr), N=3, B=1, T=300)
    nsh = (1 + 1 + 3) * 4
    assert _ws(seg=2, cu=FAKE, cuh=ctypes.addressof(arr), N=3, B=1, T=300) == (
        up(basep) + up(4 * 4) + up(4 * 300 * 128 * 2) + 2 * up(nsh * 128 * 128 * 4) + up(nsh * 128 * 128 * 4))
    assert kla.chunk_workspace_bytes(2, 4, 100, 128, 128, seg_chunks=1) == _ws(seg=1)


def test_seg_workspace_rejections():
    assert _ws(seg=-1) == 0
    assert _ws(seg=2, dk=96) == 0                              # not compiled at all
    assert _ws(seg=2, dtype=1, chunk=64, dk=128) == 0          # the general kernel: no segments
    assert _ws(seg=0, dtype=1, chunk=64, dk=128) == 0          # (no workspace there either)
    assert _ws(seg=3, T=0) > 0                                 # no tokens: empty segments still hold states


def test_seg_entry_point_rejections():
    assert _fwd_seg(-1) == E_SHAPE
    assert _fwd_seg(2, dtype=1, chunk=64, dk=128) == E_UNSUP
    assert _fwd_seg(2, q=None) == E_NULL
    assert _fwd_seg(2, ws_bytes=_ws(seg=2) - 1) == E_WS
    assert _fwd_seg(2, N=0, B=0) == OK


def test_library_choice_of_segments():
    """kla_chunk_fwd segments bf16 chunk-64 grids of fewer than 256 two-tile workgroups on long
    sequences: the T=65536 dv=256 H=16 workload gets three segments of 342 chunks (4 + 6 + 6
    64-column workgroups per head = 256); the B=4 H=16 T=4096 workload (256 two-tile
    workgroups), short sequences, fp32 and dv not a multiple of 64 keep one segment."""
    big = dict(N=1, B=1, H=16, T=65536, dk=128, dv=256)
    assert _ws(**big) == _ws(seg=342, **big) > _ws(seg=0, **big)
    one = dict(N=4, B=4, H=16, T=4096, dk=128, dv=128)
    assert _ws(**one) == _ws(seg=0, **one)
    assert _ws(N=1, B=1, H=16, T=64 * 95, dk=128, dv=256) == _ws(seg=0, N=1, B=1, H=16, T=64 * 95, dk=128, dv=256)
    assert _ws(N=1, B=1, H=4, T=64 * 96, dk=128, dv=256) > _ws(seg=0, N=1, B=1, H=4, T=64 * 96, dk=128, dv=256)
    assert _ws(N=1, B=1, H=16, T=65536, dk=128, dv=240) == _ws(seg=0, N=1, B=1, H=16, T=65536, dk=128, dv=240)
    # packed: the longest sequence sets the segment length
    arr = (ctypes.c_int32 * 3)(0, 1000, 65536)
    cu = dict(cu=FAKE, cuh=ctypes.addressof(arr), N=2, B=1, H=8, T=65536, dk=128, dv=256)
    auto = _ws(**cu)
    assert auto > _ws(seg=0, **cu)
    assert any(auto == _ws(seg=L, **cu) for L in range(100, 1025))
    # kla_chunk_fwd with less than the segmented size runs unsegmented (a GPU test covers that);
    # below the unsegmented size it is refused
    L = kla.lib()
    assert L.kla_chunk_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 1e-6, None, FAKE, FAKE, None, None, 1, 1, 16, 65536, 128,
                           256, 64, 0, FAKE, _ws(seg=0, **big) - 1, None) == E_WS


def test_segment_algebra_on_the_oracle():
    """What the segmented scan computes, on the oracle: a segment's outputs and end state are
    affine in its start state S -- o(S) = o(0) + E S and S_end(S) = S_end(0) + M S, where E and M
    are the outputs and end state of the same segment run with v = 0 from S = I (dk x dk)."""
    rng = np.random.default_rng(11)
    T, dk, dv = 40, 8, 5
    q = rng.standard_normal((1, 1, T, dk))
    k = rng.standard_normal((1, 1, T, dk)) * np.exp(rng.normal(0, 0.5, (1, 1, T, 1)))
    v = rng.standard_normal((1, 1, T, dv))
    g = -np.log1p(np.exp(rng.standard_normal((1, 1, T))))
    eta = 1 / (1 + np.exp(-rng.standard_normal((1, 1, T))))
    S = rng.standard_normal((1, 1, dk, dv))
    o_s, e_s = kla_forward(q, k, v, g, eta, 1e-6, S)
    o_0, e_0 = kla_forward(q, k, v, g, eta, 1e-6, None)
    E, M = kla_forward(q, k, np.zeros((1, 1, T, dk)), g, eta, 1e-6, np.eye(dk)[None, None])
    np.testing.assert_allclose(o_s, o_0 + E @ S, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(e_s, e_0 + M @ S, rtol=1e-10, atol=1e-10)
    # and segments chain: the second half from the first half's end state
    h = T // 2
    o_a, s_a = kla_forward(q[..., :h, :], k[..., :h, :], v[..., :h, :], g[..., :h], eta[..., :h], 1e-6, S)
    o_b0, d_b = kla_forward(q[..., h:, :], k[..., h:, :], v[..., h:, :], g[..., h:], eta[..., h:], 1e-6, None)
    E_b, M_b = kla_forward(q[..., h:, :], k[..., h:, :], np.zeros((1, 1, T - h, dk)), g[..., h:], eta[..., h:],
                           1e-6, np.eye(dk)[None, None])
    np.testing.assert_allclose(np.concatenate([o_a, o_b0 + E_b @ s_a], axis=2), o_s, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(M_b @ s_a + d_b, e_s, rtol=1e-10, atol=1e-10)
