"""Intermediate parity: what the prep kernel hands to the scan kernel, against the oracle.

After a kla_chunk_fwd call (bf16, chunk 64) the caller's workspace holds, for every (head, slot)
that carries a chunk, 6,912 bytes: the packed image of T'^T (T' = T Diag(beta), T = (I + A)^-1,
in bf16) and then gamma, Gam = exp(gamma) and d = exp(gamma_C - gamma) as 3 x 64 fp32.  The
image keeps rows s < 32 with all 64 columns and rows s >= 32 with columns 32..63 (the rest of
those rows is an upper-triangle zero block), and each row's columns in the grouped order the scan
kernel's operand reads take: inside each block of 32 columns, column 16 h + 4 a + e sits at
position 8 a + 4 h + e.  Slots follow the chunks: sequence n's chunk c is slot
n * ceil(T / 64) + c for dense batches and n + floor(cu[n] / 64) + c for packed ones.

The test decodes that layout (it is written out here from that description, not taken from the
library) and compares it with the per-chunk dump of the oracle's chunkwise form
(kla_chunkwise(..., return_chunks=True)): T'^T to 2e-2 x its largest entry (an fp32 solve from
bf16 keys, stored in bf16), the decay vectors to fp32 rounding, and exact zeros wherever the
chunk has no rows (a ragged last chunk) or T' is zero by its triangular structure.
"""

import numpy as np
import pytest
import torch

from gated_delta_rule_kla_amd import inputs, kla
from oracle import kla_chunkwise

pytestmark = pytest.mark.gpu

C = 64
SLOT_BYTES = 32 * 64 * 2 + 32 * 32 * 2 + 3 * 64 * 4  # 6,912


def _natural_col(pc):
    """Natural column held at grouped position pc of a row."""
    return (pc & ~31) | (((pc >> 2) & 1) << 4) | (((pc >> 3) & 3) << 2) | (pc & 3)


def _bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _decode_slot(buf):
    img = _bf16_to_f64(np.frombuffer(buf[:6144].tobytes(), dtype=np.uint16))
    tpt = np.zeros((C, C))
    for e in range(32 * 64):
        s, pc = divmod(e, 64)
        tpt[s, _natural_col(pc)] = img[e]
    for e in range(32 * 32):
        s, pc = 32 + e // 32, 32 + e % 32
        tpt[s, _natural_col(pc)] = img[2048 + e]
    vec = np.frombuffer(buf[6144:SLOT_BYTES].tobytes(), dtype=np.float32).astype(np.float64).reshape(3, C)
    return tpt, vec[0], vec[1], vec[2]


def _check_chunk(buf, dump, where):
    tpt, gam, Gam, d = _decode_slot(buf)
    n = len(dump["beta"])
    ref = (dump["T"] * dump["beta"][None, :]).T  # T'^T[s][r] = T[r][s] beta_s
    err = np.abs(tpt[:n, :n] - ref).max() / np.abs(ref).max()
    assert err <= 2e-2, (where, "T'^T", err)
    # zero outside the chunk's rows, and T'^T is upper triangular (T' lower)
    assert not np.any(tpt[n:, :]) and not np.any(tpt[:, n:]), (where, "rows past the chunk")
    assert not np.any(np.tril(tpt, -1)), (where, "below the diagonal of T'^T")
    g_ref = dump["gamma"]
    tol = 1e-5 * max(1.0, np.abs(g_ref).max())
    assert np.abs(gam[:n] - g_ref).max() <= tol, (where, "gamma")
    assert np.all(gam[n:] == gam[n - 1]), (where, "gamma past the chunk")
    np.testing.assert_allclose(Gam[:n], np.exp(g_ref), rtol=2e-5, atol=0, err_msg=f"{where} Gam")
    np.testing.assert_allclose(d[:n], np.exp(g_ref[-1] - g_ref), rtol=2e-5, atol=0, err_msg=f"{where} d")


def _run(x, dev):
    B, H, T, dk = x.q.shape
    dv = x.v.shape[-1]
    cu = None if x.cu_seqlens is None else x.cu_seqlens.to(dev)
    N = B if cu is None else cu.numel() - 1
    ws_bytes = kla.chunk_workspace_bytes(B, H, T, dk, dv, chunk=C, dtype=torch.bfloat16,
                                         cu_seqlens_host=None if cu is None else x.cu_seqlens)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    kla.chunk_fwd(x.q.to(dev), x.k.to(dev), x.v.to(dev), x.g.to(dev), x.eta.to(dev), x.eps,
                  None if x.initial_state is None else x.initial_state.to(dev), cu_seqlens=cu, chunk=C,
                  workspace=ws)
    torch.cuda.synchronize()
    return ws.cpu().numpy(), N


@pytest.mark.parametrize("dk", [128, 64])
def test_prep_images_and_decay_vectors_dense(dk):
    dev = torch.device("cuda:0")
    x = inputs.make_prefill(B=2, H=3, T=200, dk=dk, dv=64, chunk=C, seed=4242)
    ws, N = _run(x, dev)
    B, H, T, _ = x.q.shape
    nch = (T + C - 1) // C
    nslot = B * nch
    f = inputs.to_f64
    for b in range(B):
        for h in range(H):
            _, _, dumps = kla_chunkwise(f(x.q[b, h]), f(x.k[b, h]), f(x.v[b, h]), f(x.g[b, h]), f(x.eta[b, h]),
                                        x.eps, None, C, return_chunks=True)
            assert len(dumps) == nch
            for c, dump in enumerate(dumps):
                off = (h * nslot + b * nch + c) * SLOT_BYTES
                _check_chunk(ws[off:off + SLOT_BYTES], dump, (b, h, c))


def test_prep_images_and_decay_vectors_packed():
    dev = torch.device("cuda:0")
    x = inputs.make_prefill(H=2, dk=128, dv=64, chunk=C, lengths=[70, 0, 130, 64], seed=4243)
    ws, N = _run(x, dev)
    cu = x.cu_seqlens.numpy()
    T = int(cu[-1])
    nslot = T // C + N + 1  # the workspace's slots per head for packed sequences
    f = inputs.to_f64
    for n in range(N):
        t0, t1 = int(cu[n]), int(cu[n + 1])
        if t1 == t0:
            continue
        for h in range(x.q.shape[1]):
            sl = slice(t0, t1)
            _, _, dumps = kla_chunkwise(f(x.q[0, h, sl]), f(x.k[0, h, sl]), f(x.v[0, h, sl]), f(x.g[0, h, sl]),
                                        f(x.eta[0, h, sl]), x.eps, None, C, return_chunks=True)
            for c, dump in enumerate(dumps):
                slot = n + t0 // C + c
                off = (h * nslot + slot) * SLOT_BYTES
                _check_chunk(ws[off:off + SLOT_BYTES], dump, (n, h, c))


def test_prep_images_on_a_grid_with_multi_slot_runs():
    """A packed grid of 42,000-odd chunk-heads (H=32, 40 sequences of up to 4,000 tokens), large
    enough that each prep wave takes a run of several consecutive slots, prefetching the next
    slot's rows while it solves the current one, with runs that cross sequence boundaries.
    Every chunk of five sampled sequences is checked on three heads."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(4244)
    lengths = [int(v) for v in rng.integers(1, 4000, size=40)]
    lengths[7] = 0
    x = inputs.make_prefill(H=32, dk=64, dv=16, chunk=C, lengths=lengths, seed=4245)
    cu = x.cu_seqlens.numpy()
    T = int(cu[-1])
    N = len(lengths)
    nslot = T // C + N + 1
    assert nslot * 32 > 40960  # more than ten units of 4,096 chunk-heads: runs of several slots
    print(f"case multi-slot runs: T={T} nslot={nslot} chunk-heads={nslot * 32}", flush=True)
    ws, _ = _run(x, dev)
    f = inputs.to_f64
    for n in (0, 6, 8, 23, N - 1):
        t0, t1 = int(cu[n]), int(cu[n + 1])
        for h in (0, 17, 31):
            sl = slice(t0, t1)
            _, _, dumps = kla_chunkwise(f(x.q[0, h, sl]), f(x.k[0, h, sl]), f(x.v[0, h, sl]), f(x.g[0, h, sl]),
                                        f(x.eta[0, h, sl]), x.eps, None, C, return_chunks=True)
            for c, dump in enumerate(dumps):
                slot = n + t0 // C + c
                off = (h * nslot + slot) * SLOT_BYTES
                _check_chunk(ws[off:off + SLOT_BYTES], dump, (n, h, c))
