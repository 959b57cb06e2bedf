"""The C ABI on a host without a GPU: it loads, exports every symbol the header
declares, and rejects bad arguments with the documented status codes before
any HIP call (no compute call is made here)."""

import ctypes
import os
import re

import pytest

from gated_delta_rule_kla_amd import kla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kla.h")

pytestmark = pytest.mark.skipif(not os.path.exists(kla.lib_path()),
                                reason="libkla.so not built (run __graft_entry__.build())")

OK, E_NULL, E_SHAPE, E_DTYPE, E_UNSUP, E_SEQ, E_EPS, E_WS, E_ALIGN, E_HIP = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9
E_SCRATCH = -10
E_PARAM = -11
FAKE = 0x7F0000000000  # never dereferenced: every case below fails validation first
OK_IF_NO_TOKENS = "ok-if-no-tokens"


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"\b(kla_[a-z_0-9]+)\s*\(", txt)))


def test_exports_every_declared_symbol():
    L = kla.lib()
    names = _declared()
    assert set(names) >= {"kla_chunk_fwd", "kla_chunk_fwd_workspace_bytes", "kla_chunk_workspace_bytes",
                          "kla_decode_step", "kla_status_str",
                          "kla_abi_version", "kla_gdn_chunk_fwd", "kla_gdn_decode_step", "kla_chunk_bwd",
                          "kla_gdn_chunk_bwd", "kla_chunk_bwd_workspace_bytes", "kla_chunk_fwd_noalloc",
                          "kla_pgdn_chunk_fwd", "kla_pgdn_decode_step", "kla_pgdn_chunk_workspace_bytes"}
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_matches_header():
    v = int(re.search(r"#define KLA_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert kla.lib().kla_abi_version() == v


def test_status_strings():
    L = kla.lib()
    for s in (OK, E_NULL, E_SHAPE, E_DTYPE, E_UNSUP, E_SEQ, E_EPS, E_WS, E_ALIGN, E_HIP, E_SCRATCH, E_PARAM, -77):
        txt = L.kla_status_str(s)
        assert isinstance(txt, bytes) and len(txt) > 0


def _ws_bytes(**kw):
    a = dict(cu=None, cuh=None, N=2, B=2, H=4, T=100, dk=128, dv=128, chunk=64, dtype=0)
    a.update(kw)
    return kla.lib().kla_chunk_workspace_bytes(a["cu"], a["cuh"], a["N"], a["B"], a["H"], a["T"], a["dk"],
                                               a["dv"], a["chunk"], a["dtype"])


def _chunk(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, eta=FAKE, eps=1e-6, s0=None, o=FAKE, sf=FAKE,
             cu=None, cuh=None, N=2, B=2, H=4, T=100, dk=128, dv=128, chunk=64, ws=FAKE,
             ws_bytes=1 << 40, dtype=0)
    a.update(kw)
    return kla.lib().kla_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["eta"], a["eps"], a["s0"],
                                   a["o"], a["sf"], a["cu"], a["cuh"], a["N"], a["B"], a["H"],
                                   a["T"], a["dk"], a["dv"], a["chunk"], a["dtype"], a["ws"],
                                   a["ws_bytes"], None)


def _decode(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, eta=FAKE, eps=1e-6, S=FAKE, o=FAKE,
             N=3, H=2, dk=128, dv=128, dtype=0)
    a.update(kw)
    return kla.lib().kla_decode_step(a["q"], a["k"], a["v"], a["g"], a["eta"], a["eps"], a["S"],
                                     a["o"], a["N"], a["H"], a["dk"], a["dv"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), E_DTYPE),
    (dict(H=0), E_SHAPE),
    (dict(H=65537), E_SHAPE),                    # heads beyond a launch grid's second dimension
    (dict(T=-1), E_SHAPE),
    (dict(N=3), E_SHAPE),                        # N must equal B without cu_seqlens
    (dict(eps=-1.0), E_EPS),
    (dict(eps=float("nan")), E_EPS),
    (dict(eps=float("inf")), E_EPS),
    (dict(dk=96), E_UNSUP),
    (dict(dv=24), E_UNSUP),
    (dict(chunk=32), E_UNSUP),
    (dict(dk=256), E_UNSUP),                     # the general kernel stops at dk = 128
    (dict(q=None), E_NULL),
    (dict(o=None), E_NULL),
    (dict(k=FAKE + 8), E_ALIGN),
    (dict(sf=FAKE + 4), E_ALIGN),
    (dict(cu=FAKE), E_NULL),                     # device cu_seqlens without the host mirror
    (dict(ws=None), E_WS),
    (dict(ws_bytes=1000), E_WS),                 # two 64-token chunks x 2 sequences x 4 heads need more
    (dict(ws=FAKE + 8), E_ALIGN),
])
def test_chunk_fwd_rejects(kw, code):
    assert _chunk(**kw) == code


def test_chunk_fwd_seqlens_validation():
    def host(vals):
        arr = (ctypes.c_int32 * len(vals))(*vals)
        return arr, ctypes.addressof(arr)
    keep, h = host([0, 30, 20, 100])             # decreasing
    assert _chunk(cu=FAKE, cuh=h, N=3, B=1) == E_SEQ
    keep, h = host([0, 30, 60, 90])              # does not end at T = 100
    assert _chunk(cu=FAKE, cuh=h, N=3, B=1) == E_SEQ
    keep, h = host([5, 30, 60, 100])             # does not start at 0
    assert _chunk(cu=FAKE, cuh=h, N=3, B=1) == E_SEQ
    keep, h = host([0, 30, 60, 100])
    assert _chunk(cu=FAKE, cuh=h, N=3, B=2) == E_SHAPE   # varlen needs B == 1
    assert _chunk(cu=FAKE + 2, cuh=h, N=3, B=1) == E_ALIGN


def test_chunk_fwd_nothing_to_do():
    # zero sequences: valid, returns without touching the GPU
    assert _chunk(N=0, B=0) == OK


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), E_DTYPE),
    (dict(H=0), E_SHAPE),
    (dict(N=-1), E_SHAPE),
    (dict(eps=-0.5), E_EPS),
    (dict(dk=48), E_UNSUP),
    (dict(dv=512), E_UNSUP),
    (dict(S=None), E_NULL),
    (dict(v=FAKE + 2), E_ALIGN),
])
def test_decode_rejects(kw, code):
    assert _decode(**kw) == code


def test_decode_zero_sequences_is_noop():
    assert _decode(N=0) == OK


def _gdn_chunk(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, s0=None, o=FAKE, sf=FAKE,
             cu=None, cuh=None, N=2, B=2, H=4, T=100, dk=128, dv=128, chunk=64, ws=FAKE,
             ws_bytes=1 << 40, dtype=0)
    a.update(kw)
    return kla.lib().kla_gdn_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["o"], a["sf"],
                                       a["cu"], a["cuh"], a["N"], a["B"], a["H"], a["T"], a["dk"], a["dv"],
                                       a["chunk"], a["dtype"], a["ws"], a["ws_bytes"], None)


def _gdn_decode(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, S=FAKE, o=FAKE, N=3, H=2, dk=128, dv=128, dtype=0)
    a.update(kw)
    return kla.lib().kla_gdn_decode_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S"], a["o"], a["N"],
                                         a["H"], a["dk"], a["dv"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), E_DTYPE),
    (dict(T=-3), E_SHAPE),
    (dict(dk=96), E_UNSUP),
    (dict(beta=None), E_NULL),
    (dict(beta=FAKE + 4), E_ALIGN),
    (dict(ws=None), E_WS),
    (dict(N=0, B=0), OK),
])
def test_gdn_chunk_fwd_rejects(kw, code):
    assert _gdn_chunk(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), E_DTYPE),
    (dict(dv=24), E_UNSUP),
    (dict(beta=None), E_NULL),
    (dict(S=FAKE + 8), E_ALIGN),
    (dict(N=0), OK),
])
def test_gdn_decode_rejects(kw, code):
    assert _gdn_decode(**kw) == code


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 16)
    with pytest.raises(ValueError):
        kla.chunk_fwd(x, x, x, x[..., 0], x[..., 0])
    with pytest.raises(ValueError):
        kla.decode_step(x[0], x[0], x[0], x[0, :, 0], x[0, :, 0], 1e-6, x)
    with pytest.raises(ValueError):
        kla.gdn_chunk_fwd(x, x, x, x[..., 0], x[..., 0])
    with pytest.raises(ValueError):
        kla.gdn_decode_step(x[0], x[0], x[0], x[0, :, 0], x[0, :, 0], x)


def test_workspace_bytes():
    # bf16, chunk 64, per (chunk, head): the T'^T image packed to the part the scan reads (rows
    # 0..31 all 64 columns, rows 32..63 the last 32) and gamma, Gam, d (3 x 64 fp32)
    per = (32 * 64 + 32 * 32) * 2 + 3 * 64 * 4
    assert _ws_bytes() == 2 * 4 * 2 * per                  # B=2 rows x ceil(100/64)=2 chunks x H=4
    assert _ws_bytes(T=128) == 2 * 4 * 2 * per
    assert _ws_bytes(T=129) == 2 * 4 * 3 * per
    assert _ws_bytes(T=0) == 0 and _ws_bytes(N=0, B=0) == 0
    assert _ws_bytes(dk=96) == 0                           # unsupported -> 0
    assert _ws_bytes(H=65537) == 0 and _ws_bytes(H=65536) > 0
    # fp32 chunk 16: 16 x 16 fp32 image + 3 x 16 fp32
    assert _ws_bytes(dtype=1, chunk=16, dk=32, dv=16) == 2 * 4 * 7 * (16 * 16 * 4 + 3 * 16 * 4)
    # fp32 chunk 64: packed 64-column image (32 x 64 + 32 x 32 fp32) + 3 x 64 fp32
    assert _ws_bytes(dtype=1, chunk=64, dk=32, dv=16) == 2 * 4 * 2 * ((32 * 64 + 32 * 32) * 4 + 3 * 64 * 4)
    # packed sequences: floor(T / C) + N + 1 slots per head (rounded up to 256 bytes), then the
    # longest-first sequence order (N int32, rounded up to 256 bytes)
    arr = (ctypes.c_int32 * 4)(0, 30, 60, 100)
    img = 4 * (100 // 64 + 3 + 1) * per
    assert _ws_bytes(cu=FAKE, cuh=ctypes.addressof(arr), N=3, B=1) == (img + 255) // 256 * 256 + 256
    # the binding's helper agrees
    assert kla.chunk_workspace_bytes(2, 4, 100, 128, 128) == _ws_bytes()
    # exactly the reported size is accepted by the validation (then FAKE pointers would be used,
    # so only check that a size one byte short is rejected)
    assert _chunk(ws_bytes=_ws_bytes() - 1) == E_WS


def test_fwd_workspace_bound_query():
    """kla_chunk_fwd_workspace_bytes(B, H, T, dk, dv, chunk, num_seqs) takes neither the dtype nor
    cu_seqlens, so it bounds the exact need over both element types and both layouts."""
    L = kla.lib()
    q = lambda B, H, T, dk, dv, C, N: L.kla_chunk_fwd_workspace_bytes(B, H, T, dk, dv, C, N)
    for (B, H, T, dk, dv, C) in [(2, 4, 100, 128, 128, 64), (4, 16, 4096, 128, 128, 64), (1, 3, 777, 32, 16, 16),
                                 (1, 2, 300, 16, 32, 64)]:
        bound = q(B, H, T, dk, dv, C, B)
        exact = [_ws_bytes(B=B, N=B, H=H, T=T, dk=dk, dv=dv, chunk=C, dtype=dt) for dt in (0, 1)]
        if B == 1:  # one sequence may also come packed with cu_seqlens = [0, T]
            arr = (ctypes.c_int32 * 2)(0, T)
            exact += [_ws_bytes(cu=FAKE, cuh=ctypes.addressof(arr), N=1, B=1, H=H, T=T, dk=dk, dv=dv, chunk=C,
                                dtype=dt) for dt in (0, 1)]
        assert bound == max(exact) and bound > 0
        if B == 1:
            for N in (1, 3, 17):
                arr = (ctypes.c_int32 * (N + 1))(*([0] * N + [T]))
                ex = [_ws_bytes(cu=FAKE, cuh=ctypes.addressof(arr), N=N, B=1, H=H, T=T, dk=dk, dv=dv, chunk=C,
                                dtype=dt) for dt in (0, 1)]
                assert q(1, H, T, dk, dv, C, N) >= max(ex) > 0
                # any other split of the same tokens into N sequences needs the same bytes
                arr2 = (ctypes.c_int32 * (N + 1))(*[T * i // N for i in range(N + 1)])
                ex2 = [_ws_bytes(cu=FAKE, cuh=ctypes.addressof(arr2), N=N, B=1, H=H, T=T, dk=dk, dv=dv,
                                 chunk=C, dtype=dt) for dt in (0, 1)]
                assert ex2 == ex
    assert q(2, 4, 0, 128, 128, 64, 2) == 0
    assert q(2, 4, 100, 96, 128, 64, 2) == 0             # unsupported for both dtypes
    assert kla.chunk_fwd_workspace_bytes(2, 4, 100, 128, 128) == q(2, 4, 100, 128, 128, 64, 2)


def test_workspace_slots_never_collide():
    """The packed-sequence slot of chunk c of sequence n is n + floor(t0_n / C) + c: distinct for all
    (n, c) and below floor(T / C) + N + 1, for any lengths (brute force over random length mixes)."""
    import random
    rng = random.Random(7)
    C = 64
    for _ in range(300):
        N = rng.randint(1, 12)
        lens = [rng.choice([0, 1, 5, 63, 64, 65, 127, 128, 200, rng.randint(0, 400)]) for _ in range(N)]
        t0, seen = 0, set()
        T = sum(lens)
        for n, L in enumerate(lens):
            for c in range((L + C - 1) // C):
                s = n + t0 // C + c
                assert s not in seen and 0 <= s < T // C + N + 1
                seen.add(s)
            t0 += L


def _bwd(fn="kla_chunk_bwd", **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, eta=FAKE, eps=1e-6, s0=None, do=FAKE, dsf=None,
             dq=FAKE, dk_=FAKE, dv_=FAKE, dg=FAKE, deta=FAKE, ds0=None, cu=None, cuh=None,
             N=2, B=2, H=4, T=100, dk=128, dv=128, chunk=64, ws=FAKE, ws_bytes=1 << 40, dtype=0)
    a.update(kw)
    head = (a["q"], a["k"], a["v"], a["g"], a["eta"])
    if fn == "kla_chunk_bwd":
        head = head + (a["eps"],)
    return getattr(kla.lib(), fn)(*head, a["s0"], a["do"], a["dsf"], a["dq"], a["dk_"], a["dv_"], a["dg"],
                                  a["deta"], a["ds0"], a["cu"], a["cuh"], a["N"], a["B"], a["H"], a["T"],
                                  a["dk"], a["dv"], a["chunk"], a["dtype"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("fn", ["kla_chunk_bwd", "kla_gdn_chunk_bwd"])
@pytest.mark.parametrize("kw,code", [
    (dict(dtype=0, chunk=16), E_UNSUP),           # forward-only shapes (general kernel)
    (dict(dtype=0, dk=16), E_UNSUP),
    (dict(dtype=1, chunk=64, dk=128), E_UNSUP),
    (dict(dtype=7), E_DTYPE),
    (dict(H=0), E_SHAPE),
    (dict(N=3), E_SHAPE),
    (dict(dk=96), E_UNSUP),
    (dict(chunk=32), E_UNSUP),
    (dict(do=None), E_NULL),
    (dict(dq=None), E_NULL),
    (dict(dg=None), E_NULL),
    (dict(deta=None), E_NULL),
    (dict(dk_=FAKE + 8), E_ALIGN),
    (dict(ds0=FAKE + 4), E_ALIGN),
    (dict(dsf=FAKE + 4), E_ALIGN),
    (dict(cu=FAKE), E_NULL),
    (dict(ws=None), E_WS),
    (dict(ws_bytes=1000), E_WS),
    (dict(N=0, B=0), OK),
])
def test_chunk_bwd_rejects(fn, kw, code):
    assert _bwd(fn, **kw) == code


def test_chunk_bwd_eps_checked():
    assert _bwd(eps=-1.0) == E_EPS
    assert _bwd(eps=float("nan")) == E_EPS


def test_chunk_bwd_workspace_bytes():
    L = kla.lib()

    def ws(**kw):
        a = dict(cu=None, cuh=None, N=2, B=2, H=4, T=100, dk=128, dv=128, chunk=64, dtype=0)
        a.update(kw)
        return L.kla_chunk_bwd_workspace_bytes(a["cu"], a["cuh"], a["N"], a["B"], a["H"], a["T"], a["dk"],
                                               a["dv"], a["chunk"], a["dtype"])

    r256 = lambda x: (x + 255) // 256 * 256
    # per (chunk, head): bf16 chunk 64 -- the packed T^T image (rows < 32 all 64 columns, rows
    # >= 32 the last 32, bf16); otherwise T, P and K K^T . E (C x C in the input element type)
    # + 4 C fp32 vectors; then the chunk-start state and chunk-end state gradient (dk x dv each,
    # in the input element type); B=2 x ceil(100/64)=2 chunks x H=4; then the forward's
    # workspace (its kernels produce the chunk-start states)
    slots = 2 * 2 * 4
    assert ws() == r256(slots * (32 * 64 + 32 * 32) * 2) + 2 * r256(slots * 128 * 128 * 2) + _ws_bytes()
    assert ws(dtype=1, chunk=16, dk=32, dv=16) == (r256(2 * 7 * 4 * (3 * 16 * 16 + 4 * 16) * 4)
                                                   + 2 * r256(2 * 7 * 4 * 32 * 16 * 4)
                                                   + _ws_bytes(dtype=1, chunk=16, dk=32, dv=16))
    assert ws(T=0) == 0 and ws(N=0, B=0) == 0 and ws(dk=96) == 0
    assert kla.chunk_bwd_workspace_bytes(2, 4, 100, 128, 128) == ws()
    assert _bwd(ws_bytes=ws() - 1) == E_WS


def test_binding_refuses_cpu_tensors_bwd():
    import torch
    x = torch.zeros(1, 1, 4, 16)
    with pytest.raises(ValueError):
        kla.chunk_bwd(x, x, x, x[..., 0], x[..., 0], x)
    with pytest.raises(ValueError):
        kla.gdn_chunk_bwd(x, x, x, x[..., 0], x[..., 0], x)


def _noalloc(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, eta=FAKE, eps=1e-6, s0=None, o=FAKE, sf=FAKE,
             cu=None, cuh=None, N=2, B=2, H=4, T=100, dk=128, dv=128, chunk=64, dtype=0)
    a.update(kw)
    return kla.lib().kla_chunk_fwd_noalloc(a["q"], a["k"], a["v"], a["g"], a["eta"], a["eps"], a["s0"],
                                           a["o"], a["sf"], a["cu"], a["cuh"], a["N"], a["B"], a["H"],
                                           a["T"], a["dk"], a["dv"], a["chunk"], a["dtype"], None)


def test_noalloc_scratch_limit_and_validation():
    """kla_chunk_fwd_noalloc validates like kla_chunk_fwd and refuses, before any HIP call, a call
    whose workspace would not fit its fixed 64 MiB buffer."""
    limit = int(re.search(r"#define KLA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)",
                          open(HEADER).read()).group(1)) << 20
    assert limit == kla.NOALLOC_SCRATCH_BYTES == 64 << 20
    # B=4 H=64 T=8192 bf16: 4 x 64 x 128 chunk-heads x 6,912 B = 226 MB
    assert _ws_bytes(N=4, B=4, H=64, T=8192) > limit
    assert _noalloc(N=4, B=4, H=64, T=8192) == E_SCRATCH
    # the B=4 H=16 T=4096 workload fits (28.3 MB)
    assert _ws_bytes(N=4, B=4, H=16, T=4096) <= limit
    for kw, code in [(dict(dtype=7), E_DTYPE), (dict(eps=-1.0), E_EPS), (dict(dk=96), E_UNSUP),
                     (dict(q=None), E_NULL), (dict(k=FAKE + 8), E_ALIGN), (dict(N=3), E_SHAPE),
                     (dict(N=0, B=0), OK)]:
        assert _noalloc(**kw) == code, kw


def test_chunk_fwd_supported_shape_set():
    """The shape set of the contract: either dtype, chunk 16 or 64, dk 16 .. 128 (powers of two),
    dv a multiple of 16 up to 256; the pipelined kernels take some of it (and need a workspace),
    the general kernel the rest (no workspace)."""
    for dt in (0, 1):
        for C in (16, 64):
            for dk in (16, 32, 64, 128):
                for dv in (16, 128, 256):
                    fast = (dt == 0 and C == 64 and dk in (64, 128)) or (dt == 1 and (C == 16 or dk <= 32))
                    ws = _ws_bytes(dtype=dt, chunk=C, dk=dk, dv=dv)
                    assert (ws > 0) == fast, (dt, C, dk, dv, ws)
                    # supported: validation gets past the shape checks to the (failing) pointer check,
                    # which comes before any launch
                    assert _chunk(dtype=dt, chunk=C, dk=dk, dv=dv, q=None) == E_NULL, (dt, C, dk, dv)
    for bad in (dict(chunk=32), dict(dk=96), dict(dk=256), dict(dv=272), dict(dv=24)):
        assert _chunk(**bad) == E_UNSUP


def _pgdn(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, c=FAKE, eps=1e-6, gain=0, band=1.5, s0=None, a0=None, o=FAKE,
             sf=None, af=None, cu=None, cuh=None, N=2, B=2, H=4, T=100, dk=128, dv=128, chunk=64, dtype=0,
             ws=None, wsb=0)
    a.update(kw)
    return kla.lib().kla_pgdn_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["c"], a["eps"], a["gain"], a["band"],
                                        a["s0"], a["a0"], a["o"], a["sf"], a["af"], a["cu"], a["cuh"], a["N"],
                                        a["B"], a["H"], a["T"], a["dk"], a["dv"], a["chunk"], a["dtype"], a["ws"],
                                        a["wsb"], None)


def _pgdn_dec(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, c=FAKE, eps=1e-6, gain=1, band=1.5, S=FAKE, A=FAKE, o=FAKE,
             N=3, H=2, dk=128, dv=128, dtype=0)
    a.update(kw)
    return kla.lib().kla_pgdn_decode_step(a["q"], a["k"], a["v"], a["g"], a["c"], a["eps"], a["gain"], a["band"],
                                          a["S"], a["A"], a["o"], a["N"], a["H"], a["dk"], a["dv"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(gain=2), E_PARAM), (dict(gain=-1), E_PARAM), (dict(band=0.9), E_PARAM), (dict(band=float("nan")), E_PARAM),
    (dict(band=float("inf")), E_PARAM), (dict(gain=1, eps=-1.0), E_EPS), (dict(gain=0, eps=-1.0), OK_IF_NO_TOKENS),
    (dict(dtype=3), E_DTYPE), (dict(dk=96), E_UNSUP), (dict(chunk=32), E_UNSUP), (dict(c=None), E_NULL),
    (dict(a0=FAKE + 4), E_ALIGN), (dict(af=FAKE + 8), E_ALIGN), (dict(N=3), E_SHAPE), (dict(N=0, B=0), OK),
])
def test_pgdn_chunk_fwd_rejects(kw, code):
    if code == OK_IF_NO_TOKENS:   # eps is unused with the given gain: only the other checks apply
        assert _pgdn(N=0, B=0, **kw) == OK
        return
    assert _pgdn(**kw) == code


def test_pgdn_workspace():
    """bf16, chunk 64, dk 64 or 128 run the pipelined kernels: their workspace is the
    forward's plus, per (chunk, head), dk fp32 (chunk-start key accumulator) and
    64 x dk bf16 (write keys), each region rounded up to 256 bytes; other shapes run
    the general kernel and need none.  A call without it fails before any launch."""
    L = kla.lib()
    q = lambda dk=128, dtype=0, chunk=64, T=100: L.kla_pgdn_chunk_workspace_bytes(None, None, 2, 2, 4, T, dk, 128,
                                                                                 chunk, dtype)
    r256 = lambda x: (x + 255) // 256 * 256
    slots = 2 * 2 * 4
    for dk in (128, 64):
        assert q(dk) == r256(_ws_bytes(dk=dk)) + r256(slots * dk * 4) + slots * 64 * dk * 2
    assert q(dtype=1) == 0 and q(chunk=16) == 0 and q(dk=32) == 0 and q(T=0) == 0
    assert kla.pgdn_chunk_workspace_bytes(2, 4, 100, 128, 128) == q()
    assert _pgdn() == E_WS
    assert _pgdn(ws=FAKE, wsb=q() - 1) == E_WS


@pytest.mark.parametrize("kw,code", [
    (dict(gain=5), E_PARAM), (dict(band=0.5), E_PARAM), (dict(eps=float("nan")), E_EPS), (dict(dk=48), E_UNSUP),
    (dict(dv=300), E_UNSUP), (dict(A=None), E_NULL), (dict(A=FAKE + 4), E_ALIGN), (dict(N=0), OK),
])
def test_pgdn_decode_rejects(kw, code):
    assert _pgdn_dec(**kw) == code
