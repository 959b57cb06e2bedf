"""Thin ctypes binding over libkla.so (include/kla.h).

Argument marshalling only: shape/dtype checks, output allocation with torch
and the current HIP stream.  Every step of the operator runs in the HIP
kernels; there is no fallback.  If libkla.so is missing the call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = ["chunk_fwd", "chunk_workspace_bytes", "chunk_fwd_workspace_bytes", "pgdn_chunk_fwd", "pgdn_decode_step",
           "pgdn_chunk_workspace_bytes",
           "GAINS", "decode_step", "gdn_chunk_fwd", "gdn_decode_step", "chunk_bwd",
           "gdn_chunk_bwd", "chunk_bwd_workspace_bytes", "lib", "lib_path", "KlaError", "KLA_DT_BF16",
           "KLA_DT_F32"]

KLA_DT_BF16 = 0
KLA_DT_F32 = 1
GAINS = {"given": 0, "kaczmarz": 1}  # kla_gain_t
_DTYPES = {torch.bfloat16: KLA_DT_BF16, torch.float32: KLA_DT_F32}

_LIB: Optional[ctypes.CDLL] = None


def lib_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkla.so")


class KlaError(RuntimeError):
    """A negative kla_status_t returned by the library."""

    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libkla.so once.  torch is imported first so that the library binds
    to the HIP runtime torch already mapped (same soname)."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is not built: run `python -c 'import __graft_entry__ as g; g.build()'` "
                "(or python gated_delta_rule_kla_amd/build.py)")
        L = ctypes.CDLL(path)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.kla_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp,
                                    i32, i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]
        L.kla_chunk_fwd.restype = i32
        L.kla_chunk_workspace_bytes.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, i32]
        L.kla_chunk_workspace_bytes.restype = sz
        L.kla_chunk_fwd_seg.argtypes = [vp, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp,
                                        i32, i32, i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]
        L.kla_chunk_fwd_seg.restype = i32
        L.kla_chunk_seg_workspace_bytes.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32]
        L.kla_chunk_seg_workspace_bytes.restype = sz
        L.kla_decode_step.argtypes = [vp, vp, vp, vp, vp, f32, vp, vp,
                                      i32, i32, i32, i32, i32, vp]
        L.kla_decode_step.restype = i32
        L.kla_gdn_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                        i32, i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]
        L.kla_gdn_chunk_fwd.restype = i32
        L.kla_gdn_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
        L.kla_gdn_decode_step.restype = i32
        L.kla_chunk_bwd.argtypes = [vp, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                    i32, i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]
        L.kla_chunk_bwd.restype = i32
        L.kla_gdn_chunk_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                        i32, i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]
        L.kla_gdn_chunk_bwd.restype = i32
        L.kla_chunk_bwd_workspace_bytes.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, i32]
        L.kla_chunk_bwd_workspace_bytes.restype = sz
        L.kla_chunk_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp,
                                            i32, i32, i32, i32, i32, i32, i32, i32, vp]
        L.kla_chunk_fwd_noalloc.restype = i32
        L.kla_chunk_fwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
        L.kla_chunk_fwd_workspace_bytes.restype = sz
        L.kla_pgdn_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, f32, i32, f32, vp, vp, vp, vp, vp, vp, vp,
                                         i32, i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]
        L.kla_pgdn_chunk_fwd.restype = i32
        L.kla_pgdn_chunk_workspace_bytes.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, i32]
        L.kla_pgdn_chunk_workspace_bytes.restype = sz
        L.kla_pgdn_decode_step.argtypes = [vp, vp, vp, vp, vp, f32, i32, f32, vp, vp, vp,
                                           i32, i32, i32, i32, i32, vp]
        L.kla_pgdn_decode_step.restype = i32
        L.kla_status_str.argtypes = [i32]
        L.kla_status_str.restype = ctypes.c_char_p
        L.kla_abi_version.argtypes = []
        L.kla_abi_version.restype = i32
        _LIB = L
    return _LIB


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise KlaError(fn, status, lib().kla_status_str(status).decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _chunk_call(fn: str, q, k, v, g, coef, eps, initial_state, cu_seqlens, chunk, output_final_state,
                cu_seqlens_host, out, final_state, workspace, seg_chunks=None):
    dev = q.device
    if dev.type != "cuda":
        raise ValueError(f"kla.{fn} needs GPU tensors")
    dtype = q.dtype
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    _need(q, "q", dtype, (B, H, T, dk), dev)
    _need(k, "k", dtype, (B, H, T, dk), dev)
    _need(v, "v", dtype, (B, H, T, dv), dev)
    _need(g, "g", dtype, (B, H, T), dev)
    _need(coef, "eta" if eps is not None else "beta", dtype, (B, H, T), dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, (cu_seqlens.numel(),), dev)
        if cu_seqlens_host is None:
            cu_seqlens_host = cu_seqlens.cpu()
        cu_seqlens_host = cu_seqlens_host.to(torch.int32).contiguous()
        if cu_seqlens_host.numel() != cu_seqlens.numel():
            raise ValueError("cu_seqlens_host does not mirror cu_seqlens")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (N, H, dk, dv), dev)
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=dtype, device=dev)
    else:
        _need(out, "out", dtype, (B, H, T, dv), dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, (N, H, dk, dv), dev)
    host_ptr = None if cu_seqlens_host is None else cu_seqlens_host.data_ptr()
    if isinstance(workspace, str) and workspace == "static" and eps is not None:
        # kla_chunk_fwd_noalloc: the library's fixed per-GPU scratch, no workspace argument
        st = lib().kla_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(coef), float(eps),
                                         _ptr(initial_state), _ptr(out), _ptr(final_state), _ptr(cu_seqlens),
                                         host_ptr, N, B, H, T, dk, dv, int(chunk), _DTYPES[dtype], _stream(dev))
        _check("kla_chunk_fwd_noalloc", st)
        return out, final_state
    if isinstance(workspace, str):
        raise ValueError(f"kla.{fn}: workspace must be a tensor or None ('static' is for chunk_fwd only)")
    if seg_chunks is not None:
        if eps is None:
            raise ValueError(f"kla.{fn}: seg_chunks is for chunk_fwd only")
        ws_bytes = lib().kla_chunk_seg_workspace_bytes(_ptr(cu_seqlens), host_ptr, N, B, H, T, dk, dv, int(chunk),
                                                       _DTYPES[dtype], int(seg_chunks))
    else:
        ws_bytes = lib().kla_chunk_workspace_bytes(_ptr(cu_seqlens), host_ptr, N, B, H, T, dk, dv, int(chunk),
                                                   _DTYPES[dtype])
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    tail = (_ptr(initial_state), _ptr(out), _ptr(final_state), _ptr(cu_seqlens), host_ptr, N, B, H, T, dk, dv,
            int(chunk), _DTYPES[dtype], _ptr(workspace), workspace.numel(), _stream(dev))
    if seg_chunks is not None:
        st = lib().kla_chunk_fwd_seg(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(coef), float(eps), *tail[:13],
                                     int(seg_chunks), *tail[13:])
        _check("kla_chunk_fwd_seg", st)
    elif eps is not None:
        st = lib().kla_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(coef), float(eps), *tail)
        _check("kla_chunk_fwd", st)
    else:
        st = lib().kla_gdn_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(coef), *tail)
        _check("kla_gdn_chunk_fwd", st)
    return out, final_state


def chunk_fwd(
    q: torch.Tensor,
    k: torch.Tensor,
    v: torch.Tensor,
    g: torch.Tensor,
    eta: torch.Tensor,
    eps: float = 1e-6,
    initial_state: Optional[torch.Tensor] = None,
    cu_seqlens: Optional[torch.Tensor] = None,
    chunk: int = 64,
    output_final_state: bool = True,
    cu_seqlens_host: Optional[torch.Tensor] = None,
    out: Optional[torch.Tensor] = None,
    final_state: Optional[torch.Tensor] = None,
    workspace: Optional[torch.Tensor] = None,
    seg_chunks: Optional[int] = None,
) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """KLA chunkwise prefill (kla_chunk_fwd).

    q, k: [B, H, T, dk]; v: [B, H, T, dv]; g, eta: [B, H, T]; all bf16 or all
    fp32 on one GPU.  initial_state: [N, H, dk, dv] fp32 or None.  cu_seqlens:
    int32 [N + 1] on the GPU (B must be 1) or None.  Returns (o, final_state).
    ``final_state`` may be passed as the same tensor as ``initial_state`` to
    update it in place.  ``workspace`` (uint8, on the GPU, at least
    chunk_workspace_bytes(...) bytes) is taken from torch's caching allocator
    on the current stream when not given.  ``workspace="static"`` calls
    kla_chunk_fwd_noalloc instead, which uses the library's fixed per-GPU
    scratch buffer (KLA_NOALLOC_SCRATCH_BYTES, 64 MiB) and allocates nothing
    (pass ``out`` and ``final_state`` to keep the call allocation-free here too).
    ``seg_chunks`` (kla_chunk_fwd_seg): None lets the library choose whether to cut
    long sequences into segments scanned side by side; 0 never cuts; n > 0 cuts
    every sequence into segments of n chunks.
    """
    if seg_chunks is not None and isinstance(workspace, str):
        raise ValueError("kla.chunk_fwd: seg_chunks needs a workspace tensor or None")
    return _chunk_call("chunk_fwd", q, k, v, g, eta, eps, initial_state, cu_seqlens, chunk,
                       output_final_state, cu_seqlens_host, out, final_state, workspace, seg_chunks)


NOALLOC_SCRATCH_BYTES = 64 << 20  # KLA_NOALLOC_SCRATCH_BYTES in include/kla.h


def gdn_chunk_fwd(
    q: torch.Tensor,
    k: torch.Tensor,
    v: torch.Tensor,
    g: torch.Tensor,
    beta: torch.Tensor,
    initial_state: Optional[torch.Tensor] = None,
    cu_seqlens: Optional[torch.Tensor] = None,
    chunk: int = 64,
    output_final_state: bool = True,
    cu_seqlens_host: Optional[torch.Tensor] = None,
    out: Optional[torch.Tensor] = None,
    final_state: Optional[torch.Tensor] = None,
    workspace: Optional[torch.Tensor] = None,
) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Gated delta rule chunkwise prefill (kla_gdn_chunk_fwd): as chunk_fwd
    with the update coefficient ``beta`` [B, H, T] given instead of eta, eps."""
    return _chunk_call("gdn_chunk_fwd", q, k, v, g, beta, None, initial_state, cu_seqlens, chunk,
                       output_final_state, cu_seqlens_host, out, final_state, workspace)


def chunk_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, chunk: int = 64,
                          dtype: torch.dtype = torch.bfloat16,
                          cu_seqlens_host: Optional[torch.Tensor] = None,
                          seg_chunks: Optional[int] = None) -> int:
    """Workspace bytes kla_chunk_fwd needs (kla_chunk_workspace_bytes), or
    kla_chunk_fwd_seg with ``seg_chunks`` (kla_chunk_seg_workspace_bytes); 0 for
    arguments it would reject.  With packed sequences pass the host int32
    cu_seqlens (B must be 1)."""
    if cu_seqlens_host is not None:
        cu = cu_seqlens_host.to(torch.int32).contiguous()
        # the device pointer is only tested for NULL here
        args = (ctypes.c_void_p(16), cu.data_ptr(), cu.numel() - 1, B, H, T, dk, dv, int(chunk), _DTYPES[dtype])
    else:
        args = (None, None, B, B, H, T, dk, dv, int(chunk), _DTYPES[dtype])
    if seg_chunks is not None:
        return lib().kla_chunk_seg_workspace_bytes(*args, int(seg_chunks))
    return lib().kla_chunk_workspace_bytes(*args)


def pgdn_chunk_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, chunk: int = 64,
                               dtype: torch.dtype = torch.bfloat16) -> int:
    """Workspace bytes kla_pgdn_chunk_fwd needs for a dense batch
    (kla_pgdn_chunk_workspace_bytes); 0 where it runs the general kernel."""
    return lib().kla_pgdn_chunk_workspace_bytes(None, None, B, B, H, T, dk, dv, int(chunk), _DTYPES[dtype])


def chunk_fwd_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, chunk: int = 64,
                              num_seqs: Optional[int] = None) -> int:
    """Upper bound on the workspace bytes kla_chunk_fwd needs for these sizes,
    for either dtype and either layout (kla_chunk_fwd_workspace_bytes)."""
    return lib().kla_chunk_fwd_workspace_bytes(B, H, T, dk, dv, int(chunk), B if num_seqs is None else num_seqs)


def _bwd_call(fn, q, k, v, g, coef, eps, do, initial_state, dfinal_state, cu_seqlens, chunk, cu_seqlens_host,
              need_dinitial, workspace):
    dev = q.device
    if dev.type != "cuda":
        raise ValueError(f"kla.{fn} needs GPU tensors")
    dtype = q.dtype
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    _need(q, "q", dtype, (B, H, T, dk), dev)
    _need(k, "k", dtype, (B, H, T, dk), dev)
    _need(v, "v", dtype, (B, H, T, dv), dev)
    _need(g, "g", dtype, (B, H, T), dev)
    _need(coef, "eta" if eps is not None else "beta", dtype, (B, H, T), dev)
    _need(do, "do", dtype, (B, H, T, dv), dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, (cu_seqlens.numel(),), dev)
        if cu_seqlens_host is None:
            cu_seqlens_host = cu_seqlens.cpu()
        cu_seqlens_host = cu_seqlens_host.to(torch.int32).contiguous()
        if cu_seqlens_host.numel() != cu_seqlens.numel():
            raise ValueError("cu_seqlens_host does not mirror cu_seqlens")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (N, H, dk, dv), dev)
    if dfinal_state is not None:
        _need(dfinal_state, "dfinal_state", torch.float32, (N, H, dk, dv), dev)
    dq = torch.empty_like(q)
    dkk = torch.empty_like(k)
    dvv = torch.empty_like(v)
    dg = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    dcoef = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    ds0 = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if need_dinitial else None
    host_ptr = None if cu_seqlens_host is None else cu_seqlens_host.data_ptr()
    ws_bytes = lib().kla_chunk_bwd_workspace_bytes(_ptr(cu_seqlens), host_ptr, N, B, H, T, dk, dv, int(chunk),
                                                   _DTYPES[dtype])
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    mid = (_ptr(initial_state), _ptr(do), _ptr(dfinal_state), _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dg),
           _ptr(dcoef), _ptr(ds0), _ptr(cu_seqlens), host_ptr, N, B, H, T, dk, dv, int(chunk),
           _DTYPES[dtype], _ptr(workspace), workspace.numel(), _stream(dev))
    if eps is not None:
        st = lib().kla_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(coef), float(eps), *mid)
        _check("kla_chunk_bwd", st)
    else:
        st = lib().kla_gdn_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(coef), *mid)
        _check("kla_gdn_chunk_bwd", st)
    return dq, dkk, dvv, dg, dcoef, ds0


def chunk_bwd(
    q: torch.Tensor,
    k: torch.Tensor,
    v: torch.Tensor,
    g: torch.Tensor,
    eta: torch.Tensor,
    do: torch.Tensor,
    eps: float = 1e-6,
    initial_state: Optional[torch.Tensor] = None,
    dfinal_state: Optional[torch.Tensor] = None,
    cu_seqlens: Optional[torch.Tensor] = None,
    chunk: int = 64,
    cu_seqlens_host: Optional[torch.Tensor] = None,
    need_dinitial: bool = True,
    workspace: Optional[torch.Tensor] = None,
):
    """Gradients of chunk_fwd (kla_chunk_bwd) for upstream gradients ``do``
    [B, H, T, dv] (dtype of q) and ``dfinal_state`` [N, H, dk, dv] fp32 or None.

    Returns (dq, dk, dv, dg, deta, dinitial_state): dq, dk, dv in the inputs'
    dtype; dg, deta [B, H, T] fp32; dinitial_state [N, H, dk, dv] fp32 (None
    unless ``need_dinitial``).  Other arguments as chunk_fwd.
    """
    return _bwd_call("chunk_bwd", q, k, v, g, eta, eps, do, initial_state, dfinal_state, cu_seqlens, chunk,
                     cu_seqlens_host, need_dinitial, workspace)


def gdn_chunk_bwd(
    q: torch.Tensor,
    k: torch.Tensor,
    v: torch.Tensor,
    g: torch.Tensor,
    beta: torch.Tensor,
    do: torch.Tensor,
    initial_state: Optional[torch.Tensor] = None,
    dfinal_state: Optional[torch.Tensor] = None,
    cu_seqlens: Optional[torch.Tensor] = None,
    chunk: int = 64,
    cu_seqlens_host: Optional[torch.Tensor] = None,
    need_dinitial: bool = True,
    workspace: Optional[torch.Tensor] = None,
):
    """Gradients of gdn_chunk_fwd (kla_gdn_chunk_bwd); the fifth result is dbeta."""
    return _bwd_call("gdn_chunk_bwd", q, k, v, g, beta, None, do, initial_state, dfinal_state, cu_seqlens,
                     chunk, cu_seqlens_host, need_dinitial, workspace)


def chunk_bwd_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, chunk: int = 64,
                              dtype: torch.dtype = torch.bfloat16,
                              cu_seqlens_host: Optional[torch.Tensor] = None) -> int:
    """Workspace bytes kla_chunk_bwd needs (kla_chunk_bwd_workspace_bytes)."""
    if cu_seqlens_host is not None:
        cu = cu_seqlens_host.to(torch.int32).contiguous()
        return lib().kla_chunk_bwd_workspace_bytes(ctypes.c_void_p(16), cu.data_ptr(), cu.numel() - 1, B, H, T,
                                                   dk, dv, int(chunk), _DTYPES[dtype])
    return lib().kla_chunk_bwd_workspace_bytes(None, None, B, B, H, T, dk, dv, int(chunk), _DTYPES[dtype])


def _decode_call(fn, q, k, v, g, coef, eps, state, out):
    dev = q.device
    if dev.type != "cuda":
        raise ValueError(f"kla.{fn} needs GPU tensors")
    dtype = q.dtype
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}")
    N, H, dk = q.shape
    dv = v.shape[-1]
    _need(q, "q", dtype, (N, H, dk), dev)
    _need(k, "k", dtype, (N, H, dk), dev)
    _need(v, "v", dtype, (N, H, dv), dev)
    _need(g, "g", dtype, (N, H), dev)
    _need(coef, "eta" if eps is not None else "beta", dtype, (N, H), dev)
    _need(state, "state", torch.float32, (N, H, dk, dv), dev)
    if out is None:
        out = torch.empty((N, H, dv), dtype=dtype, device=dev)
    else:
        _need(out, "out", dtype, (N, H, dv), dev)
    tail = (_ptr(state), _ptr(out), N, H, dk, dv, _DTYPES[dtype], _stream(dev))
    if eps is not None:
        st = lib().kla_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(coef), float(eps), *tail)
        _check("kla_decode_step", st)
    else:
        st = lib().kla_gdn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(coef), *tail)
        _check("kla_gdn_decode_step", st)
    return out


def decode_step(
    q: torch.Tensor,
    k: torch.Tensor,
    v: torch.Tensor,
    g: torch.Tensor,
    eta: torch.Tensor,
    eps: float,
    state: torch.Tensor,
    out: Optional[torch.Tensor] = None,
) -> torch.Tensor:
    """One KLA recurrent step (kla_decode_step); ``state`` is updated in place.

    q, k: [N, H, dk]; v: [N, H, dv]; g, eta: [N, H]; state: [N, H, dk, dv] fp32.
    Returns o [N, H, dv].
    """
    return _decode_call("decode_step", q, k, v, g, eta, eps, state, out)


def gdn_decode_step(
    q: torch.Tensor,
    k: torch.Tensor,
    v: torch.Tensor,
    g: torch.Tensor,
    beta: torch.Tensor,
    state: torch.Tensor,
    out: Optional[torch.Tensor] = None,
) -> torch.Tensor:
    """One gated-delta-rule step (kla_gdn_decode_step): as decode_step with the
    update coefficient ``beta`` [N, H] given; ``state`` is updated in place."""
    return _decode_call("gdn_decode_step", q, k, v, g, beta, None, state, out)


def pgdn_chunk_fwd(
    q: torch.Tensor,
    k: torch.Tensor,
    v: torch.Tensor,
    g: torch.Tensor,
    coef: torch.Tensor,
    eps: float = 1e-6,
    gain: str = "given",
    band: float = 1.5,
    initial_state: Optional[torch.Tensor] = None,
    initial_acc: Optional[torch.Tensor] = None,
    cu_seqlens: Optional[torch.Tensor] = None,
    chunk: int = 64,
    output_final_state: bool = True,
    cu_seqlens_host: Optional[torch.Tensor] = None,
    out: Optional[torch.Tensor] = None,
    final_state: Optional[torch.Tensor] = None,
    final_acc: Optional[torch.Tensor] = None,
    workspace: Optional[torch.Tensor] = None,
):
    """Preconditioned gated delta rule prefill (kla_pgdn_chunk_fwd).

    As chunk_fwd, with ``coef`` [B, H, T] the update coefficient beta
    (gain="given") or eta (gain="kaczmarz": beta = eta / (k . w + eps)), the
    preconditioner's band x >= 1, and the key accumulator [N, H, dk] fp32 in
    (``initial_acc``, zeros when None) and out.  ``workspace`` (uint8, at least
    kla_pgdn_chunk_workspace_bytes(...) bytes) is taken from torch's caching
    allocator when not given.  Returns (o, final_state, final_acc) (the last two
    None unless ``output_final_state`` or given)."""
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("kla.pgdn_chunk_fwd needs GPU tensors")
    dtype = q.dtype
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}")
    if gain not in GAINS:
        raise ValueError(f"gain must be one of {sorted(GAINS)}")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    for t, name, shp in ((q, "q", (B, H, T, dk)), (k, "k", (B, H, T, dk)), (v, "v", (B, H, T, dv)),
                         (g, "g", (B, H, T)), (coef, "coef", (B, H, T))):
        _need(t, name, dtype, shp, dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, (cu_seqlens.numel(),), dev)
        if cu_seqlens_host is None:
            cu_seqlens_host = cu_seqlens.cpu()
        cu_seqlens_host = cu_seqlens_host.to(torch.int32).contiguous()
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (N, H, dk, dv), dev)
    if initial_acc is not None:
        _need(initial_acc, "initial_acc", torch.float32, (N, H, dk), dev)
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=dtype, device=dev)
    _need(out, "out", dtype, (B, H, T, dv), dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    if output_final_state and final_acc is None:
        final_acc = torch.empty((N, H, dk), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, (N, H, dk, dv), dev)
    if final_acc is not None:
        _need(final_acc, "final_acc", torch.float32, (N, H, dk), dev)
    host_ptr = None if cu_seqlens_host is None else cu_seqlens_host.data_ptr()
    ws_bytes = lib().kla_pgdn_chunk_workspace_bytes(_ptr(cu_seqlens), host_ptr, N, B, H, T, dk, dv, int(chunk),
                                                    _DTYPES[dtype])
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    st = lib().kla_pgdn_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(coef), float(eps), GAINS[gain],
                                  float(band), _ptr(initial_state), _ptr(initial_acc), _ptr(out), _ptr(final_state),
                                  _ptr(final_acc), _ptr(cu_seqlens), host_ptr, N, B, H, T, dk, dv, int(chunk),
                                  _DTYPES[dtype], _ptr(workspace), workspace.numel(), _stream(dev))
    _check("kla_pgdn_chunk_fwd", st)
    return out, final_state, final_acc


def pgdn_decode_step(
    q: torch.Tensor,
    k: torch.Tensor,
    v: torch.Tensor,
    g: torch.Tensor,
    coef: torch.Tensor,
    eps: float,
    state: torch.Tensor,
    acc: torch.Tensor,
    gain: str = "given",
    band: float = 1.5,
    out: Optional[torch.Tensor] = None,
) -> torch.Tensor:
    """One preconditioned gated-delta-rule step (kla_pgdn_decode_step);
    ``state`` [N, H, dk, dv] and ``acc`` [N, H, dk] (fp32) are updated in place."""
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("kla.pgdn_decode_step needs GPU tensors")
    dtype = q.dtype
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}")
    if gain not in GAINS:
        raise ValueError(f"gain must be one of {sorted(GAINS)}")
    N, H, dk = q.shape
    dv = v.shape[-1]
    for t, name, shp in ((q, "q", (N, H, dk)), (k, "k", (N, H, dk)), (v, "v", (N, H, dv)), (g, "g", (N, H)),
                         (coef, "coef", (N, H))):
        _need(t, name, dtype, shp, dev)
    _need(state, "state", torch.float32, (N, H, dk, dv), dev)
    _need(acc, "acc", torch.float32, (N, H, dk), dev)
    if out is None:
        out = torch.empty((N, H, dv), dtype=dtype, device=dev)
    _need(out, "out", dtype, (N, H, dv), dev)
    st = lib().kla_pgdn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(coef), float(eps), GAINS[gain],
                                    float(band), _ptr(state), _ptr(acc), _ptr(out), N, H, dk, dv, _DTYPES[dtype],
                                    _stream(dev))
    _check("kla_pgdn_decode_step", st)
    return out
