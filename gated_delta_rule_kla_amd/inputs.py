"""Seeded synthetic inputs for the KLA operator (prefill and decode).

This module only draws random numbers and rounds them to the input dtype; it
holds none of the operator's arithmetic.  Both the HIP path (through the
binding) and the fp64 oracle consume the *same* rounded values: the GPU gets
the bf16/fp32 tensors, the oracle gets those exact values widened to fp64.

Distributions follow the workloads the operator is measured on:

* q, k, v ~ N(0, 1) per element;
* each key vector k_t is multiplied by one scalar exp(N(0, sigma_k)) per
  (batch, head, token), so key norms vary (this is what the norm-normalised
  Kaczmarz step is about);
* log-decay g_t = -g_scale * softplus(N(0, 1)) per (batch, head, token);
* relaxation gate eta_t = sigmoid(N(eta_mu, 1)) per (batch, head, token);
* initial state S_0 ~ N(0, s0_std) (std, not variance) or absent.

Draw order is fixed: lengths (varlen only) -> q -> k -> k-scale -> v -> g ->
eta -> S_0.  Normal draws are taken in float32 from numpy's default_rng (the
float32 ziggurat) so that the large workloads can be generated quickly; the
values are then rounded once with round-to-nearest-even to the input dtype.
"""

from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

__all__ = [
    "PrefillInputs",
    "DecodeInputs",
    "make_prefill",
    "make_decode",
    "prefill_config",
    "decode_config",
    "CONFIGS",
    "to_f64",
    "make_upstream",
]


def _softplus(x: np.ndarray) -> np.ndarray:
    # numerically safe log(1 + e^x)
    return np.logaddexp(0.0, x)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def _round(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """Round an array once (RNE) to ``dtype`` and return a CPU tensor."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dtype)


def to_f64(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Widen a CPU/GPU tensor to an fp64 numpy array without changing values."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()


@dataclass
class PrefillInputs:
    """Inputs of one chunked-prefill call, all on the CPU.

    Layout is [B, H, T, d] for q/k/v and [B, H, T] for g/eta.  Packed
    variable-length batches use B = 1 and ``cu_seqlens`` (int32, N + 1
    offsets); ``initial_state`` is [N, H, dk, dv] fp32 with N = B when
    ``cu_seqlens`` is None.
    """

    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    eta: torch.Tensor
    eps: float
    initial_state: Optional[torch.Tensor]
    cu_seqlens: Optional[torch.Tensor]
    chunk: int
    name: str = ""

    @property
    def dims(self):
        B, H, T, dk = self.q.shape
        return B, H, T, dk, self.v.shape[-1]

    @property
    def num_seqs(self) -> int:
        return self.q.shape[0] if self.cu_seqlens is None else self.cu_seqlens.numel() - 1

    @property
    def total_tokens(self) -> int:
        B, H, T, _, _ = self.dims
        return B * T


@dataclass
class DecodeInputs:
    """Inputs of ``steps`` consecutive single-token decode calls.

    q/k: [steps, N, H, dk]; v: [steps, N, H, dv]; g/eta: [steps, N, H];
    state: [N, H, dk, dv] fp32 (the state before the first step).
    """

    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    eta: torch.Tensor
    eps: float
    state: torch.Tensor
    name: str = ""


def _f32(x: float) -> float:
    """The fp32 value the GPU will see for a scalar argument."""
    return float(np.float32(x))


def _draw_tokens(rng, shape_tok, dk, dv, sigma_k, g_scale, eta_mu, dtype):
    """Draw q, k, v, g, eta for token grid ``shape_tok`` in the fixed order."""
    q = rng.standard_normal(shape_tok + (dk,), dtype=np.float32)
    k = rng.standard_normal(shape_tok + (dk,), dtype=np.float32)
    kscale = np.exp(sigma_k * rng.standard_normal(shape_tok, dtype=np.float32))
    k *= kscale[..., None]
    v = rng.standard_normal(shape_tok + (dv,), dtype=np.float32)
    g = -g_scale * _softplus(rng.standard_normal(shape_tok, dtype=np.float32))
    eta = _sigmoid(rng.standard_normal(shape_tok, dtype=np.float32) + np.float32(eta_mu))
    return (_round(q, dtype), _round(k, dtype), _round(v, dtype),
            _round(g, dtype), _round(eta, dtype))


def make_prefill(
    *,
    B: int = 1,
    H: int = 1,
    T: int = 256,
    dk: int = 16,
    dv: int = 16,
    chunk: int = 64,
    dtype: torch.dtype = torch.bfloat16,
    sigma_k: float = 0.5,
    g_scale: float = 1.0,
    eta_mu: float = 0.0,
    eps: float = 1e-6,
    s0_std: float = 0.0,
    lengths: Optional[list] = None,
    seed: int = 0,
    name: str = "",
    rng: Optional[np.random.Generator] = None,
) -> PrefillInputs:
    """Seeded prefill inputs.

    With ``lengths`` given, sequences of those lengths are packed into B = 1,
    T = sum(lengths) and ``cu_seqlens`` is returned.  ``rng`` continues an
    existing stream (used when the lengths were drawn from it first).
    """
    if rng is None:
        rng = np.random.default_rng(seed)
    cu = None
    if lengths is not None:
        lengths = [int(x) for x in lengths]
        B, T = 1, int(sum(lengths))
        cu = torch.tensor([0] + list(np.cumsum(lengths)), dtype=torch.int32)
    q, k, v, g, eta = _draw_tokens(rng, (B, H, T), dk, dv, sigma_k, g_scale, eta_mu, dtype)
    n_seq = B if cu is None else cu.numel() - 1
    s0 = None
    if s0_std > 0.0:
        s0 = torch.from_numpy(
            s0_std * rng.standard_normal((n_seq, H, dk, dv), dtype=np.float32))
    return PrefillInputs(q, k, v, g, eta, _f32(eps), s0, cu, chunk, name)


def make_decode(
    *,
    N: int,
    H: int,
    dk: int,
    dv: int,
    steps: int,
    dtype: torch.dtype = torch.bfloat16,
    sigma_k: float = 0.5,
    g_scale: float = 1.0,
    eta_mu: float = 0.0,
    eps: float = 1e-6,
    s0_std: float = 0.02,
    seed: int = 0,
    name: str = "",
) -> DecodeInputs:
    """Seeded inputs for ``steps`` consecutive decode steps of N sequences."""
    rng = np.random.default_rng(seed)
    q, k, v, g, eta = _draw_tokens(rng, (steps, N, H), dk, dv, sigma_k, g_scale, eta_mu, dtype)
    s0 = torch.from_numpy(s0_std * rng.standard_normal((N, H, dk, dv), dtype=np.float32))
    return DecodeInputs(q, k, v, g, eta, _f32(eps), s0, name)


def unit_keys(x):
    """A copy of prefill or decode inputs ``x`` with every key vector scaled to
    unit length (in fp64 from the rounded keys, then rounded again), for the
    gated-delta-rule mode: there the update coefficient is given, and keys of
    length 1 with coefficients in (0, 1) are the regime in which that rule is
    contractive.  The ``eta`` draws (sigmoid of a normal) then serve as the
    coefficients beta.  Everything else is shared with ``x``."""
    k = x.k.to(torch.float64)
    k = k / torch.linalg.vector_norm(k, dim=-1, keepdim=True).clamp_min(1e-30)
    out = dataclasses.replace(x, k=k.to(x.k.dtype))
    out.name = (x.name or "inputs") + "-unitkeys"
    return out


def _log_uniform_lengths(rng, n, lo, hi):
    u = rng.uniform(math.log(lo), math.log(hi), size=n)
    return [int(x) for x in np.floor(np.exp(u))]


# The five workloads the operator is measured and checked on.  Index = config id.
CONFIGS = {
    0: "tiny fp32: B=1 H=1 T=256 dk=dv=16 chunk=16",
    1: "prefill bf16: B=4 H=16 T=4096 dk=dv=128 chunk=64",
    2: "long-context prefill bf16: B=1 H=16 T=65536 dk=128 dv=256 chunk=64",
    3: "decode bf16: N=256 H=16 dk=dv=128, 512 steps, fp32 state",
    4: "varlen prefill bf16: 32 seqs, lengths log-uniform in [512,16384], H=32 dk=dv=128 chunk=64",
}


def prefill_config(i: int, *, H: Optional[int] = None, T: Optional[int] = None,
                   B: Optional[int] = None) -> PrefillInputs:
    """Prefill workload ``i`` (0, 1, 2 or 4); H/T/B may be overridden to shrink it."""
    seed = 1000 + i
    if i == 0:
        return make_prefill(B=B or 1, H=H or 1, T=T or 256, dk=16, dv=16, chunk=16,
                            dtype=torch.float32, seed=seed, name="cfg0")
    if i == 1:
        return make_prefill(B=B or 4, H=H or 16, T=T or 4096, dk=128, dv=128, chunk=64,
                            seed=seed, name="cfg1")
    if i == 2:
        return make_prefill(B=B or 1, H=H or 16, T=T or 65536, dk=128, dv=256, chunk=64,
                            sigma_k=1.0, g_scale=0.1, eta_mu=1.0, seed=seed, name="cfg2")
    if i == 4:
        rng = np.random.default_rng(seed)
        lengths = _log_uniform_lengths(rng, 32, 512, 16384)
        return make_prefill(H=H or 32, dk=128, dv=128, chunk=64, s0_std=0.02,
                            lengths=lengths, rng=rng, name="cfg4")
    raise ValueError(f"config {i} is not a prefill workload")


def decode_config(steps: int = 512, N: int = 256, H: int = 16) -> DecodeInputs:
    """Decode workload 3 (N sequences x H heads, 128x128 fp32 state)."""
    return make_decode(N=N, H=H, dk=128, dv=128, steps=steps, seed=1003, name="cfg3")


def make_upstream(x: PrefillInputs, seed: int, *, ds_std: Optional[float] = 1.0):
    """Seeded upstream gradients for a prefill call: dL/do ~ N(0, 1) per element,
    rounded to the inputs' dtype ([B, H, T, dv]), and dL/dS_final ~ N(0, ds_std)
    fp32 [N, H, dk, dv] (None when ``ds_std`` is None)."""
    B, H, T, dk, dv = x.dims
    rng = np.random.default_rng(seed)
    do = _round(rng.standard_normal((B, H, T, dv), dtype=np.float32), x.q.dtype)
    ds = None
    if ds_std is not None:
        ds = torch.from_numpy(
            (np.float32(ds_std) * rng.standard_normal((x.num_seqs, H, dk, dv), dtype=np.float32)).copy())
    return do, ds
