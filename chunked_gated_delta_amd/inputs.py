"""Seeded synthetic inputs for the KDA chunked forward.

This module holds no arithmetic of the method itself (no gate, no prefix, no
recurrence): it only draws random tensors with the distributions of the
workloads and rounds them to the compute dtype.  Both the HIP path and the
oracle receive exactly the values produced here.

Recipe (per workload):
  q, k ~ N(0, 1) per token, L2-normalised over dk (in float64), then rounded;
  v ~ N(0, 1);  beta = sigmoid(N(0, 1)) per (token, head);
  w ~ N(mu, sd) per (token, channel), sd being the standard deviation;
  S0 ~ N(0, s0_sd) in float32 when the workload has an initial state.
Rounding to bf16 is round-to-nearest-even.

Two generators:
  * ``make_numpy`` draws each (b, h) from its own numpy stream
    ``default_rng([seed, b, h])`` in the order q, k, v, beta-logit, w, S0.
    Used at sizes the oracle handles whole.
  * ``make_torch`` draws whole tensors with one seeded torch generator on the
    target device.  Used at full workload sizes, where the oracle checks
    sampled heads whose inputs are copied back from these same tensors.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    dtype: str            # "bf16" or "f32"
    w_mu: float = 0.0
    w_sd: float = 2.0
    s0_sd: Optional[float] = None
    g_min: float = -5.0   # -inf selects the unbounded gate
    chunk: int = 16

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def token_heads(self) -> int:
        return self.B * self.H * self.T


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 1, 64, 32, 32, "f32"),
    "bf16_4k": Workload("bf16_4k", 2, 16, 4096, 128, 128, "bf16"),
    "decay_stress": Workload("decay_stress", 1, 32, 65536, 128, 128, "bf16",
                             w_mu=6.0, w_sd=1.0, s0_sd=0.1),
    "million": Workload("million", 1, 16, 1048576, 128, 128, "bf16"),
    "unbounded": Workload("unbounded", 2, 16, 4096, 128, 128, "bf16",
                          w_mu=3.0, w_sd=3.0, g_min=-math.inf),
    "headline": Workload("headline", 1, 16, 65536, 128, 128, "bf16"),
    # recurrent decode: a serving batch advanced by one token, fp32 states resident in HBM (512 MiB of
    # state, more than the last-level cache, so that each call streams it from HBM)
    "decode_b512": Workload("decode_b512", 512, 16, 1, 128, 128, "bf16", s0_sd=0.5),
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float values to the nearest bf16 (ties to even); returns float32."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    # NaN stays NaN (never produced by the generators, kept for completeness)
    return np.where(np.isnan(f), f, out)


def _round(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    return np.asarray(x, dtype=np.float32)


def _l2norm(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, 1e-30)


def make_numpy(wl: Workload, seed: int = 0) -> dict:
    """Per-(b,h) streams; values are float32 arrays holding dtype-rounded numbers."""
    B, H, T, dk, dv = wl.B, wl.H, wl.T, wl.dk, wl.dv
    q = np.empty((B, H, T, dk), np.float32)
    k = np.empty((B, H, T, dk), np.float32)
    v = np.empty((B, H, T, dv), np.float32)
    w = np.empty((B, H, T, dk), np.float32)
    beta = np.empty((B, H, T), np.float32)
    S0 = np.empty((B, H, dk, dv), np.float32) if wl.s0_sd is not None else None
    for b in range(B):
        for h in range(H):
            rng = np.random.default_rng([seed, b, h])
            q[b, h] = _round(_l2norm(rng.standard_normal((T, dk))), wl.dtype)
            k[b, h] = _round(_l2norm(rng.standard_normal((T, dk))), wl.dtype)
            v[b, h] = _round(rng.standard_normal((T, dv)), wl.dtype)
            beta[b, h] = _round(1.0 / (1.0 + np.exp(-rng.standard_normal(T))), wl.dtype)
            w[b, h] = _round(rng.normal(wl.w_mu, wl.w_sd, (T, dk)), wl.dtype)
            if S0 is not None:
                S0[b, h] = rng.normal(0.0, wl.s0_sd, (dk, dv)).astype(np.float32)
    return dict(q=q, k=k, v=v, w=w, beta=beta, S0=S0, dtype=wl.dtype, g_min=wl.g_min)


def make_cotangents(wl: Workload, seed: int = 0, with_dSf: bool = True) -> dict:
    """Seeded adjoints for a backward pass: dO ~ N(0, 1) [B,H,T,dv] rounded to the workload dtype,
    and dS_final ~ N(0, 1) fp32 [B,H,dk,dv] (or None).  Streams are per (b, h) and distinct from
    make_numpy's."""
    B, H, T, dk, dv = wl.B, wl.H, wl.T, wl.dk, wl.dv
    dO = np.empty((B, H, T, dv), np.float32)
    dSf = np.empty((B, H, dk, dv), np.float32) if with_dSf else None
    for b in range(B):
        for h in range(H):
            rng = np.random.default_rng([seed, b, h, 7])
            dO[b, h] = _round(rng.standard_normal((T, dv)), wl.dtype)
            if dSf is not None:
                dSf[b, h] = rng.standard_normal((dk, dv)).astype(np.float32)
    return dict(dO=dO, dSf=dSf)


def torch_dtype(dtype: str):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def numpy_to_torch(inp: dict, device) -> dict:
    """Move make_numpy output to torch tensors of the compute dtype (exact: values are pre-rounded)."""
    import torch
    td = torch_dtype(inp["dtype"])
    out = {}
    for key in ("q", "k", "v", "w", "beta"):
        out[key] = torch.from_numpy(inp[key]).to(device=device, dtype=td).contiguous()
    out["S0"] = None if inp["S0"] is None else torch.from_numpy(inp["S0"]).to(device).contiguous()
    out["dtype"] = inp["dtype"]
    out["g_min"] = inp["g_min"]
    return out


def make_torch(wl: Workload, seed: int = 0, device="cuda") -> dict:
    """Whole-tensor draws with one seeded torch generator on ``device``."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1000003 + 12345)
    B, H, T, dk, dv = wl.B, wl.H, wl.T, wl.dk, wl.dv
    td = torch_dtype(wl.dtype)

    def normal(shape, mu=0.0, sd=1.0):
        x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        if sd != 1.0:
            x.mul_(sd)
        if mu != 0.0:
            x.add_(mu)
        return x

    def unit(shape):
        x = normal(shape)
        x = x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)
        return x.to(td).contiguous()

    q = unit((B, H, T, dk))
    k = unit((B, H, T, dk))
    v = normal((B, H, T, dv)).to(td).contiguous()
    beta = torch.sigmoid(normal((B, H, T))).to(td).contiguous()
    w = normal((B, H, T, dk), wl.w_mu, wl.w_sd).to(td).contiguous()
    S0 = None
    if wl.s0_sd is not None:
        S0 = normal((B, H, dk, dv), 0.0, wl.s0_sd).contiguous()
    return dict(q=q, k=k, v=v, w=w, beta=beta, S0=S0, dtype=wl.dtype, g_min=wl.g_min)


def head_to_f64(inp: dict, b: int, h: int) -> dict:
    """float64 numpy copies of one (b, h) slice, shaped [1,1,...] (exact for bf16/f32)."""
    def f(x):
        if x is None:
            return None
        a = x[b:b + 1, h:h + 1]
        if hasattr(a, "detach"):
            a = a.detach().float().cpu().numpy()
        return np.asarray(a, dtype=np.float64)
    return {key: f(inp[key]) for key in ("q", "k", "v", "w", "beta", "S0")}


def all_to_f64(inp: dict) -> dict:
    def f(x):
        if x is None:
            return None
        if hasattr(x, "detach"):
            x = x.detach().float().cpu().numpy()
        return np.asarray(x, dtype=np.float64)
    return {key: f(inp[key]) for key in ("q", "k", "v", "w", "beta", "S0")}
