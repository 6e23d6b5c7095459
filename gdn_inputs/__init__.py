"""Seeded synthetic inputs for the Gated DeltaNet mixer (forward and backward).

This module is shared by the tests, the bench and the smoke check.  It holds none
of the method's arithmetic: it only draws random tensors and shapes them into the
inputs the mixer receives (unit-norm q and k, beta in (0, 1), log-decay g <= 0).
Normalising q and k, the sigmoid on beta and the softplus clamp on g are done
here, before the call, in fp32; the kernels and the oracle take the stored
tensors as given.  The per-key-channel gate follows the clamp of the Atomic-GDN2
card, section 2.1: g = -min(softplus(g_raw), 5), so alpha = exp(g) lies in
[e^-5, 1].

Every tensor is drawn from one ``torch.Generator`` seeded once, in the fixed order
q, k, v, beta_raw, g_raw, S0.  CPU and GPU generators give different streams;
each test draws once and hands the same stored tensors to both sides.

``grad_inputs`` draws the cotangents of a backward call (dL/do, dL/dS_T) from a
generator of their own, so that adding them changes none of the forward inputs.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import torch

__all__ = ["ChunkConfig", "DecodeConfig", "CHUNK_CONFIGS", "DECODE_CONFIG", "BWD_CONFIG",
           "chunk_inputs", "decode_inputs", "grad_inputs", "prologue_inputs", "head_tokens",
           "hard_reset_gate", "decoupled_gates"]


@dataclass(frozen=True)
class ChunkConfig:
    name: str
    B: int
    H: int
    T: int
    K: int
    V: int
    dtype: str            # "fp32" or "bf16": storage of q, k, v and o
    gate: str             # "head" (scalar per head-token) or "channel" (per key channel)
    g_sigma: float = 1.0  # g_raw ~ N(0, g_sigma^2)
    g_cap: Optional[float] = None   # channel clamp: g = -min(softplus(g_raw), g_cap)
    g_scale: float = 1.0  # multiplies g after the clamp (stress cases use 0 or 0.01)
    s0_sigma: float = 0.0  # 0 => S0 absent (zeros)
    chunk: int = 64
    seed: int = 0

    def with_(self, **kw) -> "ChunkConfig":
        return replace(self, **kw)


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    N: int
    H: int
    K: int
    V: int
    steps: int
    dtype: str = "bf16"
    gate: str = "channel"
    g_sigma: float = 2.0
    g_cap: Optional[float] = 5.0
    s_sigma: float = 0.02
    seed: int = 0

    def with_(self, **kw) -> "DecodeConfig":
        return replace(self, **kw)


CHUNK_CONFIGS = {
    # small fp32 correctness case
    "scalar_fp32_small": ChunkConfig("scalar_fp32_small", B=1, H=2, T=256, K=64, V=64,
                                     dtype="fp32", gate="head"),
    # scalar-gate prefill, bf16 inputs, fp32 state: the headline throughput case
    "scalar_bf16": ChunkConfig("scalar_bf16", B=8, H=12, T=8192, K=128, V=128,
                               dtype="bf16", gate="head"),
    # per-key-channel gate, bf16 inputs
    "channel_bf16": ChunkConfig("channel_bf16", B=16, H=8, T=2048, K=128, V=128,
                                dtype="bf16", gate="channel", g_sigma=2.0, g_cap=5.0),
    # long prefill, 48 heads of 128x128 fp32 state (3 MiB per layer)
    "channel_long": ChunkConfig("channel_long", B=1, H=48, T=262144, K=128, V=128,
                                dtype="bf16", gate="channel", g_sigma=2.0, g_cap=5.0,
                                s0_sigma=0.02),
}

DECODE_CONFIG = DecodeConfig("decode_256x48", N=256, H=48, K=128, V=128, steps=64)

# forward + backward at the shape of the Atomic-GDN2 card's kernel benchmark
# (section 5.1: batch 4, head dimension 128, up to 6 heads, 4096 tokens; the
# log-decay domain [-5, 0] of section 5)
BWD_CONFIG = ChunkConfig("bwd_channel_bf16", B=4, H=6, T=4096, K=128, V=128, dtype="bf16",
                         gate="channel", g_sigma=2.0, g_cap=5.0, s0_sigma=0.02)

_DT = {"fp32": torch.float32, "bf16": torch.bfloat16}


def head_tokens(cfg: ChunkConfig) -> int:
    return cfg.B * cfg.H * cfg.T


def _unit(x: torch.Tensor) -> torch.Tensor:
    """Scale each trailing vector to unit L2 norm (fp32)."""
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)


def _gate(raw: torch.Tensor, cap: Optional[float], scale: float) -> torch.Tensor:
    sp = torch.nn.functional.softplus(raw)
    if cap is not None:
        sp = sp.clamp(max=cap)
    return (-sp * scale).contiguous()


def _gen(device, seed):
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return gen


def chunk_inputs(cfg: ChunkConfig, device="cpu", seed: Optional[int] = None):
    """Inputs of one prefill call: dict with q, k [B,T,H,K], v [B,T,H,V] (storage
    dtype), g [B,T,H] or [B,T,H,K] fp32, beta [B,T,H] fp32, S0 [B,H,K,V] fp32 or None."""
    device = torch.device(device)
    gen = _gen(device, cfg.seed if seed is None else seed)
    dt = _DT[cfg.dtype]
    B, T, H, K, V = cfg.B, cfg.T, cfg.H, cfg.K, cfg.V
    f32 = dict(device=device, dtype=torch.float32, generator=gen)
    q = _unit(torch.randn(B, T, H, K, **f32)).to(dt)
    k = _unit(torch.randn(B, T, H, K, **f32)).to(dt)
    v = torch.randn(B, T, H, V, **f32).to(dt)
    beta = torch.sigmoid(torch.randn(B, T, H, **f32))
    gshape = (B, T, H, K) if cfg.gate == "channel" else (B, T, H)
    g = _gate(cfg.g_sigma * torch.randn(*gshape, **f32), cfg.g_cap, cfg.g_scale)
    S0 = None
    if cfg.s0_sigma > 0:
        S0 = cfg.s0_sigma * torch.randn(B, H, K, V, **f32)
    return dict(q=q.contiguous(), k=k.contiguous(), v=v.contiguous(), g=g,
                beta=beta.contiguous(), S0=S0)


def decode_inputs(cfg: DecodeConfig, device="cpu", seed: Optional[int] = None):
    """Inputs of a chain of decode steps: q, k [steps,N,H,K], v [steps,N,H,V],
    g [steps,N,H,K] or [steps,N,H] fp32, beta [steps,N,H] fp32, S0 [N,H,K,V] fp32."""
    device = torch.device(device)
    gen = _gen(device, cfg.seed if seed is None else seed)
    dt = _DT[cfg.dtype]
    n, N, H, K, V = cfg.steps, cfg.N, cfg.H, cfg.K, cfg.V
    f32 = dict(device=device, dtype=torch.float32, generator=gen)
    q = _unit(torch.randn(n, N, H, K, **f32)).to(dt)
    k = _unit(torch.randn(n, N, H, K, **f32)).to(dt)
    v = torch.randn(n, N, H, V, **f32).to(dt)
    beta = torch.sigmoid(torch.randn(n, N, H, **f32))
    gshape = (n, N, H, K) if cfg.gate == "channel" else (n, N, H)
    g = _gate(cfg.g_sigma * torch.randn(*gshape, **f32), cfg.g_cap, 1.0)
    S0 = cfg.s_sigma * torch.randn(N, H, K, V, **f32)
    return dict(q=q.contiguous(), k=k.contiguous(), v=v.contiguous(), g=g,
                beta=beta.contiguous(), S0=S0.contiguous())


def hard_reset_gate(shape, seed: int, device="cpu") -> torch.Tensor:
    """Scalar log-decays with hard resets: most values from -softplus(N(0,1)), about
    one in eight drawn uniformly from [-200, -20] (alpha below e^-20 wipes the
    state), so that a scalar-gate path sees g far below the per-channel clamp."""
    gen = _gen(torch.device(device), seed)
    f32 = dict(device=device, dtype=torch.float32, generator=gen)
    g = -torch.nn.functional.softplus(torch.randn(*shape, **f32))
    reset = torch.rand(*shape, **f32) < 0.125
    deep = -20.0 - 180.0 * torch.rand(*shape, **f32)
    return torch.where(reset, deep, g).contiguous()


def decoupled_gates(shape, seed: int, device="cpu"):
    """Erase and write gates of the decoupled-gate variant: two independent draws
    of sigmoid(N(0, 1)) of the given shape (beta's distribution), from a generator
    seeded with seed + 104729 so that adding them changes none of the other inputs.
    Returns (erase, write) fp32."""
    gen = _gen(torch.device(device), seed + 104729)
    f32 = dict(device=device, dtype=torch.float32, generator=gen)
    erase = torch.sigmoid(torch.randn(*shape, **f32))
    write = torch.sigmoid(torch.randn(*shape, **f32))
    return erase.contiguous(), write.contiguous()


def grad_inputs(cfg: ChunkConfig, device="cpu", seed: Optional[int] = None):
    """Cotangents of one backward call: d_o [B,T,H,V] (storage dtype) ~ N(0, 1) and
    dS_T [B,H,K,V] fp32 ~ N(0, 1), from a generator seeded with seed + 7919."""
    device = torch.device(device)
    gen = _gen(device, (cfg.seed if seed is None else seed) + 7919)
    f32 = dict(device=device, dtype=torch.float32, generator=gen)
    d_o = torch.randn(cfg.B, cfg.T, cfg.H, cfg.V, **f32).to(_DT[cfg.dtype])
    dS_T = torch.randn(cfg.B, cfg.H, cfg.K, cfg.V, **f32)
    return dict(d_o=d_o.contiguous(), dS_T=dS_T.contiguous())


def prologue_inputs(B: int, T: int, H: int, K: int, V: int, dtype: str = "bf16",
                    gate: str = "channel", state: bool = True, device="cpu", seed: int = 0):
    """Raw inputs of the prologue: the projections' outputs q_raw, k_raw [B,T,H,K],
    v_raw [B,T,H,V] ~ N(0,1) (storage dtype), g_raw [B,T,H(,K)] ~ N(0, 2^2),
    b_raw [B,T,H] ~ N(0,1); depthwise taps w_q, w_k [H*K,4], w_v [H*V,4] ~ N(0, 0.5^2)
    fp32; carried states cs_q, cs_k [B,3,H*K], cs_v [B,3,H*V] ~ N(0,1) (storage
    dtype) or None.  Drawn in that order from one generator."""
    device = torch.device(device)
    gen = _gen(device, seed)
    dt = _DT[dtype]
    f32 = dict(device=device, dtype=torch.float32, generator=gen)
    d = dict(q_raw=torch.randn(B, T, H, K, **f32).to(dt), k_raw=torch.randn(B, T, H, K, **f32).to(dt),
             v_raw=torch.randn(B, T, H, V, **f32).to(dt))
    d["g_raw"] = 2.0 * torch.randn(*((B, T, H, K) if gate == "channel" else (B, T, H)), **f32)
    d["b_raw"] = torch.randn(B, T, H, **f32)
    d["w_q"] = 0.5 * torch.randn(H * K, 4, **f32)
    d["w_k"] = 0.5 * torch.randn(H * K, 4, **f32)
    d["w_v"] = 0.5 * torch.randn(H * V, 4, **f32)
    if state:
        d["cs_q"] = torch.randn(B, 3, H * K, **f32).to(dt)
        d["cs_k"] = torch.randn(B, 3, H * K, **f32).to(dt)
        d["cs_v"] = torch.randn(B, 3, H * V, **f32).to(dt)
    else:
        d["cs_q"] = d["cs_k"] = d["cs_v"] = None
    return {n: (x.contiguous() if x is not None else None) for n, x in d.items()}
