"""GPU parity of the decoupled erase/write gates (gdn_chunk_fwd_decoupled,
gdn_recurrent_step_decoupled) against the fp64 oracle ``oracle.decoupled``.

Reading of the MindPattern "Gated DeltaNet" page (finding of 2026-05-22, beta
split into separate gates): S_t = (I - e_t k_t k_t^T) Diag(alpha_t) S_{t-1}
+ w_t k_t v_t^T, o_t = S_t^T q_t.  Tolerances are those of the card's recurrence
(per-slice relative error, 2e-2 for bf16 inputs, 1e-4 for fp32 inputs); every
case prints what it runs before the GPU call.
"""
import sys

import numpy as np
import pytest
import torch

import gated_deltanet_layer_amd as gdn
from oracle import decoupled as dg
from gdn_inputs import (ChunkConfig, DecodeConfig, chunk_inputs, decode_inputs, decoupled_gates,
                        hard_reset_gate)
from tests.parity import TOL_BF16, TOL_FP32, slice_rel, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dev(d):
    return {k: (None if v is None else v.to(DEV)) for k, v in d.items()}


def _tol(dtype):
    return TOL_BF16 if dtype == "bf16" else TOL_FP32


def _chunk_case(cfg, e, w, d=None, label=""):
    d = _dev(chunk_inputs(cfg)) if d is None else d
    e, w = e.to(DEV), w.to(DEV)
    _say(f"[dg] chunk {label}: B{cfg.B} H{cfg.H} T{cfg.T} K{cfg.K} V{cfg.V} {cfg.dtype} {cfg.gate}")
    o, S = gdn.chunk_fwd_decoupled(d["q"], d["k"], d["v"], d["g"], e, w, d["S0"])
    torch.cuda.synchronize()
    ro, rS = dg.forward(d["q"], d["k"], d["v"], d["g"], e, w, d["S0"])
    eo, eS = slice_rel(to_np(o), ro, (0, 2)), slice_rel(to_np(S), rS, (0, 1))
    _say(f"[dg] chunk {label}: err o {eo:.3e}, S_T {eS:.3e}")
    assert np.isfinite(to_np(o)).all() and np.isfinite(to_np(S)).all()
    assert max(eo, eS) <= _tol(cfg.dtype)
    return d, o, S


CASES = [
    # (B, H, T, K, V, dtype, gate, s0)
    (1, 2, 300, 128, 128, "bf16", "channel", 0.05),   # ragged last chunk
    (2, 2, 257, 128, 128, "bf16", "head", 0.0),        # one token in the last chunk, no S0
    (1, 3, 200, 64, 128, "bf16", "channel", 0.05),
    (1, 2, 190, 128, 64, "bf16", "head", 0.05),
    (1, 2, 150, 64, 64, "bf16", "head", 0.05),         # the scalar-gate kernel at K = 64
    (2, 1, 200, 64, 128, "bf16", "head", 0.0),
    (1, 2, 130, 64, 64, "fp32", "head", 0.05),
    (2, 1, 129, 64, 64, "fp32", "channel", 0.0),
]


@pytest.mark.parametrize("B,H,T,K,V,dtype,gate,s0", CASES)
def test_chunk_decoupled_matches_oracle(B, H, T, K, V, dtype, gate, s0):
    cfg = ChunkConfig("dg", B=B, H=H, T=T, K=K, V=V, dtype=dtype, gate=gate,
                      g_sigma=2.0 if gate == "channel" else 1.0,
                      g_cap=5.0 if gate == "channel" else None, s0_sigma=s0)
    e, w = decoupled_gates((B, T, H), seed=1)
    _chunk_case(cfg, e, w, label="random gates")


@pytest.mark.parametrize("dtype,K,gate", [("bf16", 128, "channel"), ("bf16", 128, "head"),
                                          ("fp32", 64, "channel")])
def test_chunk_equal_gates_is_the_card_recurrence(dtype, K, gate):
    """e = w = beta: the same results as gdn_chunk_fwd, within the rounding of
    w v - e K+S against beta (v - K+S)."""
    cfg = ChunkConfig("dg", B=1, H=2, T=333, K=K, V=K, dtype=dtype, gate=gate,
                      g_sigma=2.0 if gate == "channel" else 1.0,
                      g_cap=5.0 if gate == "channel" else None, s0_sigma=0.05)
    d = _dev(chunk_inputs(cfg))
    _, o, S = _chunk_case(cfg, d["beta"], d["beta"], d=d, label="e = w = beta")
    ro, rS = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], workspace=False)
    torch.cuda.synchronize()
    agree = 2e-2 if dtype == "bf16" else 1e-5
    assert slice_rel(to_np(o), to_np(ro), (0, 2)) <= agree
    assert slice_rel(to_np(S), to_np(rS), (0, 1)) <= agree


def test_chunk_no_erase_and_no_write():
    """e = 0 (the memory only adds) and w = 0 (the memory only forgets).  g is
    scaled by 0.01 so that S0 survives the 200 tokens: at the full gate scale a
    forget-only state falls below the fp32 range and its relative error says
    nothing."""
    cfg = ChunkConfig("dg", B=1, H=2, T=200, K=128, V=128, dtype="bf16", gate="channel",
                      g_sigma=2.0, g_cap=5.0, g_scale=0.01, s0_sigma=0.5)
    d = _dev(chunk_inputs(cfg))
    e, w = decoupled_gates((1, 200, 2), seed=2)
    _chunk_case(cfg, torch.zeros_like(e), w, d=d, label="e = 0")
    _chunk_case(cfg, e, torch.zeros_like(w), d=d, label="w = 0")


def test_chunk_decoupled_hard_resets():
    """Scalar log-decays down to -200 with decoupled gates."""
    cfg = ChunkConfig("dg", B=1, H=2, T=260, K=128, V=128, dtype="bf16", gate="head",
                      s0_sigma=0.05)
    d = _dev(chunk_inputs(cfg))
    d["g"] = hard_reset_gate((1, 260, 2), seed=3, device=DEV)
    e, w = decoupled_gates((1, 260, 2), seed=3)
    _chunk_case(cfg, e, w, d=d, label="hard resets")


def test_chunk_decoupled_long_sampled_heads():
    """8192 tokens, 12 heads, per-channel gate (the prefill shape of the 8-sequence
    scalar workload, one sequence): every head's state and output against the
    oracle on three heads, S_T split state passing checked on the GPU side."""
    cfg = ChunkConfig("dg", B=1, H=12, T=8192, K=128, V=128, dtype="bf16", gate="channel",
                      g_sigma=2.0, g_cap=5.0, s0_sigma=0.02)
    d = _dev(chunk_inputs(cfg))
    e, w = (x.to(DEV) for x in decoupled_gates((1, 8192, 12), seed=4))
    _say("[dg] chunk long: B1 H12 T8192 bf16 channel")
    o, S = gdn.chunk_fwd_decoupled(d["q"], d["k"], d["v"], d["g"], e, w, d["S0"])
    # the same call in two halves, the state carried through S_T
    half = 4096
    sl = lambda x: x[:, :half].contiguous()
    sr = lambda x: x[:, half:].contiguous()
    o1, S1 = gdn.chunk_fwd_decoupled(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]), sl(e),
                                     sl(w), d["S0"])
    o2, S2 = gdn.chunk_fwd_decoupled(sr(d["q"]), sr(d["k"]), sr(d["v"]), sr(d["g"]), sr(e),
                                     sr(w), S1)
    torch.cuda.synchronize()
    assert torch.equal(o[:, :half], o1) and torch.equal(o[:, half:], o2) and torch.equal(S, S2)
    heads = [0, 5, 11]
    hs = lambda x: x[:, :, heads].contiguous()
    ro, rS = dg.forward(hs(d["q"]), hs(d["k"]), hs(d["v"]), hs(d["g"]), hs(e), hs(w),
                        d["S0"][:, heads])
    eo = slice_rel(to_np(o[:, :, heads]), ro, (0, 2))
    eS = slice_rel(to_np(S[:, heads]), rS, (0, 1))
    _say(f"[dg] chunk long: err o {eo:.3e}, S_T {eS:.3e} (heads {heads})")
    assert max(eo, eS) <= TOL_BF16


# --- decode ---------------------------------------------------------------------------
def _decode_chain(cfg, e, w, d=None, label=""):
    d = _dev(decode_inputs(cfg)) if d is None else d
    e, w = e.to(DEV), w.to(DEV)
    _say(f"[dg] decode {label}: N{cfg.N} H{cfg.H} K{cfg.K} V{cfg.V} {cfg.dtype} {cfg.gate}, "
         f"{cfg.steps} steps")
    S = d["S0"].clone()
    outs = [gdn.recurrent_step_decoupled_(d["q"][s], d["k"][s], d["v"][s], d["g"][s], e[s], w[s], S)
            for s in range(cfg.steps)]
    torch.cuda.synchronize()
    ro, rS = dg.decode(d["q"], d["k"], d["v"], d["g"], e, w, d["S0"])
    eo = slice_rel(to_np(torch.stack(outs)), ro, (0, 1, 2))
    eS = slice_rel(to_np(S), rS, (0, 1))
    _say(f"[dg] decode {label}: err o {eo:.3e}, S {eS:.3e}")
    assert max(eo, eS) <= _tol(cfg.dtype)
    return d, torch.stack(outs), S


@pytest.mark.parametrize("K,V", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("gate", ["head", "channel"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_decode_decoupled_matches_oracle(K, V, gate, dtype):
    cfg = DecodeConfig("dg", N=8, H=3, K=K, V=V, steps=6, dtype=dtype, gate=gate)
    e, w = decoupled_gates((6, 8, 3), seed=5)
    _decode_chain(cfg, e, w, label="random gates")


def test_decode_equal_gates_and_edge_gates():
    cfg = DecodeConfig("dg", N=16, H=4, K=128, V=128, steps=5)
    d = _dev(decode_inputs(cfg))
    _, o, S = _decode_chain(cfg, d["beta"], d["beta"], d=d, label="e = w = beta")
    S_ref = d["S0"].clone()
    o_ref = torch.stack([gdn.recurrent_step_(d["q"][s], d["k"][s], d["v"][s], d["g"][s],
                                             d["beta"][s], S_ref) for s in range(cfg.steps)])
    torch.cuda.synchronize()
    assert slice_rel(to_np(o), to_np(o_ref), (0, 1, 2)) <= 2e-2
    assert slice_rel(to_np(S), to_np(S_ref), (0, 1)) <= 1e-5
    e, w = decoupled_gates((5, 16, 4), seed=6)
    _decode_chain(cfg, torch.zeros_like(e), w, d=d, label="e = 0")
    _decode_chain(cfg, e, torch.zeros_like(w), d=d, label="w = 0")


def test_decode_decoupled_full_shape_sampled():
    """256 sequences x 48 heads (the decode workload), 4 steps, every slice
    against the oracle."""
    cfg = DecodeConfig("dg", N=256, H=48, K=128, V=128, steps=4)
    e, w = decoupled_gates((4, 256, 48), seed=7)
    _decode_chain(cfg, e, w, label="256 x 48")
