"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Every case draws seeded inputs once (gdn_inputs), runs the HIP kernels on the
GPU and the oracle on the host on the same stored tensors, and compares with the
per-slice relative error of tests/parity.py: 1e-4 for fp32 inputs, 2e-2 for bf16
inputs with fp32 state, on o and on the final state.
"""
import sys

import numpy as np
import pytest
import torch

import gated_deltanet_layer_amd as gdn
import oracle
from gdn_inputs import (CHUNK_CONFIGS, DECODE_CONFIG, ChunkConfig, chunk_inputs, decode_inputs,
                        hard_reset_gate)
from tests.parity import TOL_BF16, TOL_FP32, slice_rel, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _to(d, dev):
    return {k: (None if v is None else v.to(dev)) for k, v in d.items()}


def _tol(cfg):
    return TOL_FP32 if cfg.dtype == "fp32" else TOL_BF16


def _run_chunk(cfg, d, want_o=True):
    dd = _to(d, DEV)
    o, S = gdn.chunk_fwd(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["S0"], want_o=want_o)
    torch.cuda.synchronize()
    return (to_np(o) if o is not None else None), to_np(S)


def _check_chunk(cfg, d, label):
    _say(f"[parity] {label}: B{cfg.B} H{cfg.H} T{cfg.T} K{cfg.K} V{cfg.V} {cfg.dtype} {cfg.gate}")
    o, S = _run_chunk(cfg, d)
    ro, rS = oracle.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    eo = slice_rel(o, ro, (0, 2))      # o [B,T,H,V]: slices (b, h)
    eS = slice_rel(S, rS, (0, 1))      # S [B,H,K,V]
    _say(f"[parity] {label}: err_o={eo:.3e} err_S={eS:.3e} tol={_tol(cfg):.0e}")
    assert np.isfinite(o).all() and np.isfinite(S).all()
    assert eo <= _tol(cfg) and eS <= _tol(cfg)
    return eo, eS


# ----------------------------------------------------------------------------- decode
@pytest.mark.parametrize("K,V", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("gate", ["head", "channel"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_decode_small(K, V, gate, dtype):
    cfg = DECODE_CONFIG.with_(N=5, H=3, K=K, V=V, steps=6, dtype=dtype, gate=gate,
                              g_cap=5.0 if gate == "channel" else None, g_sigma=1.0)
    d = decode_inputs(cfg)
    _say(f"[parity] decode small {K}x{V} {gate} {dtype}")
    dd = _to(d, DEV)
    S = dd["S0"].clone()
    outs = []
    for s in range(cfg.steps):
        outs.append(gdn.recurrent_step_(dd["q"][s], dd["k"][s], dd["v"][s], dd["g"][s],
                                        dd["beta"][s], S))
    torch.cuda.synchronize()
    o = to_np(torch.stack(outs))
    ro, rS = oracle.decode(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    tol = TOL_FP32 if dtype == "fp32" else TOL_BF16
    assert slice_rel(o, ro, (0, 1, 2)) <= tol
    assert slice_rel(to_np(S), rS, (0, 1)) <= tol


@pytest.mark.timeout(600)
def test_decode_full_config_every_slice():
    """256 sequences x 48 heads of 128x128 fp32 state, 64 chained in-place steps;
    the oracle follows every (n, h) slice through all 64 steps."""
    cfg = DECODE_CONFIG
    _say(f"[parity] decode full N{cfg.N} H{cfg.H} steps{cfg.steps}, every slice")
    d = decode_inputs(cfg, device=DEV)
    S = d["S0"].clone()
    o = torch.empty(cfg.steps, cfg.N, cfg.H, cfg.V, dtype=torch.bfloat16, device=DEV)
    for s in range(cfg.steps):
        gdn.gdn_recurrent_step(d["q"][s], d["k"][s], d["v"][s], d["g"][s], d["beta"][s], S, o[s])
    torch.cuda.synchronize()
    _say("[parity] decode full: GPU done, oracle on every slice")
    ro, rS = oracle.decode(d["q"].cpu(), d["k"].cpu(), d["v"].cpu(), d["g"].cpu(), d["beta"].cpu(),
                           d["S0"].cpu())
    eo = slice_rel(to_np(o), ro, (0, 1, 2))
    eS = slice_rel(to_np(S), rS, (0, 1))
    _say(f"[parity] decode full: err_o={eo:.3e} err_S={eS:.3e} over {cfg.N * cfg.H} slices")
    assert eo <= TOL_BF16 and eS <= TOL_BF16


# ----------------------------------------------------------------------------- chunk
def test_chunk_scalar_fp32_small_config():
    cfg = CHUNK_CONFIGS["scalar_fp32_small"]
    _check_chunk(cfg, chunk_inputs(cfg), "scalar fp32 B1 H2 T256")


@pytest.mark.parametrize("T", [1, 17, 63, 64, 65, 130])
@pytest.mark.parametrize("gate", ["head", "channel"])
def test_chunk_fp32_ragged(T, gate):
    cfg = ChunkConfig("t", B=2, H=3, T=T, K=64, V=64, dtype="fp32", gate=gate,
                      g_cap=5.0 if gate == "channel" else None, s0_sigma=0.1)
    _check_chunk(cfg, chunk_inputs(cfg), f"fp32 ragged T{T} {gate}")


@pytest.mark.parametrize("K,V", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("gate", ["head", "channel"])
def test_chunk_bf16_small(K, V, gate):
    cfg = ChunkConfig("t", B=2, H=4, T=200, K=K, V=V, dtype="bf16", gate=gate,
                      g_sigma=2.0 if gate == "channel" else 1.0,
                      g_cap=5.0 if gate == "channel" else None, s0_sigma=0.02)
    _check_chunk(cfg, chunk_inputs(cfg), f"bf16 small {K}x{V} {gate}")


def _check_chunk_full(cfg, label):
    """The full-size workload on the GPU in the launch configuration the bench
    times, and the oracle on every (b, h) slice of the same stored inputs."""
    _say(f"[parity] {label}: full size B{cfg.B} H{cfg.H} T{cfg.T}, every slice")
    d = chunk_inputs(cfg, device=DEV)
    o, S = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    torch.cuda.synchronize()
    o_h, S_h = to_np(o), to_np(S)
    del o, S
    host = {n: (None if x is None else x.cpu()) for n, x in d.items()}
    del d
    _say(f"[parity] {label}: GPU done, oracle on {cfg.B * cfg.H} slices")
    ro, rS = oracle.forward(host["q"], host["k"], host["v"], host["g"], host["beta"], host["S0"])
    eo = slice_rel(o_h, ro, (0, 2))
    eS = slice_rel(S_h, rS, (0, 1))
    _say(f"[parity] {label}: err_o={eo:.3e} err_S={eS:.3e} over {cfg.B * cfg.H} slices")
    assert np.isfinite(o_h).all() and np.isfinite(S_h).all()
    assert eo <= _tol(cfg) and eS <= _tol(cfg)


@pytest.mark.timeout(300)
def test_chunk_scalar_bf16_full_every_slice():
    _check_chunk_full(CHUNK_CONFIGS["scalar_bf16"], "scalar bf16")


@pytest.mark.timeout(300)
def test_chunk_channel_bf16_full_every_slice():
    _check_chunk_full(CHUNK_CONFIGS["channel_bf16"], "channel bf16")


# ----------------------------------------------------------------------------- hard resets
@pytest.mark.parametrize("dtype,K", [("bf16", 128), ("bf16", 64), ("fp32", 64)])
def test_chunk_scalar_hard_resets(dtype, K):
    cfg = ChunkConfig("reset", B=2, H=3, T=1000, K=K, V=K, dtype=dtype, gate="head", s0_sigma=0.1)
    d = chunk_inputs(cfg)
    d["g"] = hard_reset_gate(d["g"].shape, seed=123)
    assert d["g"].min().item() < -150.0
    _check_chunk(cfg, d, f"scalar hard resets {dtype} K{K}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_decode_scalar_hard_resets(dtype):
    cfg = DECODE_CONFIG.with_(N=6, H=3, K=128, V=128, steps=8, dtype=dtype, gate="head",
                              g_cap=None, g_sigma=1.0)
    d = decode_inputs(cfg)
    d["g"] = hard_reset_gate(d["g"].shape, seed=321)
    _say(f"[parity] decode scalar hard resets {dtype}")
    dd = _to(d, DEV)
    S = dd["S0"].clone()
    outs = [gdn.recurrent_step_(dd["q"][s], dd["k"][s], dd["v"][s], dd["g"][s], dd["beta"][s], S)
            for s in range(cfg.steps)]
    torch.cuda.synchronize()
    ro, rS = oracle.decode(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    tol = TOL_FP32 if dtype == "fp32" else TOL_BF16
    eo = slice_rel(to_np(torch.stack(outs)), ro, (0, 1, 2))
    eS = slice_rel(to_np(S), rS, (0, 1))
    _say(f"[parity] decode hard resets: err_o={eo:.3e} err_S={eS:.3e}")
    assert eo <= tol and eS <= tol
