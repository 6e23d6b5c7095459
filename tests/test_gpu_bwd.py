"""GPU parity of gdn_chunk_bwd (the chunkwise backward) against the fp64 backward
oracle (oracle.backward: reverse mode of the recurrence, token by token).

Every gradient (dq, dk, dv, dg, dbeta, dS0) is compared slice by slice with the
parity metric of tests/parity.py, at sizes that span several chunks and a ragged
tail, for both gates, both storage types and every (K, V); then the edge cases
(lengths around the chunk size, zero length, absent S0 / dS_T / dS0) and the
card's kernel-benchmark shape (B=4 H=6 T=4096, d_k = d_v = 128) on every slice.
"""
import sys

import numpy as np
import pytest
import torch

import gated_deltanet_layer_amd as gdn
from gdn_inputs import BWD_CONFIG, ChunkConfig, chunk_inputs, grad_inputs
from oracle.backward import backward as oracle_backward
from tests.parity import TOL_BF16, TOL_FP32, slice_rel, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
# slice axes of each gradient: (b, h)
AXES = dict(dq=(0, 2), dk=(0, 2), dv=(0, 2), dg=(0, 2), dbeta=(0, 2), dS0=(0, 1))


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _cfg(B, T, H, K, V, dtype, gate, seed=0, s0=0.5):
    return ChunkConfig("bwd_case", B=B, H=H, T=T, K=K, V=V, dtype=dtype, gate=gate,
                       g_sigma=2.0 if gate == "channel" else 1.0,
                       g_cap=5.0 if gate == "channel" else None, s0_sigma=s0, seed=seed)


def _run(d, gr, S0=True, dS_T=True, want_dS0=True):
    t = {n: (x.to(DEV) if x is not None else None) for n, x in {**d, **gr}.items()}
    out = gdn.chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["S0"] if S0 else None,
                        t["d_o"], t["dS_T"] if dS_T else None, want_dS0=want_dS0)
    torch.cuda.synchronize()
    return out


def _errors(out, ref):
    return {n: slice_rel(to_np(out[n]), ref[n], AXES[n]) for n in AXES if out.get(n) is not None}


@pytest.mark.parametrize("K,V", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("gate", ["head", "channel"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_bwd_small(K, V, gate, dtype):
    cfg = _cfg(2, 150, 2, K, V, dtype, gate)      # 3 chunks, the last one of 22 tokens
    d, gr = chunk_inputs(cfg), grad_inputs(cfg)
    _say(f"[bwd] small {K}x{V} {gate} {dtype} T=150")
    out = _run(d, gr)
    ref = oracle_backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], gr["d_o"], gr["dS_T"])
    err = _errors(out, ref)
    tol = TOL_FP32 if dtype == "fp32" else TOL_BF16
    _say(f"[bwd] " + " ".join(f"{n}={e:.2e}" for n, e in err.items()) + f" tol={tol:.0e}")
    assert max(err.values()) <= tol, err


@pytest.mark.parametrize("T", [1, 63, 64, 65, 128, 200])
def test_bwd_lengths(T):
    cfg = _cfg(1, T, 3, 128, 128, "fp32", "channel", seed=T)
    d, gr = chunk_inputs(cfg), grad_inputs(cfg)
    _say(f"[bwd] length T={T}")
    out = _run(d, gr)
    ref = oracle_backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], gr["d_o"], gr["dS_T"])
    err = _errors(out, ref)
    _say(f"[bwd] " + " ".join(f"{n}={e:.2e}" for n, e in err.items()))
    assert max(err.values()) <= TOL_FP32, err


def test_bwd_without_state_and_state_gradient():
    cfg = _cfg(2, 100, 2, 64, 128, "bf16", "head", seed=4)
    d, gr = chunk_inputs(cfg), grad_inputs(cfg)
    _say("[bwd] no S0, no dS_T, no dS0")
    out = _run(d, gr, S0=False, dS_T=False, want_dS0=False)
    assert out["dS0"] is None
    ref = oracle_backward(d["q"], d["k"], d["v"], d["g"], d["beta"], None, gr["d_o"], None)
    err = _errors(out, ref)
    assert max(err.values()) <= TOL_BF16, err


def test_bwd_zero_length_passes_the_state_gradient():
    cfg = _cfg(2, 0, 3, 128, 64, "fp32", "channel")
    d, gr = chunk_inputs(cfg), grad_inputs(cfg)
    out = _run(d, gr)
    assert torch.equal(out["dS0"].cpu(), gr["dS_T"])
    out = _run(d, gr, dS_T=False)
    assert torch.count_nonzero(out["dS0"]).item() == 0


def test_bwd_is_deterministic():
    cfg = _cfg(2, 300, 2, 128, 128, "bf16", "channel", seed=9)
    d, gr = chunk_inputs(cfg), grad_inputs(cfg)
    a, b = _run(d, gr), _run(d, gr)
    for n in a:
        assert torch.equal(a[n], b[n]), n


@pytest.mark.timeout(600)
def test_bwd_benchmark_shape_every_slice():
    """B=4 H=6 T=4096 d_k=d_v=128, per-channel gate, bf16 (the card's kernel
    benchmark shape); the oracle computes every (b, h) slice."""
    cfg = BWD_CONFIG
    _say(f"[bwd] full B{cfg.B} H{cfg.H} T{cfg.T}, every slice")
    d = chunk_inputs(cfg, device=DEV)
    gr = grad_inputs(cfg, device=DEV)
    out = gdn.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], gr["d_o"], gr["dS_T"])
    torch.cuda.synchronize()
    _say("[bwd] full: GPU done, oracle on every slice")
    ref = oracle_backward(*(d[n].cpu() for n in ("q", "k", "v", "g", "beta", "S0")),
                          gr["d_o"].cpu(), gr["dS_T"].cpu())
    got = {n: x.cpu() for n, x in out.items()}
    err = _errors(got, ref)
    _say("[bwd] full: " + " ".join(f"{n}={e:.2e}" for n, e in err.items()))
    assert max(err.values()) <= TOL_BF16, err


@pytest.mark.parametrize("gval", [-5.0, 0.0])
@pytest.mark.parametrize("gate", ["channel", "head"])
def test_bwd_decay_at_the_domain_edges(gate, gval):
    """Every log-decay at the edge of the per-channel domain [-5, 0] (the
    Atomic-GDN2 card, section 2.1): the largest in-chunk decay range the pair
    products have to carry, and no decay at all."""
    cfg = _cfg(2, 200, 2, 128, 128, "fp32", gate, seed=11)
    d, gr = chunk_inputs(cfg), grad_inputs(cfg)
    d["g"] = torch.full_like(d["g"], gval)
    _say(f"[bwd] g = {gval} everywhere, {gate} gate")
    out = _run(d, gr)
    for n, t in out.items():
        assert torch.isfinite(t).all(), n
    ref = oracle_backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], gr["d_o"], gr["dS_T"])
    err = _errors(out, ref)
    _say(f"[bwd] " + " ".join(f"{n}={e:.2e}" for n, e in err.items()))
    assert max(err.values()) <= TOL_FP32, err


@pytest.mark.parametrize("K,V", [(128, 64), (64, 128)])
def test_bwd_slice_count_multiple_of_eight(K, V):
    """8 slices: the sweeps keep the value blocks of a slice on one XCD (the
    other tests use slice counts that take the plain mapping)."""
    cfg = _cfg(2, 130, 4, K, V, "fp32", "channel", seed=21)
    d, gr = chunk_inputs(cfg), grad_inputs(cfg)
    _say(f"[bwd] 8 slices {K}x{V}")
    out = _run(d, gr)
    ref = oracle_backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], gr["d_o"], gr["dS_T"])
    err = _errors(out, ref)
    _say(f"[bwd] " + " ".join(f"{n}={e:.2e}" for n, e in err.items()))
    assert max(err.values()) <= TOL_FP32, err
