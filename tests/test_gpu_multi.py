"""GPU parity of gdn_recurrent_steps (M tokens per sequence from one state, the
verification step of speculative decoding) against the fp64 oracle's chained
decode steps, and against the one-token entry point.

Inputs are drawn as a chain of decode steps ([M, N, H, ...], gdn_inputs) and
handed to the multi-token entry in its [N, M, H, ...] layout.  The oracle runs the
same tokens as M chained recurrent steps; the state after every token (S_hist)
is the oracle's state after that many steps.
"""
import sys

import numpy as np
import pytest
import torch

import gated_deltanet_layer_amd as gdn
import oracle
from gdn_inputs import DECODE_CONFIG, decode_inputs
from tests.parity import TOL_BF16, TOL_FP32, slice_rel, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _nm(t):
    """[M, N, H, ...] -> [N, M, H, ...] contiguous."""
    return t.transpose(0, 1).contiguous()


def _inputs(N, H, K, V, M, dtype, gate, seed=0):
    cfg = DECODE_CONFIG.with_(N=N, H=H, K=K, V=V, steps=M, dtype=dtype, gate=gate,
                              g_cap=5.0 if gate == "channel" else None, g_sigma=1.0, seed=seed)
    return cfg, decode_inputs(cfg)


def _run(d, dev=DEV, S0=True, want_o=True, want_T=True, want_hist=True, in_place=False):
    q, k, v, g, beta = (_nm(d[n]).to(dev) for n in ("q", "k", "v", "g", "beta"))
    N, M, H, K = q.shape
    V = v.shape[-1]
    s0 = d["S0"].to(dev).clone() if S0 else None
    o = torch.empty(N, M, H, V, dtype=q.dtype, device=dev) if want_o else None
    S_T = (s0 if in_place else torch.empty(N, H, K, V, dtype=torch.float32, device=dev)) if want_T else None
    S_hist = torch.empty(N, M, H, K, V, dtype=torch.float32, device=dev) if want_hist else None
    gdn.gdn_recurrent_steps(q, k, v, g, beta, s0, o, S_T, S_hist)
    torch.cuda.synchronize()
    return o, S_T, S_hist


def _oracle_hist(d, S0):
    """Oracle state after each of the M tokens: [M, N, H, K, V]."""
    M = d["q"].shape[0]
    S = S0
    hist = []
    for j in range(M):
        _, S = oracle.decode(d["q"][j:j + 1], d["k"][j:j + 1], d["v"][j:j + 1], d["g"][j:j + 1],
                             d["beta"][j:j + 1], S)
        hist.append(S.copy())
    return np.stack(hist)


@pytest.mark.parametrize("K,V", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("gate", ["head", "channel"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_steps_small(K, V, gate, dtype):
    cfg, d = _inputs(5, 3, K, V, 4, dtype, gate)
    _say(f"[multi] small {K}x{V} {gate} {dtype} M=4")
    o, S_T, S_hist = _run(d)
    ro, rS = oracle.decode(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    rh = _oracle_hist(d, d["S0"])
    tol = TOL_FP32 if dtype == "fp32" else TOL_BF16
    eo = slice_rel(to_np(o).transpose(1, 0, 2, 3), ro, (0, 1, 2))
    eS = slice_rel(to_np(S_T), rS, (0, 1))
    eh = slice_rel(to_np(S_hist).transpose(1, 0, 2, 3, 4), rh, (0, 1, 2))
    _say(f"[multi] err_o={eo:.3e} err_S={eS:.3e} err_hist={eh:.3e} tol={tol:.0e}")
    assert eo <= tol and eS <= tol and eh <= tol


@pytest.mark.parametrize("M", [1, 2, 3, 7, 8])
@pytest.mark.parametrize("gate", ["head", "channel"])
def test_steps_equal_chained_single_steps(M, gate):
    """Token j of the multi-token call is computed exactly as the one-token entry
    point computes it: o, the final state and every intermediate state agree bit
    for bit with M chained gdn_recurrent_step calls."""
    _, d = _inputs(6, 4, 128, 128, M, "bf16", gate, seed=3)
    _say(f"[multi] vs chained steps M={M} {gate}")
    o, S_T, S_hist = _run(d)
    dd = {n: t.to(DEV) for n, t in d.items()}
    S = dd["S0"].clone()
    for j in range(M):
        oj = gdn.recurrent_step_(dd["q"][j], dd["k"][j], dd["v"][j], dd["g"][j], dd["beta"][j], S)
        torch.cuda.synchronize()
        assert torch.equal(o[:, j], oj), f"o of token {j}"
        assert torch.equal(S_hist[:, j], S), f"state after token {j}"
    assert torch.equal(S_T, S)


def test_steps_in_place_zero_state_and_optional_outputs():
    _, d = _inputs(3, 2, 128, 128, 5, "bf16", "channel", seed=5)
    o_ref, S_ref, H_ref = _run(d)
    # S_T written over S0
    o, S_T, _ = _run(d, in_place=True, want_hist=False)
    assert torch.equal(o, o_ref) and torch.equal(S_T, S_ref)
    # history only
    _, _, S_hist = _run(d, want_o=False, want_T=False)
    assert torch.equal(S_hist, H_ref)
    # no S0: starts from zeros
    o0, S0T, _ = _run(d, S0=False, want_hist=False)
    d0 = dict(d)
    d0["S0"] = torch.zeros_like(d["S0"])
    o1, S1T, _ = _run(d0, want_hist=False)
    assert torch.equal(o0, o1) and torch.equal(S0T, S1T)


def test_steps_zero_tokens_copies_the_state():
    _, d = _inputs(2, 3, 64, 128, 1, "fp32", "head")
    dd = {n: (t[:0] if n != "S0" else t) for n, t in d.items()}   # M = 0
    q, k, v, g, beta = (_nm(dd[n]).to(DEV) for n in ("q", "k", "v", "g", "beta"))
    S0 = d["S0"].to(DEV)
    S_T = torch.full_like(S0, float("nan"))
    gdn.gdn_recurrent_steps(q, k, v, g, beta, S0, None, S_T, None)
    torch.cuda.synchronize()
    assert torch.equal(S_T, S0)


@pytest.mark.timeout(600)
def test_steps_full_size_every_slice():
    """256 sequences x 48 heads of 128x128 fp32 state, M = 4 draft tokens with the
    per-token states kept; the oracle follows every (n, h) slice."""
    cfg = DECODE_CONFIG.with_(steps=4)
    _say(f"[multi] full N{cfg.N} H{cfg.H} M{cfg.steps}, every slice")
    d = decode_inputs(cfg, device=DEV)
    o, S_T, S_hist = _run(d)
    sel = {n: d[n].cpu() for n in ("q", "k", "v", "g", "beta")}
    S0 = d["S0"].cpu()
    _say("[multi] full: GPU done, oracle on every slice")
    ro, rS = oracle.decode(sel["q"], sel["k"], sel["v"], sel["g"], sel["beta"], S0)
    rh = _oracle_hist(sel, S0)
    eo = slice_rel(to_np(o).transpose(1, 0, 2, 3), ro, (0, 1, 2))
    eS = slice_rel(to_np(S_T), rS, (0, 1))
    eh = slice_rel(to_np(S_hist).transpose(1, 0, 2, 3, 4), rh, (0, 1, 2))
    _say(f"[multi] full: err_o={eo:.3e} err_S={eS:.3e} err_hist={eh:.3e}")
    assert eo <= TOL_BF16 and eS <= TOL_BF16 and eh <= TOL_BF16
