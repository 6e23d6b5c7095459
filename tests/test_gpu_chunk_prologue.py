"""GPU parity of the prologue fused into the chunkwise forward
(gdn_chunk_fwd_prologue): raw projections in, o and S_T out.

Against the fp64 oracles chained: ``oracle.prologue.prologue`` (convolution,
activation, q/k norm, gates) followed by ``oracle.forward`` on its outputs, on
every K/V, both gates, both activations, both storage types, lengths that are
ragged, shorter than a chunk and shorter than the filter, with and without
carried convolution states.  The carried states out are copies of raw inputs
and are compared exactly.  A sequence cut in two at a chunk boundary, with the
convolution state and S_T carried across, gives the one-call results bit for
bit; and the fused call agrees with gdn_prologue followed by gdn_chunk_fwd.
"""
import sys

import numpy as np
import pytest
import torch

import gated_deltanet_layer_amd as gdn
import oracle
from gdn_inputs import prologue_inputs
from oracle import prologue as P
from tests.parity import TOL_BF16, TOL_FP32, slice_rel, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dev(d):
    return {n: (x.to(DEV) if x is not None else None) for n, x in d.items()}


def _raw(d):
    return {n: d[n] for n in ("q_raw", "k_raw", "v_raw", "g_raw", "b_raw", "w_q", "w_k", "w_v")}


def _state(d, on):
    return (d["cs_q"], d["cs_k"], d["cs_v"]) if on else None


def _reference(d, act, with_state, S0, cap=5.0):
    """oracle.prologue then oracle.forward; returns (o, S_T, prologue dict)."""
    ref = P.prologue(d["q_raw"], d["k_raw"], d["v_raw"], d["g_raw"], d["b_raw"], d["w_q"],
                     d["w_k"], d["w_v"], silu_act=act == "silu", cap=cap,
                     state_q=d["cs_q"] if with_state else None,
                     state_k=d["cs_k"] if with_state else None,
                     state_v=d["cs_v"] if with_state else None)
    o, S = oracle.forward(ref["q"], ref["k"], ref["v"], ref["g"], ref["beta"], S0)
    return o, S, ref


def _case(B, T, H, K, V, dtype, gate, act, with_state, s0=0.05, seed=0):
    d = prologue_inputs(B, T, H, K, V, dtype, gate, seed=seed)
    S0 = None
    if s0:
        gen = torch.Generator().manual_seed(seed + 11)
        S0 = s0 * torch.randn(B, H, K, V, generator=gen)
    _say(f"[chunk+prologue] B{B} T{T} H{H} K{K} V{V} {dtype} {gate} {act} "
         f"state={with_state} S0={'yes' if S0 is not None else 'no'}")
    dd = _dev(d)
    o, S_T, st = gdn.chunk_fwd_prologue(**_raw(dd), state=_state(dd, with_state),
                                        S0=None if S0 is None else S0.to(DEV), act=act)
    torch.cuda.synchronize()
    ro, rS, ref = _reference(d, act, with_state, S0)
    tol = TOL_FP32 if dtype == "fp32" else TOL_BF16
    eo = slice_rel(to_np(o), ro, (0, 2)) if T > 0 else 0.0
    eS = slice_rel(to_np(S_T), rS, (0, 1))
    _say(f"[chunk+prologue] err o {eo:.3e}, S_T {eS:.3e}")
    assert np.isfinite(to_np(S_T)).all()
    assert max(eo, eS) <= tol
    for i, n in enumerate(("state_q", "state_k", "state_v")):
        assert np.array_equal(to_np(st[i]), ref[n]), n
    return dd, o, S_T, st


@pytest.mark.parametrize("K,V", [(128, 128), (64, 128), (128, 64), (64, 64)])
@pytest.mark.parametrize("gate", ["channel", "head"])
def test_fused_bf16_matches_oracle(K, V, gate):
    _case(2, 150, 3, K, V, "bf16", gate, "silu", True, seed=K + V)


@pytest.mark.parametrize("gate", ["channel", "head"])
@pytest.mark.parametrize("act", ["silu", "none"])
def test_fused_fp32_matches_oracle(gate, act):
    _case(2, 133, 2, 64, 64, "fp32", gate, act, True, seed=3)


@pytest.mark.parametrize("T", [0, 1, 2, 3, 5, 64, 65])
def test_fused_short_and_edge_lengths(T):
    _case(2, T, 2, 128, 128, "bf16", "channel", "silu", True, seed=T)


def test_fused_without_state_or_S0_and_no_activation():
    _case(1, 200, 2, 128, 128, "bf16", "head", "none", False, s0=0.0, seed=5)


def test_fused_split_at_a_chunk_boundary_is_bitwise_one_call():
    B, T, H, K, V = 2, 256, 2, 128, 128
    d = _dev(prologue_inputs(B, T, H, K, V, "bf16", "channel", seed=7))
    S0 = 0.05 * torch.randn(B, H, K, V, device=DEV)
    st0 = (d["cs_q"], d["cs_k"], d["cs_v"])
    o, S, st = gdn.chunk_fwd_prologue(**_raw(d), state=st0, S0=S0)
    cut = 128
    part = lambda x, sl: x[:, sl].contiguous()
    first = {n: (part(x, slice(0, cut)) if n in ("q_raw", "k_raw", "v_raw", "g_raw", "b_raw") else x)
             for n, x in _raw(d).items()}
    second = {n: (part(x, slice(cut, T)) if n in ("q_raw", "k_raw", "v_raw", "g_raw", "b_raw") else x)
              for n, x in _raw(d).items()}
    o1, S1, st1 = gdn.chunk_fwd_prologue(**first, state=st0, S0=S0)
    o2, S2, st2 = gdn.chunk_fwd_prologue(**second, state=st1, S0=S1)
    torch.cuda.synchronize()
    assert torch.equal(o[:, :cut], o1) and torch.equal(o[:, cut:], o2)
    assert torch.equal(S, S2)
    for a, b in zip(st, st2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("gate", ["channel", "head"])
def test_fused_agrees_with_prologue_then_chunk(gate):
    """The fused call against the two-launch pipeline at the 8-sequence workload's
    head count and a 2048-token length."""
    B, T, H, K, V = 2, 2048, 12, 128, 128
    d = _dev(prologue_inputs(B, T, H, K, V, "bf16", gate, seed=9))
    S0 = 0.02 * torch.randn(B, H, K, V, device=DEV)
    _say(f"[chunk+prologue] fused vs two launches, {gate}")
    o, S, st = gdn.chunk_fwd_prologue(**_raw(d), state=(d["cs_q"], d["cs_k"], d["cs_v"]), S0=S0)
    r = gdn.prologue(**_raw(d), state=(d["cs_q"], d["cs_k"], d["cs_v"]))
    o2, S2 = gdn.chunk_fwd(r["q"], r["k"], r["v"], r["g"], r["beta"], S0, workspace=False)
    torch.cuda.synchronize()
    eo = slice_rel(to_np(o), to_np(o2), (0, 2))
    eS = slice_rel(to_np(S), to_np(S2), (0, 1))
    _say(f"[chunk+prologue] fused vs two launches: o {eo:.3e}, S_T {eS:.3e}")
    assert max(eo, eS) <= TOL_BF16
    for a, b in zip(st, r["state"]):
        assert torch.equal(a, b)
    # and both against the oracles on three heads
    heads = [0, 6, 11]
    hs = lambda x: x[:, :, heads].contiguous().cpu()
    ref = P.prologue(hs(d["q_raw"]), hs(d["k_raw"]), hs(d["v_raw"]), hs(d["g_raw"]), hs(d["b_raw"]),
                     torch.cat([d["w_q"].view(H, K, 4)[h] for h in heads]).cpu(),
                     torch.cat([d["w_k"].view(H, K, 4)[h] for h in heads]).cpu(),
                     torch.cat([d["w_v"].view(H, V, 4)[h] for h in heads]).cpu(),
                     state_q=d["cs_q"].view(B, 3, H, K)[:, :, heads].reshape(B, 3, -1).cpu(),
                     state_k=d["cs_k"].view(B, 3, H, K)[:, :, heads].reshape(B, 3, -1).cpu(),
                     state_v=d["cs_v"].view(B, 3, H, V)[:, :, heads].reshape(B, 3, -1).cpu())
    ro, rS = oracle.forward(ref["q"], ref["k"], ref["v"], ref["g"], ref["beta"], S0[:, heads].cpu())
    assert slice_rel(to_np(o[:, :, heads]), ro, (0, 2)) <= TOL_BF16
    assert slice_rel(to_np(S[:, heads]), rS, (0, 1)) <= TOL_BF16
