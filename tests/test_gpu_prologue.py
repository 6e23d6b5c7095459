"""GPU parity of the prologue entry points against the fp64 prologue oracle
(oracle.prologue), alone and chained into the recurrence:

* gdn_prologue: q, k, v, g, beta and the carried states, every K/V, both gates,
  both activations, both storage types; lengths shorter than the filter; zero
  length; the state updated in place; a sequence cut in two with the state
  carried across the cut; the prologue feeding gdn_chunk_fwd end to end;
* gdn_recurrent_step_prologue: o, the new state S and the carried convolution
  states against the oracle's prologue followed by its decode step, every K/V,
  both gates, both activations, both storage types; M chained fused steps
  against the chunk-mode prologue and recurrence over the same M tokens; the
  decode workload's size on sampled sequences.
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


def _oracle(d, act, cap=5.0):
    return P.prologue(d["q_raw"], d["k_raw"], d["v_raw"], d["g_raw"], d["b_raw"], d["w_q"], d["w_k"],
                      d["w_v"], silu_act=act == "silu", cap=cap, state_q=d["cs_q"],
                      state_k=d["cs_k"], state_v=d["cs_v"])


def _check_prologue(out, ref, tol):
    err = {}
    for n, axes in (("q", (0, 2)), ("k", (0, 2)), ("v", (0, 2)), ("g", (0, 2)), ("beta", (0, 2))):
        err[n] = slice_rel(to_np(out[n]), ref[n], axes)
    assert max(err.values()) <= tol, err
    return err


@pytest.mark.parametrize("K,V", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("gate", ["channel", "head"])
@pytest.mark.parametrize("act", ["silu", "none"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_prologue_matches_oracle(K, V, gate, act, dtype):
    d = prologue_inputs(2, 70, 3, K, V, dtype, gate, seed=K + V)
    _say(f"[prologue] {K}x{V} {gate} {act} {dtype}")
    r = gdn.prologue(**{n: x for n, x in _dev(d).items() if not n.startswith("cs_")},
                     state=(d["cs_q"].to(DEV), d["cs_k"].to(DEV), d["cs_v"].to(DEV)), act=act)
    torch.cuda.synchronize()
    ref = _oracle(d, act)
    err = _check_prologue(r, ref, TOL_FP32 if dtype == "fp32" else TOL_BF16)
    _say("[prologue] " + " ".join(f"{n}={e:.2e}" for n, e in err.items()))
    # the carried states are copies of raw inputs: exact
    for i, n in enumerate(("state_q", "state_k", "state_v")):
        assert np.array_equal(to_np(r["state"][i]), ref[n]), n


@pytest.mark.parametrize("T", [0, 1, 2, 3, 5])
def test_prologue_short_sequences(T):
    d = prologue_inputs(2, T, 2, 64, 128, "fp32", "channel", seed=T)
    r = gdn.prologue(**{n: x for n, x in _dev(d).items() if not n.startswith("cs_")},
                     state=(d["cs_q"].to(DEV), d["cs_k"].to(DEV), d["cs_v"].to(DEV)))
    torch.cuda.synchronize()
    ref = _oracle(d, "silu")
    if T > 0:
        _check_prologue(r, ref, TOL_FP32)
    for i, n in enumerate(("state_q", "state_k", "state_v")):
        assert np.array_equal(to_np(r["state"][i]), ref[n]), n


def test_prologue_state_in_place_and_split_sequence():
    d = prologue_inputs(2, 40, 3, 128, 64, "bf16", "head", seed=7)
    t = _dev(d)
    base = {n: x for n, x in t.items() if not n.startswith("cs_")}
    whole = gdn.prologue(**base, state=(t["cs_q"], t["cs_k"], t["cs_v"]))
    # in place: the state buffers are read and overwritten by one call
    cs = [t["cs_q"].clone(), t["cs_k"].clone(), t["cs_v"].clone()]
    outs = {n: torch.empty_like(whole[n]) for n in ("q", "k", "v", "g", "beta")}
    gdn.gdn_prologue(base["q_raw"], base["k_raw"], base["v_raw"], base["g_raw"], base["b_raw"],
                     base["w_q"], base["w_k"], base["w_v"], cs[0], cs[1], cs[2], outs["q"], outs["k"],
                     outs["v"], outs["g"], outs["beta"], cs[0], cs[1], cs[2])
    torch.cuda.synchronize()
    for n in outs:
        assert torch.equal(outs[n], whole[n]), n
    for i in range(3):
        assert torch.equal(cs[i], whole["state"][i])
    # cut at 17: the second half continues from the first half's state
    cut = 17
    first = gdn.prologue(**{n: (x[:, :cut].contiguous() if x.dim() >= 3 and n not in ("w_q", "w_k", "w_v") else x)
                            for n, x in base.items()}, state=(t["cs_q"], t["cs_k"], t["cs_v"]))
    second = gdn.prologue(**{n: (x[:, cut:].contiguous() if x.dim() >= 3 and n not in ("w_q", "w_k", "w_v") else x)
                             for n, x in base.items()}, state=first["state"])
    torch.cuda.synchronize()
    for n in ("q", "k", "v", "g", "beta"):
        assert torch.equal(torch.cat([first[n], second[n]], dim=1), whole[n]), n
    for i in range(3):
        assert torch.equal(second["state"][i], whole["state"][i])


@pytest.mark.parametrize("gate", ["channel", "head"])
def test_prologue_feeds_chunk_fwd(gate):
    """Raw projections -> gdn_prologue -> gdn_chunk_fwd, against the oracle's
    prologue followed by its recurrence."""
    d = prologue_inputs(2, 150, 2, 128, 128, "bf16", gate, seed=3)
    t = _dev(d)
    r = gdn.prologue(**{n: x for n, x in t.items() if not n.startswith("cs_")},
                     state=(t["cs_q"], t["cs_k"], t["cs_v"]))
    o, S_T = gdn.chunk_fwd(r["q"], r["k"], r["v"], r["g"], r["beta"])
    torch.cuda.synchronize()
    ref = _oracle(d, "silu")
    # the oracle's recurrence on the oracle's prologue output, rounded to the storage type as
    # the GPU path stores it
    rq = torch.tensor(ref["q"]).to(torch.bfloat16)
    rk = torch.tensor(ref["k"]).to(torch.bfloat16)
    rv = torch.tensor(ref["v"]).to(torch.bfloat16)
    ro, rS = oracle.forward(rq, rk, rv, torch.tensor(ref["g"]).float(), torch.tensor(ref["beta"]).float())
    eo = slice_rel(to_np(o), ro, (0, 2))
    eS = slice_rel(to_np(S_T), rS, (0, 1))
    _say(f"[prologue->fwd] {gate}: err_o={eo:.2e} err_S={eS:.2e}")
    assert eo <= TOL_BF16 and eS <= TOL_BF16


def _step_oracle(d, S0, act, cap=5.0):
    """One token from the raw projections: the oracle prologue (T = 1) then the
    oracle decode step.  d holds [N, H, *] raw tensors and [N, 3, D] states."""
    one = {n: (x[:, None] if n in ("q_raw", "k_raw", "v_raw", "g_raw", "b_raw") else x)
           for n, x in d.items()}
    pr = _oracle(one, act, cap)
    o, S = oracle.decode(pr["q"].transpose(1, 0, 2, 3), pr["k"].transpose(1, 0, 2, 3),
                         pr["v"].transpose(1, 0, 2, 3),
                         np.moveaxis(pr["g"], 1, 0), pr["beta"].transpose(1, 0, 2), S0)
    return o[0], S, pr


@pytest.mark.parametrize("K,V", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("gate", ["channel", "head"])
@pytest.mark.parametrize("act", ["silu", "none"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_step_prologue_matches_oracle(K, V, gate, act, dtype):
    N, H = 5, 3
    d = prologue_inputs(N, 1, H, K, V, dtype, gate, seed=K * 3 + V)
    d = {n: (x[:, 0] if n in ("q_raw", "k_raw", "v_raw", "g_raw", "b_raw") else x) for n, x in d.items()}
    S0 = 0.3 * torch.randn(N, H, K, V, generator=torch.Generator().manual_seed(1))
    t = _dev(d)
    S = S0.to(DEV).clone()
    o = torch.empty(N, H, V, dtype=t["q_raw"].dtype, device=DEV)
    cso = [torch.empty_like(t["cs_q"]), torch.empty_like(t["cs_k"]), torch.empty_like(t["cs_v"])]
    _say(f"[step_prologue] {K}x{V} {gate} {act} {dtype}")
    gdn.gdn_recurrent_step_prologue(t["q_raw"], t["k_raw"], t["v_raw"], t["g_raw"], t["b_raw"],
                                    t["w_q"], t["w_k"], t["w_v"], t["cs_q"], t["cs_k"], t["cs_v"],
                                    cso[0], cso[1], cso[2], S, o, act=act)
    torch.cuda.synchronize()
    ro, rS, pr = _step_oracle(d, S0.numpy(), act)
    tol = TOL_FP32 if dtype == "fp32" else TOL_BF16
    eo = slice_rel(to_np(o), ro, (0, 1))
    eS = slice_rel(to_np(S), rS, (0, 1))
    _say(f"[step_prologue] err_o={eo:.2e} err_S={eS:.2e}")
    assert eo <= tol and eS <= tol
    for i, n in enumerate(("state_q", "state_k", "state_v")):
        assert np.array_equal(to_np(cso[i]), pr[n]), n


@pytest.mark.parametrize("gate", ["channel", "head"])
def test_chained_fused_steps_equal_the_chunk_mode(gate):
    """M fused decode steps (states alternating between two buffers) against
    gdn_prologue + gdn_chunk_fwd over the same M tokens."""
    N, H, K, V, M = 4, 2, 64, 128, 9          # fp32 chunk path: K = 64
    d = prologue_inputs(N, M, H, K, V, "fp32", gate, seed=5)
    t = _dev(d)
    S = torch.zeros(N, H, K, V, device=DEV)
    cs = [[t["cs_q"].clone(), t["cs_k"].clone(), t["cs_v"].clone()],
          [torch.empty_like(t["cs_q"]), torch.empty_like(t["cs_k"]), torch.empty_like(t["cs_v"])]]
    outs = []
    for j in range(M):
        a, b = cs[j % 2], cs[(j + 1) % 2]
        o = torch.empty(N, H, V, device=DEV)
        gdn.gdn_recurrent_step_prologue(t["q_raw"][:, j].contiguous(), t["k_raw"][:, j].contiguous(),
                                        t["v_raw"][:, j].contiguous(), t["g_raw"][:, j].contiguous(),
                                        t["b_raw"][:, j].contiguous(), t["w_q"], t["w_k"], t["w_v"],
                                        a[0], a[1], a[2], b[0], b[1], b[2], S, o)
        outs.append(o)
    r = gdn.prologue(**{n: x for n, x in t.items() if not n.startswith("cs_")},
                     state=(t["cs_q"], t["cs_k"], t["cs_v"]))
    o_ref, S_ref = gdn.chunk_fwd(r["q"], r["k"], r["v"], r["g"], r["beta"])
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, dim=1)
    eo = slice_rel(to_np(o_dec), to_np(o_ref), (0, 2))
    eS = slice_rel(to_np(S), to_np(S_ref), (0, 1))
    _say(f"[fused steps vs chunk mode] {gate}: err_o={eo:.2e} err_S={eS:.2e}")
    assert eo <= TOL_FP32 and eS <= TOL_FP32
    fin = cs[M % 2]
    for i, x in enumerate(r["state"]):
        assert torch.equal(fin[i], x)


@pytest.mark.timeout(600)
def test_step_prologue_decode_size_every_slice():
    """256 sequences x 48 heads, d_k = d_v = 128, bf16, per-channel gate; the
    oracle follows every sequence."""
    N, H, K, V = 256, 48, 128, 128
    d = prologue_inputs(N, 1, H, K, V, "bf16", "channel", device=DEV, seed=2)
    d = {n: (x[:, 0].contiguous() if n in ("q_raw", "k_raw", "v_raw", "g_raw", "b_raw") else x)
         for n, x in d.items()}
    S0 = 0.02 * torch.randn(N, H, K, V, device=DEV, generator=torch.Generator(device=DEV).manual_seed(3))
    S = S0.clone()
    o = torch.empty(N, H, V, dtype=torch.bfloat16, device=DEV)
    cso = [torch.empty_like(d["cs_q"]), torch.empty_like(d["cs_k"]), torch.empty_like(d["cs_v"])]
    _say("[step_prologue] full N256 H48")
    gdn.gdn_recurrent_step_prologue(d["q_raw"], d["k_raw"], d["v_raw"], d["g_raw"], d["b_raw"],
                                    d["w_q"], d["w_k"], d["w_v"], d["cs_q"], d["cs_k"], d["cs_v"],
                                    cso[0], cso[1], cso[2], S, o)
    torch.cuda.synchronize()
    _say("[step_prologue] full: GPU done, oracle on every sequence")
    sel = {n: x.cpu() for n, x in d.items()}
    ro, rS, _ = _step_oracle(sel, S0.cpu().numpy(), "silu")
    eo = slice_rel(to_np(o), ro, (0, 1))
    eS = slice_rel(to_np(S), rS, (0, 1))
    _say(f"[step_prologue] full: err_o={eo:.2e} err_S={eS:.2e}")
    assert eo <= TOL_BF16 and eS <= TOL_BF16
