"""GPU parity of the sequence-parallel chunkwise forward (gdn_chunk_fwd_ws for a
final-state-only call): the sequence of each (b, h) cut into segments that run
at once, each later segment reduced to its affine map S -> M S + N, the maps
applied in order in fp32.

Every case compares the final state with the fp64 oracle (per-slice relative
error, 2e-2 for bf16 inputs with fp32 state) and with the sequential kernels'
result (gdn_chunk_fwd), and names the number of segments the call used.
"""
import sys

import numpy as np
import pytest
import torch

import gated_deltanet_layer_amd as gdn
import oracle
from gdn_inputs import CHUNK_CONFIGS, ChunkConfig, chunk_inputs
from tests.parity import TOL_BF16, slice_rel, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dev(d):
    return {k: (None if v is None else v.to(DEV)) for k, v in d.items()}


def _nseg(cfg):
    n = gdn.gdn_chunk_fwd_workspace_size(cfg.B, cfg.T, cfg.H, cfg.K, cfg.V, torch.bfloat16,
                                         gdn.GDN_GATE_CHANNEL, False)
    per = cfg.B * cfg.H * 2 * cfg.K * cfg.K * 4
    return 1 + n // per if n else 1


def _state_only(d):
    """(S_T from the segment form, S_T from the sequential kernels)."""
    _, S_seg = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], want_o=False)
    _, S_seq = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], want_o=False,
                             workspace=False)
    torch.cuda.synchronize()
    return S_seg, S_seq


def _check(cfg, d, label, oracle_heads=None):
    nseg = _nseg(cfg)
    _say(f"[seg] {label}: B{cfg.B} H{cfg.H} T{cfg.T}, {nseg} segments")
    assert nseg >= 2, "case does not exercise the segment form"
    S_seg, S_seq = _state_only(d)
    assert torch.isfinite(S_seg).all()
    e_seq = slice_rel(to_np(S_seg), to_np(S_seq), (0, 1))
    # the oracle in groups of at most 8 heads, a progress line after each
    heads = list(range(cfg.H)) if oracle_heads is None else list(oracle_heads)
    e_or = e_seq_or = 0.0
    for i in range(0, len(heads), 8):
        hs = heads[i:i + 8]
        sel = lambda x: x[:, :, hs].contiguous().cpu()
        S0 = d["S0"]
        S0h = None if S0 is None else S0[:, hs].cpu()
        kh = sel(d["k"])
        # q only enters o, which a final-state call does not compute: k stands in
        _, rS = oracle.forward(kh, kh, sel(d["v"]), sel(d["g"]), sel(d["beta"]), S0h, want_o=False)
        e_or = max(e_or, slice_rel(to_np(S_seg[:, hs]), rS, (0, 1)))
        e_seq_or = max(e_seq_or, slice_rel(to_np(S_seq[:, hs]), rS, (0, 1)))
        _say(f"[seg] {label}: oracle on heads {hs[0]}..{hs[-1]} done")
    _say(f"[seg] {label}: err vs oracle {e_or:.3e} (sequential kernels {e_seq_or:.3e}), "
         f"segment form vs sequential {e_seq:.3e}")
    assert e_or <= TOL_BF16 and e_seq <= TOL_BF16
    return e_or


def _cfg(B, H, T, s0=0.02, **kw):
    return ChunkConfig("seg", B=B, H=H, T=T, K=128, V=128, dtype="bf16", gate="channel",
                       g_sigma=2.0, g_cap=5.0, s0_sigma=s0, **kw)


@pytest.mark.parametrize("B,H,T,s0", [
    (1, 2, 2048, 0.02),      # four segments of 8 chunks
    (1, 2, 4196, 0.0),       # eight segments, the last one ragged (a partial last chunk), S0 absent
    (2, 3, 8192, 0.02),      # sixteen segments, six sequences
    (1, 1, 4096 + 1, 0.1),   # one head, one token in the last chunk
])
def test_segments_match_oracle(B, H, T, s0):
    cfg = _cfg(B, H, T, s0)
    _check(cfg, _dev(chunk_inputs(cfg)), f"random T{T}")


def test_segments_slow_decay():
    """g scaled by 0.01: the state (and each segment's M) carries across many
    chunks, so every segment boundary matters."""
    cfg = _cfg(1, 2, 8192, 0.05, g_scale=0.01)
    _check(cfg, _dev(chunk_inputs(cfg)), "slow decay")


def test_segments_no_decay():
    """g = 0: each segment's M is a product of (I - beta k k^T) factors only."""
    cfg = _cfg(1, 2, 4096, 0.05, g_scale=0.0)
    _check(cfg, _dev(chunk_inputs(cfg)), "g = 0")


def test_segments_channel_gate_extremes():
    """Half the key channels never decay (g = 0), the other half at the clamp
    (g = -5): both ends of the gate's domain (Atomic-GDN2 card, section 2.1)."""
    cfg = _cfg(1, 2, 4096, 0.1)
    d = _dev(chunk_inputs(cfg))
    g = torch.zeros_like(d["g"])
    g[..., 1::2] = -5.0
    d["g"] = g
    _check(cfg, d, "g in {0, -5}")


def test_segments_in_place_and_deterministic():
    cfg = _cfg(1, 3, 4096, 0.05)
    d = _dev(chunk_inputs(cfg))
    _say(f"[seg] in place / determinism, {_nseg(cfg)} segments")
    _, S1 = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], want_o=False)
    _, S2 = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], want_o=False)
    S_io = d["S0"].clone()
    n = gdn.gdn_chunk_fwd_workspace_size(cfg.B, cfg.T, cfg.H, cfg.K, cfg.V, torch.bfloat16,
                                         gdn.GDN_GATE_CHANNEL, False)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    gdn.gdn_chunk_fwd_ws(d["q"], d["k"], d["v"], d["g"], d["beta"], S_io, None, S_io, ws)
    torch.cuda.synchronize()
    assert torch.equal(S1, S2)
    assert torch.equal(S_io, S1)


@pytest.mark.timeout(900)
def test_long_prefill_segments_48_heads():
    """The 262,144-token, 48-head prefill (final state only, random S0) in the
    launch configuration the bench times: every head against the sequential
    kernels' state and against the fp64 oracle over the whole sequence."""
    cfg = CHUNK_CONFIGS["channel_long"]
    d = chunk_inputs(cfg, device=DEV)
    _check(cfg, d, "long prefill")


# --- the sequence-parallel form of a call that also writes o ----------------------------
def _gpu_rel(x, ref):
    """Per-batch-row slice_rel of one head's [B, T, V] output, on the GPU; also
    checks that x is finite."""
    x, ref = x.float(), ref.float()
    assert torch.isfinite(x).all()
    err = (x - ref).abs().amax(dim=(1, 2))
    scale = ref.abs().amax(dim=(1, 2))
    return float((err / torch.where(scale > 0, scale, torch.ones_like(scale))).max())


def _with_o(d):
    """(o, S_T) from the segment form and from the sequential kernels."""
    o_seg, S_seg = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], want_o=True)
    o_seq, S_seq = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], want_o=True,
                                 workspace=False)
    torch.cuda.synchronize()
    return o_seg, S_seg, o_seq, S_seq


def _check_o(cfg, d, label, oracle_heads=None):
    n = gdn.gdn_chunk_fwd_workspace_size(cfg.B, cfg.T, cfg.H, cfg.K, cfg.V, torch.bfloat16,
                                         gdn.GDN_GATE_CHANNEL, True)
    nseg = 1 + n // (cfg.B * cfg.H * 3 * cfg.K * cfg.K * 4) if n else 1
    _say(f"[seg+o] {label}: B{cfg.B} H{cfg.H} T{cfg.T}, {nseg} segments")
    assert nseg >= 2, "case does not exercise the segment form"
    o_seg, S_seg, o_seq, S_seq = _with_o(d)
    # segment form against the sequential kernels on every head, reduced on the
    # GPU (the long prefill's o is 1.6 G elements)
    e_o = max(_gpu_rel(o_seg[:, :, h], o_seq[:, :, h]) for h in range(cfg.H))
    assert torch.isfinite(S_seg).all()
    e_S = slice_rel(to_np(S_seg), to_np(S_seq), (0, 1))
    _say(f"[seg+o] {label}: vs sequential o {e_o:.3e} S_T {e_S:.3e}; oracle next")
    heads = list(range(cfg.H)) if oracle_heads is None else oracle_heads
    hs = lambda x: x[:, :, heads].contiguous().cpu()
    S0 = d["S0"]
    ro, rS = oracle.forward(hs(d["q"]), hs(d["k"]), hs(d["v"]), hs(d["g"]), hs(d["beta"]),
                            None if S0 is None else S0[:, heads].cpu())
    eo_or = slice_rel(to_np(o_seg[:, :, heads]), ro, (0, 2))
    eS_or = slice_rel(to_np(S_seg[:, heads]), rS, (0, 1))
    _say(f"[seg+o] {label}: vs oracle o {eo_or:.3e} S_T {eS_or:.3e}")
    assert max(e_o, e_S, eo_or, eS_or) <= TOL_BF16


@pytest.mark.parametrize("B,H,T,s0", [
    (1, 2, 2048, 0.02),      # four segments
    (1, 2, 4196, 0.0),       # eight segments, the last one ragged, S0 absent
    (2, 3, 8192, 0.02),      # sixteen segments, six sequences
    (4, 6, 4096, 0.02),      # the backward benchmark's forward: eight segments, 24 sequences
])
def test_segments_with_o_match(B, H, T, s0):
    cfg = _cfg(B, H, T, s0)
    _check_o(cfg, _dev(chunk_inputs(cfg)), f"random T{T}")


def test_segments_with_o_slow_decay():
    cfg = _cfg(1, 2, 8192, 0.05, g_scale=0.01)
    _check_o(cfg, _dev(chunk_inputs(cfg)), "slow decay")


def test_segments_with_o_in_place_state_runs_sequentially():
    """S_T = S0 with o: the o pass would need S0 after it is overwritten, so the
    call runs the sequential kernels (bit for bit gdn_chunk_fwd)."""
    cfg = _cfg(1, 2, 4096, 0.05)
    d = _dev(chunk_inputs(cfg))
    n = gdn.gdn_chunk_fwd_workspace_size(cfg.B, cfg.T, cfg.H, cfg.K, cfg.V, torch.bfloat16,
                                         gdn.GDN_GATE_CHANNEL, True)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    S_io = d["S0"].clone()
    o = torch.empty_like(d["v"])
    gdn.gdn_chunk_fwd_ws(d["q"], d["k"], d["v"], d["g"], d["beta"], S_io, o, S_io, ws)
    o2, S2 = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], workspace=False)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(S_io, S2)


@pytest.mark.timeout(600)
def test_long_prefill_with_o_segments_48_heads():
    """The 262,144-token, 48-head prefill writing o and S_T: every head against the
    sequential kernels, three heads against the fp64 oracle."""
    cfg = CHUNK_CONFIGS["channel_long"]
    d = chunk_inputs(cfg, device=DEV)
    _check_o(cfg, d, "long prefill", oracle_heads=[0, 17, 47])
