"""gdn_chunk_fwd_noalloc: the final-state forward for callers that cannot
allocate, its segment maps in the library's static device buffer.

Checked through the C ABI against gdn_chunk_fwd_ws (the entry point it is a
variant of) on two calls in a row, the second smaller, and against the fp64
oracle to the bf16 bound; a call the buffer cannot hold is refused on the host.
"""
import sys

import numpy as np
import pytest
import torch

import gated_deltanet_layer_amd as gdn
import oracle
from gdn_inputs import ChunkConfig, chunk_inputs
from tests.parity import TOL_BF16, slice_rel, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _cfg(B, H, T, seed):
    return ChunkConfig("na", B=B, H=H, T=T, K=128, V=128, dtype="bf16", gate="channel",
                       g_sigma=2.0, g_cap=5.0, s0_sigma=0.05, seed=seed)


def test_noalloc_equals_workspace_entry_on_two_calls():
    # the second call is smaller, so it reuses (and must fully overwrite) what the
    # first one left in the shared buffer
    for B, H, T, seed in ((1, 8, 8192 + 37, 0), (1, 2, 2048, 1)):
        cfg = _cfg(B, H, T, seed)
        need = gdn.gdn_chunk_fwd_workspace_size(B, T, H, 128, 128, torch.bfloat16,
                                                gdn.GDN_GATE_CHANNEL, False)
        nseg = 1 + need // (B * H * 2 * 128 * 128 * 4)
        _say(f"[noalloc] B{B} H{H} T{T}: {nseg} segments, maps {need} bytes")
        assert nseg >= 2 and need <= 64 << 20
        d = {n: (None if x is None else x.to(DEV)) for n, x in chunk_inputs(cfg).items()}
        S_na = torch.empty(B, H, 128, 128, dtype=torch.float32, device=DEV)
        gdn.gdn_chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], None, S_na)
        _, S_ws = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], want_o=False)
        torch.cuda.synchronize()
        assert torch.equal(S_na, S_ws)
        _, rS = oracle.forward(*(d[n].cpu() for n in ("q", "k", "v", "g", "beta")), d["S0"].cpu(),
                               want_o=False)
        e = slice_rel(to_np(S_na), rS, (0, 1))
        _say(f"[noalloc] err vs oracle {e:.3e}")
        assert np.isfinite(to_np(S_na)).all() and e <= TOL_BF16


def test_noalloc_without_segments_runs_the_sequential_kernels():
    """o requested: no maps, the call is gdn_chunk_fwd's, bit for bit."""
    cfg = _cfg(2, 3, 300, 2)
    d = {n: (None if x is None else x.to(DEV)) for n, x in chunk_inputs(cfg).items()}
    o1 = torch.empty_like(d["v"])
    S1 = torch.empty_like(d["S0"])
    gdn.gdn_chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], o1, S1)
    o2, S2 = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], workspace=False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_noalloc_refuses_maps_past_its_buffer():
    """The 48-head, 262,144-token prefill needs 90 MiB of maps, more than the
    64 MiB buffer: refused on the host, nothing enqueued (fake addresses: the
    call must return before touching them)."""
    L = gdn.lib()
    base, sep = 1 << 44, 1 << 36
    p = [base + i * sep for i in range(8)]
    rc = L.gdn_chunk_fwd_noalloc(p[0], p[1], p[2], p[3], p[4], p[5], None, p[7],
                                 1, 262144, 48, 128, 128, 64, gdn.GDN_BF16,
                                 gdn.GDN_GATE_CHANNEL, None)
    assert rc == gdn.GDN_ENOTSUP
