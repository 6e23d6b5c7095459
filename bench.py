"""Throughput of the Gated DeltaNet mixer forward on one MI355X.

A step is one chunkwise forward over the long-prefill workload: B=1, H=48,
T=262144 tokens, d_k=d_v=128, chunk 64, per-key-channel gate
g = -min(softplus(N(0,2)), 5), bf16 k/v, fp32 g/beta and a random fp32 S0,
returning the final state (3 MiB per layer), through gdn_chunk_fwd_ws (the
sequence-parallel form: segments of each sequence reduced to affine state maps,
combined in order).  Inputs are synthetic, seeded and resident in HBM before the
timed region.  ``value`` is tokens/s of that step (B*T tokens; a token counts
once across all heads) in millions.

The same run times, each as its own entry: the same prefill returning o as well
(sequential kernels), the scalar-gate prefill B=8 H=12 T=8192 and the
per-channel prefill B=16 H=8 T=2048 (o and S_T), the fused recurrent decode step
(256 sequences x 48 heads, 64 chained in-place steps), the multi-token verify
step, the chunkwise backward and the prologue; and the fp64 CPU oracle on a
bounded sample of the headline workload.

Timing: ``--warmup`` untimed launches, then more untimed launches until the
launch times have settled (the clocks of a fresh device ramp over the first few
tens of milliseconds; the count is recorded), then ``--steps`` launches, each
bracketed by its own pair of HIP events on the stream the kernels run on, with a
512 MB buffer written before each launch (outside the events) so that the 256 MB
last-level cache holds none of the inputs.  Mean and median per launch are
reported; ``value`` and the roofline use the mean.

Prints one JSON line.  Options: --gpus (1 only), --steps, --warmup, --no-cpu,
--only {all,headline,chunk,decode,verify,bwd,prologue}.
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA
CHUNK = 64
CSRC = os.path.join(ROOT, "gated_deltanet_layer_amd", "csrc")
FLUSH_BYTES = 512 << 20        # twice the 256 MB last-level cache

# HBM bytes per launch from rocprofv3 --pmc, one pass of FETCH_SIZE and one of
# WRITE_SIZE (KiB per dispatch) on this script's own workloads, scaled by 2.0
# (FETCH_SIZE) and 1.0 (WRITE_SIZE): the factors that make the same counters read
# 1 GiB each way for a plain elementwise copy of a 1 GiB fp32 tensor.  Each entry
# is keyed by a digest of the kernel's sources, so that a kernel changed since its
# counters were taken reports null.  For a call of several kernels the entry is
# the sum over its kernels.
MEASURED_TRAFFIC = {
    "chunk_fwd_ws_kernel<128>": (("chunk_fwd_ws.hip", "ws_common.h", "gdn_common.h",
                                  "mfma_frag.h"),
                                 "5df1a38c069ce213", 862547296),
    "chunk_fwd_wsc_kernel<128>": (("chunk_fwd_wsc.hip", "ws_common.h", "gdn_common.h",
                                   "mfma_frag.h"),
                                  "919f74973a0c28f3", 420173184),
    "recurrent_step_kernel<bf16,128,128,channel>": (("recurrent_step.hip", "gdn_common.h"),
                                                    "6075e5972b67aade", 1642950528),
    "recurrent_multi_kernel<bf16,128,128,channel>/final": (("recurrent_multi.hip", "gdn_common.h"),
                                                           "67d516fbad7f5b32", 1739688128),
    "recurrent_multi_kernel<bf16,128,128,channel>/hist": (("recurrent_multi.hip", "gdn_common.h"),
                                                          "67d516fbad7f5b32", 4159179904),
    "prologue_kernel<bf16,128,128,scalar,silu>": (("prologue.hip", "prologue.h", "prologue_ops.h",
                                                   "gdn_common.h"), "672309d493c963a2", 1307198496),
    "recurrent_step_prologue_kernel<bf16,128,128,channel,silu>": (("prologue.hip", "prologue.h",
                                                                  "prologue_ops.h", "gdn_common.h"),
                                                                 "672309d493c963a2", 1719409472),
    "chunk_fwd_seg/channel_long": (("chunk_fwd_seg.hip", "ws_common.h", "gdn_common.h",
                                    "mfma_frag.h"), "db896b910e4d7fd9", 13454399872),
    "chunk_fwd_seg/channel_long/o": (("chunk_fwd_seg.hip", "chunk_fwd_wsc.hip", "ws_common.h",
                                      "gdn_common.h", "mfma_frag.h"), "0980df048bf9396b", 33386495168),
    # the whole backward call (prep, sweeps, grad) at B4 H6 T4096, per-channel gate, bf16
    "chunk_bwd/channel_bf16": (("chunk_bwd.hip", "chunk_bwd.h", "ws_common.h", "gdn_common.h",
                                "mfma_frag.h"), "909863fa64a1af75", 1350448320),
}

# bf16 matrix-core work per launch (SQ_INSTS_VALU_MFMA_MOPS_BF16, units of 512
# flops), keyed like MEASURED_TRAFFIC.
MEASURED_MFMA_MOPS = {
    "chunk_fwd_ws_kernel<128>": (("chunk_fwd_ws.hip", "ws_common.h", "gdn_common.h",
                                  "mfma_frag.h"),
                                 "5df1a38c069ce213", 257949696),
}


def _digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _keyed(table, key, scale=1):
    if key not in table:
        return None
    files, digest, n = table[key]
    return n * scale if _digest(files) == digest else None


def measured_traffic(key):
    """Counter-measured HBM bytes per launch, or None when the kernel's sources
    changed since the counters were taken."""
    return _keyed(MEASURED_TRAFFIC, key)


def measured_mfma_flops(key):
    return _keyed(MEASURED_MFMA_MOPS, key, 512)


# ------------------------------------------------------------------ work counts
def chunk_bytes(B, T, H, K, V, es, channel, s0, want_o):
    """Algorithmic HBM bytes of one chunkwise forward: every input it needs read
    once, every output written once (q is not needed when o is not wanted)."""
    per_ht = (2 * K if want_o else K) * es + V * es + (V * es if want_o else 0) \
        + (K if channel else 1) * 4 + 4
    state = B * H * K * V * 4 * ((1 if s0 else 0) + 1)
    return B * T * H * per_ht + state


def chunk_flops(B, T, H, K, V, want_o, C=CHUNK):
    """Flops of the chunkwise forward per call, the lower-triangular C x C blocks
    counted at half ("useful") or whole ("dense"), per head-token:
      with o:  C (3K + 2V) + 6KV + C^2/3   (Gram K K^T and Q K^T, W, U, P D; K+ S,
               Q+ S, K-^T D; the triangular inverse)
      state:   C (2K + V)  + 4KV + C^2/3   (no Q K^T, P D or Q+ S)
    and the dense count doubles the C-terms."""
    a = (3 * K + 2 * V) if want_o else (2 * K + V)
    kv = (6 if want_o else 4) * K * V
    n = B * T * H
    return n * (C * a + kv + C * C / 3), n * (2 * C * a + kv + C * C / 3)


def decode_bytes(N, H, K, V, es, channel):
    per = 2 * K * V * 4 + 2 * K * es + V * es + V * es + (K if channel else 1) * 4 + 4
    return N * H * per


# ------------------------------------------------------------------ timing
class Timer:
    """Per-launch HIP-event timing with warm-up, settling and a cache flush."""

    def __init__(self, torch, steps, warmup, settle_s=0.3, max_settle=2000):
        self.torch, self.steps, self.warmup = torch, steps, warmup
        self.settle_s, self.max_settle = settle_s, max_settle
        self.flush_buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")

    def flush(self):
        self.flush_buf.zero_()

    def _ev(self):
        E = self.torch.cuda.Event
        return E(enable_timing=True), E(enable_timing=True)

    def run(self, fn, steps=None, warmup=None, per_launch=1):
        """fn() enqueues one step; returns dict of per-step ms (mean, median, min,
        max) and the warm-up actually performed.  per_launch > 1: fn enqueues
        that many launches and the times are divided by it."""
        torch = self.torch
        steps = self.steps if steps is None else steps
        warmup = self.warmup if warmup is None else warmup
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        extra, recent, t0 = 0, [], time.perf_counter()
        while extra < self.max_settle:
            e0, e1 = self._ev()
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            recent.append(e0.elapsed_time(e1))
            extra += 1
            if time.perf_counter() - t0 >= self.settle_s and len(recent) >= 8:
                last = recent[-8:]
                if (max(last) - min(last)) / min(last) < 0.03:
                    break
        pairs = [self._ev() for _ in range(steps)]
        torch.cuda.synchronize()
        for e0, e1 in pairs:
            self.flush()
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        ts = [a.elapsed_time(b) / per_launch for a, b in pairs]
        return dict(ms=statistics.fmean(ts), ms_median=statistics.median(ts), ms_min=min(ts),
                    ms_max=max(ts), steps=steps, warmup_requested=warmup,
                    warmup_performed=warmup + extra)


# ------------------------------------------------------------------ workloads
def bench_prefill(torch, gdn, timer, name, want_o, use_ws, steps=None, warmup=None):
    from gdn_inputs import CHUNK_CONFIGS, chunk_inputs
    cfg = CHUNK_CONFIGS[name]
    d = chunk_inputs(cfg, device="cuda")
    B, T, H, K, V = cfg.B, cfg.T, cfg.H, cfg.K, cfg.V
    channel = cfg.gate == "channel"
    o = torch.empty(B, T, H, V, dtype=d["v"].dtype, device="cuda") if want_o else None
    S_T = torch.empty(B, H, K, V, dtype=torch.float32, device="cuda")
    gate = gdn.GDN_GATE_CHANNEL if channel else gdn.GDN_GATE_HEAD
    nws = gdn.gdn_chunk_fwd_workspace_size(B, T, H, K, V, d["q"].dtype, gate, want_o) if use_ws else 0
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None
    if use_ws:
        run = lambda: gdn.gdn_chunk_fwd_ws(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"],
                                           o, S_T, ws)
    else:
        run = lambda: gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], o, S_T)
    t = timer.run(run, steps, warmup)
    es = 2 if cfg.dtype == "bf16" else 4
    nbytes = chunk_bytes(B, T, H, K, V, es, channel, d["S0"] is not None, want_o)
    useful, dense = chunk_flops(B, T, H, K, V, want_o)
    nseg = 1 + (nws // (B * H * (3 if want_o else 2) * K * K * 4) if nws else 0)
    if nseg > 1:
        kernels = ["chunk_fwd_seg_kernel", "seg_combine_kernel"]
        if want_o:
            kernels.append("chunk_fwd_wsc_kernel<128, true, false>")
        tkey = "chunk_fwd_seg/" + name + ("/o" if want_o else "")
    elif channel:
        kernels = ["chunk_fwd_wsc_kernel<128, %s, false>" % ("true" if want_o else "false")]
        tkey = "chunk_fwd_wsc_kernel<128>" + ("" if name == "channel_bf16" else "/" + name)
    else:
        kernels = ["chunk_fwd_ws_kernel<128, false>"]
        tkey = "chunk_fwd_ws_kernel<128>"
    s = t["ms"] / 1e3
    gbs = nbytes / s / 1e9
    inputs = d if name == "channel_long" and not want_o else None
    if inputs is None:
        del d
    ent = {
        "workload": (f"{'per-key-channel' if channel else 'scalar'}-gate GDN chunkwise forward, "
                     f"B={B} H={H} T={T} d_k=d_v={K} chunk={cfg.chunk}, {cfg.dtype} "
                     f"{'q/k/v/o' if want_o else 'k/v (q not read)'}, fp32 g/beta/state, "
                     + ("S0 ~ N(0, 0.02), " if cfg.s0_sigma else "S0 = 0, ")
                     + ("returns o and S_T" if want_o else "returns S_T only")),
        "entry": "gdn_chunk_fwd_ws" if use_ws else "gdn_chunk_fwd",
        "segments": nseg, "workspace_bytes": nws,
        "tokens": B * T, "head_tokens": B * T * H,
        "mtok_s": B * T / s / 1e6, "gbs": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
        "bytes_per_launch": nbytes,
        "useful_tflops": useful / s / 1e12, "dense_tile_tflops": dense / s / 1e12,
        "frac_bf16_peak_useful": useful / s / 1e12 / BF16_PEAK_TFLOPS,
        "kernels": kernels, "traffic": measured_traffic(tkey),
    }
    ent.update(t)
    return ent, inputs, cfg


def bench_decode(torch, gdn, timer):
    from gdn_inputs import DECODE_CONFIG, decode_inputs
    cfg = DECODE_CONFIG
    d = decode_inputs(cfg, device="cuda")
    N, H, K, V = cfg.N, cfg.H, cfg.K, cfg.V
    S = d["S0"].clone()
    o = torch.empty(cfg.steps, N, H, V, dtype=torch.bfloat16, device="cuda")
    step = [0]

    def one():   # the next step of the 64-token chain, in place; the chain restarts from S0
        s = step[0]
        if s == 0:
            S.copy_(d["S0"])
        gdn.gdn_recurrent_step(d["q"][s], d["k"][s], d["v"][s], d["g"][s], d["beta"][s], S, o[s])
        step[0] = (s + 1) % cfg.steps

    # a whole chain per measurement run so that every step index is timed; the
    # restore copy at step 0 sits inside that step's events only on the first
    # step of each chain, so time steps 1..63 of chains
    t = timer.run(one, steps=cfg.steps * 2, warmup=cfg.steps)
    nbytes = decode_bytes(N, H, K, V, 2, True)
    s = t["ms_median"] / 1e3
    ent = {"workload": f"fused recurrent decode, N={N} H={H} d_k=d_v={K}, per-channel gate, bf16 "
                       f"q/k/v/o, fp32 state in place, {cfg.steps} chained steps",
           "ms_per_step": t["ms_median"], "gbs": nbytes / s / 1e9,
           "frac_hbm": nbytes / s / 1e9 / HBM_PEAK_GBS, "bytes_per_step": nbytes,
           "traffic": measured_traffic("recurrent_step_kernel<bf16,128,128,channel>"),
           "kernel": "recurrent_step_kernel<bf16,128,128,channel>",
           "note": "median over per-step event pairs (the chain's first step also restores S0)"}
    ent.update(t)
    return ent


def bench_verify(torch, gdn, timer, M, keep_hist):
    from gdn_inputs import DECODE_CONFIG, decode_inputs
    cfg = DECODE_CONFIG.with_(steps=M)
    d = decode_inputs(cfg, device="cuda")
    N, H, K, V = cfg.N, cfg.H, cfg.K, cfg.V
    nm = lambda t: t.transpose(0, 1).contiguous()
    q, k, v, g, beta = (nm(d[n]) for n in ("q", "k", "v", "g", "beta"))
    S0 = d["S0"]
    o = torch.empty(N, M, H, V, dtype=torch.bfloat16, device="cuda")
    S_T = None if keep_hist else torch.empty_like(S0)
    S_hist = torch.empty(N, M, H, K, V, dtype=torch.float32, device="cuda") if keep_hist else None
    t = timer.run(lambda: gdn.gdn_recurrent_steps(q, k, v, g, beta, S0, o, S_T, S_hist),
                  steps=max(10, timer.steps), warmup=5)
    state = K * V * 4
    per_tok = 2 * K * 2 + V * 2 + V * 2 + K * 4 + 4
    nbytes = N * H * (state + (M * state if keep_hist else state) + M * per_tok)
    s = t["ms"] / 1e3
    ent = {"workload": f"{M} draft tokens per sequence from one state, N={N} H={H} d_k=d_v={K}, "
                       f"per-channel gate, bf16 q/k/v/o, fp32 state; "
                       + ("state after every token kept" if keep_hist else "final state written"),
           "M": M, "tokens_per_s": N * M / s, "gbs": nbytes / s / 1e9,
           "frac_hbm": nbytes / s / 1e9 / HBM_PEAK_GBS, "bytes_per_call": nbytes,
           "traffic": measured_traffic("recurrent_multi_kernel<bf16,128,128,channel>/"
                                       + ("hist" if keep_hist else "final")),
           "kernel": "recurrent_multi_kernel<bf16,128,128,channel>"}
    ent.update(t)
    return ent


def bench_decoupled(torch, gdn, timer):
    """The decoupled erase/write gates: a prefill at the per-channel workload's
    shape through gdn_chunk_fwd_decoupled, and the decode step through
    gdn_recurrent_step_decoupled.  Algorithmic bytes are those of the card's
    recurrence plus the write gate (4 bytes per head-token)."""
    from gdn_inputs import CHUNK_CONFIGS, DECODE_CONFIG, chunk_inputs, decode_inputs, decoupled_gates
    cfg = CHUNK_CONFIGS["channel_bf16"]
    d = chunk_inputs(cfg, device="cuda")
    B, T, H, K, V = cfg.B, cfg.T, cfg.H, cfg.K, cfg.V
    e, w = (x.cuda() for x in decoupled_gates((B, T, H), seed=0))
    o = torch.empty(B, T, H, V, dtype=d["v"].dtype, device="cuda")
    S_T = torch.empty(B, H, K, V, dtype=torch.float32, device="cuda")
    t = timer.run(lambda: gdn.gdn_chunk_fwd_decoupled(d["q"], d["k"], d["v"], d["g"], e, w,
                                                      d["S0"], o, S_T), max(20, timer.steps), 5)
    nbytes = chunk_bytes(B, T, H, K, V, 2, True, True, True) + B * T * H * 4
    s = t["ms"] / 1e3
    pre = {"workload": f"per-key-channel-gate chunkwise forward with decoupled erase/write gates, "
                       f"B={B} H={H} T={T} d_k=d_v={K}, bf16 q/k/v/o, fp32 g/e/w/state, "
                       "returns o and S_T",
           "entry": "gdn_chunk_fwd_decoupled", "kernel": "chunk_fwd_wsc_kernel<128, true, true>",
           "mtok_s": B * T / s / 1e6, "gbs": nbytes / s / 1e9,
           "frac_hbm": nbytes / s / 1e9 / HBM_PEAK_GBS, "bytes_per_launch": nbytes}
    pre.update(t)
    del d, o, S_T
    dc = DECODE_CONFIG
    dd = decode_inputs(dc, device="cuda")
    N, H, K, V = dc.N, dc.H, dc.K, dc.V
    e, w = (x.cuda() for x in decoupled_gates((dc.steps, N, H), seed=0))
    S = dd["S0"].clone()
    o = torch.empty(dc.steps, N, H, V, dtype=torch.bfloat16, device="cuda")
    step = [0]

    def one():
        s_ = step[0]
        if s_ == 0:
            S.copy_(dd["S0"])
        gdn.gdn_recurrent_step_decoupled(dd["q"][s_], dd["k"][s_], dd["v"][s_], dd["g"][s_],
                                         e[s_], w[s_], S, o[s_])
        step[0] = (s_ + 1) % dc.steps

    t = timer.run(one, steps=dc.steps * 2, warmup=dc.steps)
    nbytes = decode_bytes(N, H, K, V, 2, True) + N * H * 4
    s = t["ms_median"] / 1e3
    dec = {"workload": f"fused recurrent decode with decoupled erase/write gates, N={N} H={H} "
                       f"d_k=d_v={K}, per-channel gate, bf16 q/k/v/o, fp32 state in place",
           "entry": "gdn_recurrent_step_decoupled",
           "kernel": "recurrent_step_kernel<bf16,128,128,channel>",
           "ms_per_step": t["ms_median"], "gbs": nbytes / s / 1e9,
           "frac_hbm": nbytes / s / 1e9 / HBM_PEAK_GBS, "bytes_per_step": nbytes}
    dec.update(t)
    return {"prefill": pre, "decode": dec}


def bwd_bytes(B, T, H, K, V, es, channel):
    """Algorithmic HBM bytes of one chunkwise backward: q, k, v, g, beta, S0, d_o and
    dS_T read once, dq, dk, dv, dg, dbeta and dS0 written once."""
    gb = (K if channel else 1) * 4
    per_ht = (2 * K + 2 * V) * es + gb + 4          # q, k, v, d_o, g, beta
    per_ht += (2 * K + V) * es + gb + 4             # dq, dk, dv, dg, dbeta
    return B * T * H * per_ht + 3 * B * H * K * V * 4


def bench_bwd(torch, gdn, timer):
    """gdn_chunk_bwd at the card's kernel-benchmark shape (B=4 H=6 T=4096,
    d_k = d_v = 128, per-channel gate in [-5, 0], bf16), alone and after the
    forward (the card times forward and backward together)."""
    from gdn_inputs import BWD_CONFIG, chunk_inputs, grad_inputs
    cfg = BWD_CONFIG
    d = chunk_inputs(cfg, device="cuda")
    gr = grad_inputs(cfg, device="cuda")
    B, T, H, K, V = cfg.B, cfg.T, cfg.H, cfg.K, cfg.V
    nws = gdn.gdn_chunk_bwd_workspace_size(B, T, H, K, V)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    g = dict(dq=torch.empty_like(d["q"]), dk=torch.empty_like(d["k"]), dv=torch.empty_like(d["v"]),
             dg=torch.empty_like(d["g"]), dbeta=torch.empty_like(d["beta"]),
             dS0=torch.empty_like(d["S0"]))
    o = torch.empty_like(d["v"])
    S_T = torch.empty_like(d["S0"])
    bwd = lambda: gdn.gdn_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], gr["d_o"],
                                    gr["dS_T"], g["dq"], g["dk"], g["dv"], g["dg"], g["dbeta"],
                                    g["dS0"], ws)
    # the forward with its workspace: at this shape (24 slices of 64 chunks) the
    # sequence-parallel form with o
    nwf = gdn.gdn_chunk_fwd_workspace_size(B, T, H, K, V, torch.bfloat16, gdn.GDN_GATE_CHANNEL, True)
    wsf = torch.empty(nwf, dtype=torch.uint8, device="cuda") if nwf else None
    fwd = lambda: gdn.gdn_chunk_fwd_ws(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], o, S_T,
                                       wsf)
    tb = timer.run(bwd, steps=max(10, timer.steps), warmup=5)
    tf = timer.run(fwd, steps=max(10, timer.steps), warmup=5)
    tfb = timer.run(lambda: (fwd(), bwd()), steps=max(10, timer.steps), warmup=5)
    nbytes = bwd_bytes(B, T, H, K, V, 2, True)
    s = tb["ms"] / 1e3
    traffic = measured_traffic("chunk_bwd/channel_bf16")
    return {"workload": f"chunkwise backward, B={B} H={H} T={T} d_k=d_v={K} chunk=64, per-channel "
                        f"gate, bf16 q/k/v/do and dq/dk/dv, fp32 g/beta/states and their gradients, "
                        f"dL/do and dL/dS_T ~ N(0, 1)",
            "ms": tb["ms"], "ms_median": tb["ms_median"], "ms_fwd": tf["ms"], "ms_fwd_bwd": tfb["ms"],
            "mtok_s_fwd_bwd": B * T / (tfb["ms"] / 1e3) / 1e6,
            "gbs": nbytes / s / 1e9, "frac_hbm": nbytes / s / 1e9 / HBM_PEAK_GBS,
            "bytes_per_call": nbytes, "traffic_bytes": traffic,
            "traffic_x_algorithmic": None if traffic is None else traffic / nbytes,
            "workspace_bytes": nws, "fwd_workspace_bytes": nwf, "steps": tb["steps"],
            "warmup_performed": tb["warmup_performed"],
            "kernels": ["bwd_prep_kernel", "bwd_sweeps_kernel", "bwd_grad_kernel"],
            "forward": "gdn_chunk_fwd_ws: chunk_fwd_seg_kernel, seg_combine_kernel, "
                       "chunk_fwd_wsc_kernel<128, true, false> per segment"}


def prologue_bytes(B, T, H, K, V, es, channel):
    """Algorithmic HBM bytes of gdn_prologue: raw q, k, v, g, b read once, q, k, v,
    g, beta written once, the taps and the carried states once."""
    gb = (K if channel else 1) * 4
    per_ht = 2 * ((2 * K + V) * es + gb + 4)
    return B * T * H * per_ht + H * (2 * K + V) * 16 + 2 * B * 3 * H * (2 * K + V) * es


def bench_prologue(torch, gdn, timer):
    """gdn_prologue on the scalar prefill's shape (B=8 H=12 T=8192, d_k=d_v=128,
    bf16, SiLU) and, on the decode shape (N=256 H=48, per-channel gate), the fused
    decode token against the prologue and the step as two launches."""
    from gdn_inputs import prologue_inputs
    out = {}
    B, T, H, K, V = 8, 8192, 12, 128, 128
    d = prologue_inputs(B, T, H, K, V, "bf16", "head", device="cuda")
    r = {n: torch.empty_like(d[n]) for n in ("q_raw", "k_raw", "v_raw", "g_raw", "b_raw")}
    cso = [torch.empty_like(d["cs_q"]), torch.empty_like(d["cs_k"]), torch.empty_like(d["cs_v"])]
    run = lambda: gdn.gdn_prologue(d["q_raw"], d["k_raw"], d["v_raw"], d["g_raw"], d["b_raw"],
                                   d["w_q"], d["w_k"], d["w_v"], d["cs_q"], d["cs_k"], d["cs_v"],
                                   r["q_raw"], r["k_raw"], r["v_raw"], r["g_raw"], r["b_raw"],
                                   cso[0], cso[1], cso[2])
    t = timer.run(run)
    nbytes = prologue_bytes(B, T, H, K, V, 2, False)
    s = t["ms"] / 1e3
    out["chunk"] = {"workload": f"gdn_prologue, B={B} T={T} H={H} d_k=d_v={K}, scalar gate, bf16, "
                                f"SiLU, carried states in and out",
                    "gbs": nbytes / s / 1e9, "frac_hbm": nbytes / s / 1e9 / HBM_PEAK_GBS,
                    "bytes_per_call": nbytes,
                    "traffic": measured_traffic("prologue_kernel<bf16,128,128,scalar,silu>"),
                    "kernel": "prologue_kernel<bf16,128,128,scalar,silu>"}
    out["chunk"].update(t)
    # the prologue fused into the chunkwise forward, against the two launches
    # (gdn_prologue, then gdn_chunk_fwd on its outputs), on the same raw inputs
    fused = []
    for gate, (Bf, Tf, Hf) in (("head", (B, T, H)), ("channel", (16, 2048, 8))):
        if gate != "head":
            del d, r, cso
            d = prologue_inputs(Bf, Tf, Hf, K, V, "bf16", gate, device="cuda", seed=2)
            r = {n: torch.empty_like(d[n]) for n in ("q_raw", "k_raw", "v_raw", "g_raw", "b_raw")}
            cso = [torch.empty_like(d["cs_q"]), torch.empty_like(d["cs_k"]),
                   torch.empty_like(d["cs_v"])]
        S0 = 0.02 * torch.randn(Bf, Hf, K, V, device="cuda")
        o = torch.empty(Bf, Tf, Hf, V, dtype=torch.bfloat16, device="cuda")
        S_T = torch.empty_like(S0)
        raw = [d[n] for n in ("q_raw", "k_raw", "v_raw", "g_raw", "b_raw", "w_q", "w_k", "w_v",
                              "cs_q", "cs_k", "cs_v")]
        one = lambda: gdn.gdn_chunk_fwd_prologue(*raw, cso[0], cso[1], cso[2], S0, o, S_T)

        def two():
            gdn.gdn_prologue(*raw, r["q_raw"], r["k_raw"], r["v_raw"], r["g_raw"], r["b_raw"],
                             cso[0], cso[1], cso[2])
            gdn.gdn_chunk_fwd(r["q_raw"], r["k_raw"], r["v_raw"], r["g_raw"], r["b_raw"], S0, o, S_T)

        tf = timer.run(one, max(20, timer.steps), 5)
        t2 = timer.run(two, max(20, timer.steps), 5)
        fused.append({"workload": f"prologue + chunkwise forward from the raw projections, "
                                  f"B={Bf} T={Tf} H={Hf} d_k=d_v={K}, "
                                  f"{'scalar' if gate == 'head' else 'per-key-channel'} gate, bf16, "
                                  "SiLU, carried states in and out, o and S_T",
                      "entry": "gdn_chunk_fwd_prologue",
                      "kernel": f"chunk_fwd_kernel<bf16,128,{'false' if gate == 'head' else 'true'},pro>",
                      "ms_fused": tf["ms"], "ms_median_fused": tf["ms_median"],
                      "ms_two_launches": t2["ms"], "ms_median_two_launches": t2["ms_median"],
                      "mtok_s_fused": Bf * Tf / (tf["ms"] / 1e3) / 1e6})
        del S0, o, S_T
    out["chunk_fused"] = fused
    del d, r, cso
    N, H = 256, 48
    d = prologue_inputs(N, 1, H, K, V, "bf16", "channel", device="cuda", seed=1)
    d = {n: (x[:, 0].contiguous() if n in ("q_raw", "k_raw", "v_raw", "g_raw", "b_raw") else x)
         for n, x in d.items()}
    S = 0.02 * torch.randn(N, H, K, V, device="cuda")
    o = torch.empty(N, H, V, dtype=torch.bfloat16, device="cuda")
    cs = [[d["cs_q"], d["cs_k"], d["cs_v"]],
          [torch.empty_like(d["cs_q"]), torch.empty_like(d["cs_k"]), torch.empty_like(d["cs_v"])]]
    pro = {n: torch.empty(N, 1, *d[n].shape[1:], dtype=d[n].dtype, device="cuda")
           for n in ("q_raw", "k_raw", "v_raw", "g_raw", "b_raw")}
    raw1 = {n: d[n].unsqueeze(1) for n in ("q_raw", "k_raw", "v_raw", "g_raw", "b_raw")}
    j = [0]

    def fused():
        a, b = cs[j[0] % 2], cs[(j[0] + 1) % 2]
        j[0] += 1
        gdn.gdn_recurrent_step_prologue(d["q_raw"], d["k_raw"], d["v_raw"], d["g_raw"], d["b_raw"],
                                        d["w_q"], d["w_k"], d["w_v"], a[0], a[1], a[2], b[0], b[1],
                                        b[2], S, o)

    def two():
        a, b = cs[j[0] % 2], cs[(j[0] + 1) % 2]
        j[0] += 1
        gdn.gdn_prologue(raw1["q_raw"], raw1["k_raw"], raw1["v_raw"], raw1["g_raw"], raw1["b_raw"],
                         d["w_q"], d["w_k"], d["w_v"], a[0], a[1], a[2], pro["q_raw"], pro["k_raw"],
                         pro["v_raw"], pro["g_raw"], pro["b_raw"], b[0], b[1], b[2])
        gdn.gdn_recurrent_step(pro["q_raw"][:, 0], pro["k_raw"][:, 0], pro["v_raw"][:, 0],
                               pro["g_raw"][:, 0], pro["b_raw"][:, 0], S, o)

    tf = timer.run(fused)
    t2 = timer.run(two)
    state = N * H * K * V * 4
    nb = 2 * state + N * H * ((2 * K + V) * 2 + K * 4 + 4 + V * 2) + H * (2 * K + V) * 16 \
        + 2 * N * 3 * H * (2 * K + V) * 2
    out["decode"] = {"workload": f"decode token from the raw projections, N={N} H={H} "
                                 f"d_k=d_v={K}, per-channel gate, bf16, SiLU, state in place",
                     "ms_fused": tf["ms"], "ms_two_launches": t2["ms"],
                     "gbs_fused": nb / (tf["ms"] / 1e3) / 1e9,
                     "frac_hbm_fused": nb / (tf["ms"] / 1e3) / 1e9 / HBM_PEAK_GBS,
                     "bytes_per_step": nb,
                     "traffic": measured_traffic("recurrent_step_prologue_kernel<bf16,128,128,channel,silu>"),
                     "kernel": "recurrent_step_prologue_kernel<bf16,128,128,channel,silu>"}
    return out


# ------------------------------------------------------------------ CPU baseline
def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(d, cfg, target_s=12.0):
    """The fp64 oracle on a bounded sample of the headline workload: every head of
    the batch over a prefix of the sequence, final state only, from the same S0,
    one OpenMP thread per head.  Sized from a short run on all threads so that
    the sample takes about target_s seconds."""
    import oracle
    H = cfg.H
    threads = oracle.max_threads()
    S0 = d["S0"].cpu()
    host = lambda t, n: t[:, :n].cpu().contiguous()
    # one head, one thread
    n1 = 2048
    t0 = time.perf_counter()
    oracle.forward(host(d["q"], n1)[:, :, :1], host(d["k"], n1)[:, :, :1], host(d["v"], n1)[:, :, :1],
                   host(d["g"], n1)[:, :, :1], host(d["beta"], n1)[:, :, :1], S0[:, :1].contiguous(),
                   want_o=False, nthreads=1)
    r1 = n1 / (time.perf_counter() - t0)
    # every head, all threads, short prefix: the rate the host really gives
    n2 = 1024
    args = [host(d[n], n2) for n in ("q", "k", "v", "g", "beta")]
    t0 = time.perf_counter()
    oracle.forward(*args, S0, want_o=False)
    rN = H * n2 / (time.perf_counter() - t0)
    Ts = int(max(1024, min(cfg.T, target_s * rN / H)) // 64 * 64)
    args = [host(d[n], Ts) for n in ("q", "k", "v", "g", "beta")]
    t0 = time.perf_counter()
    oracle.forward(*args, S0, want_o=False)
    wall = time.perf_counter() - t0
    ht_s = H * Ts / wall
    used = min(threads, H)
    return dict(value=ht_s / H / 1e6, unit="Mtok/s", cores=used, kind="oracle",
                sample=(f"fp64 oracle, final state only, all {H} heads over the first {Ts} of "
                        f"{cfg.T} tokens of the same inputs (from the same S0): {H * Ts} "
                        f"head-tokens in {wall:.2f} s on {used} OpenMP threads; Mtok/s = "
                        f"head-tokens/s / H"),
                wall_s=wall, head_tokens_per_s=ht_s, single_thread_head_tokens_per_s=r1,
                effective_parallelism=ht_s / r1, host_cpus=len(os.sched_getaffinity(0)),
                cpu_model=_cpu_model())


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", choices=["all", "headline", "chunk", "decode", "verify", "bwd",
                                       "prologue", "decoupled"], default="all")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_deltanet_layer_amd as gdn
    if not os.path.exists(gdn.LIB_PATH):
        from gated_deltanet_layer_amd import build
        build.build()
    gdn.lib()
    torch.manual_seed(0)
    timer = Timer(torch, args.steps, args.warmup)

    out = {
        "metric": "GDN chunk fwd Mtok/s + %bf16 MFMA peak; decode step GB/s + %HBM peak",
        "value": None, "unit": "Mtok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": ("synthetic, seeded: k unit-norm, v ~ N(0,1), beta = sigmoid(N(0,1)), "
                 "g = -min(softplus(N(0,2)), 5) per key channel, S0 ~ N(0, 0.02)"),
    }
    head = head_in = head_cfg = None
    if args.only in ("all", "headline"):
        head, head_in, head_cfg = bench_prefill(torch, gdn, timer, "channel_long", False, True)
        out["value"] = head["mtok_s"]
        out["ms_per_step"] = head["ms"]
        out["config"] = {"workload": head["workload"] + " (gdn_chunk_fwd_ws, "
                         f"{head['segments']} segments per sequence)",
                         "global_batch": head_cfg.B, "seq_len": head_cfg.T, "heads": head_cfg.H,
                         "d_k": head_cfg.K, "d_v": head_cfg.V, "parallelism": "single GPU",
                         "note": ("later segments stop carrying the M part of their map once it "
                                  "has decayed to exactly zero (same result bit for bit; how soon "
                                  "depends on the gates: within a few chunks for these)")}
        out["timing"] = {k: head[k] for k in ("ms", "ms_median", "ms_min", "ms_max", "steps",
                                              "warmup_requested", "warmup_performed")}
        out["roofline"] = {"bound": "hbm", "achieved": head["gbs"], "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": head["gbs"] / HBM_PEAK_GBS,
                           "traffic": head["traffic"], "kernel": " + ".join(head["kernels"]),
                           "algorithmic_bytes_per_launch": head["bytes_per_launch"]}
        out["mfma"] = {"useful_tflops": head["useful_tflops"],
                       "dense_tile_tflops": head["dense_tile_tflops"],
                       "peak_tflops": BF16_PEAK_TFLOPS,
                       "frac_useful": head["useful_tflops"] / BF16_PEAK_TFLOPS,
                       "flop_count": "useful per head-token C(2K+V) + 4KV + C^2/3 (final state "
                                     "only; dense doubles the C-terms)"}
        out["head_tokens_per_s"] = head["head_tokens"] / (head["ms"] / 1e3)
    if args.only in ("all", "chunk"):
        ents = []
        for name, want_o, use_ws in (("channel_long", True, True), ("scalar_bf16", True, True),
                                     ("channel_bf16", True, True)):
            e, _, _ = bench_prefill(torch, gdn, timer, name, want_o, use_ws,
                                    steps=max(5, min(args.steps, 20)) if name == "channel_long"
                                    else max(20, args.steps))
            if want_o:
                e["mfma_note"] = ("useful per head-token C(3K+2V) + 6KV + C^2/3 (the triangular "
                                  "blocks counted at half); dense doubles the C-terms")
                if name == "scalar_bf16":
                    cfl = measured_mfma_flops("chunk_fwd_ws_kernel<128>")
                    e["counter_mfma_flops_per_launch"] = cfl
                    e["counter_frac_issued"] = (None if cfl is None else
                                                cfl / (e["ms"] / 1e3) / (BF16_PEAK_TFLOPS * 1e12))
            ents.append(e)
        out["chunk"] = ents
        if out["value"] is None:
            out["value"], out["ms_per_step"] = ents[0]["mtok_s"], ents[0]["ms"]
            out["config"] = {"workload": ents[0]["workload"]}
    if args.only in ("all", "decode"):
        out["decode"] = bench_decode(torch, gdn, timer)
        if out["value"] is None:
            out["value"], out["unit"] = out["decode"]["gbs"], "GB/s"
            out["ms_per_step"] = out["decode"]["ms_per_step"]
            out["config"] = {"workload": out["decode"]["workload"]}
    if args.only in ("all", "verify"):
        ver = [bench_verify(torch, gdn, timer, 4, False), bench_verify(torch, gdn, timer, 4, True)]
        if "decode" in out:
            for x in ver:   # the same tokens as M one-token decode steps
                x["vs_single_steps"] = x["M"] * out["decode"]["ms_per_step"] / x["ms"]
        out["verify"] = ver
    if args.only in ("all", "bwd"):
        out["backward"] = bench_bwd(torch, gdn, timer)
    if args.only in ("all", "prologue"):
        out["prologue"] = bench_prologue(torch, gdn, timer)
    if args.only in ("all", "decoupled"):
        out["decoupled"] = bench_decoupled(torch, gdn, timer)
    if head_in is not None and not args.no_cpu:
        torch.cuda.synchronize()
        out["cpu_baseline"] = cpu_baseline(head_in, head_cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
