"""Throughput of the Gated DeltaNet mixer forward on one MI355X.

A step is one chunkwise forward (the prefill hot path) over the scalar-gate
workload B=8, H=12, T=8192, d_k=d_v=128, chunk 64, bf16 q/k/v/o with fp32
g/beta/state, synthetic seeded inputs resident in HBM.  ``value`` is tokens/s
of that step (B*T tokens per step) in millions.  The same run also times the
fused recurrent decode step (256 sequences x 48 heads of 128x128 fp32 state, 64
chained in-place steps) and reports its HBM bandwidth, and times the fp64 CPU
oracle on a bounded sample of the prefill workload.

Prints one JSON line.  Options: --gpus (1 only), --steps (100), --warmup (50:
the clocks settle over the first tens of launches),
--no-cpu (skip the CPU baseline), --only {all,chunk,decode}.
"""
import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA
CHUNK = 64
CSRC = os.path.join(ROOT, "gated_deltanet_layer_amd", "csrc")

# HBM bytes per launch read from rocprofv3 --pmc, one pass of FETCH_SIZE and one
# of WRITE_SIZE (KiB per dispatch) on this script's own workloads.  FETCH_SIZE
# is scaled by 2.0 and WRITE_SIZE by 1.0: the factors that make the same counters
# read 1 GiB in and 1 GiB out for a plain elementwise copy of a 1 GiB fp32
# tensor.  Each entry is keyed by a digest of the kernel's sources, so that a
# kernel changed since its counters were taken reports null.
MEASURED_TRAFFIC = {
    "chunk_fwd_ws_kernel<128>": (("chunk_fwd_ws.hip", "ws_common.h", "gdn_common.h",
                                  "mfma_frag.h"),
                                 "34acdf37d6007014", 862390784),
    # the B=16 H=8 T=2048 channel-gate case (o and S_T written)
    "chunk_fwd_wsc_kernel<128>": (("chunk_fwd_wsc.hip", "ws_common.h", "gdn_common.h",
                                   "mfma_frag.h"),
                                  "4db84347cb4fcae9", 420155567),
    # the B=1 H=48 T=262144 channel-gate case (S_T only, from a random S0; no q read)
    "chunk_fwd_wsc_kernel<128>/long": (("chunk_fwd_wsc.hip", "ws_common.h", "gdn_common.h",
                                        "mfma_frag.h"),
                                       "4db84347cb4fcae9", 14202992153),
    "recurrent_step_kernel<bf16,128,128,channel>": (("recurrent_step.hip", "gdn_common.h"),
                                                    "1864f0aa1a777d85", 1642879983),
    # M = 4 draft tokens on the decode shape: final state only / every token's state
    "recurrent_multi_kernel<bf16,128,128,channel>/final": (("recurrent_multi.hip", "gdn_common.h"),
                                                           "e96c18f898c72e85", 1739625626),
    "recurrent_multi_kernel<bf16,128,128,channel>/hist": (("recurrent_multi.hip", "gdn_common.h"),
                                                          "e96c18f898c72e85", 4158918874),
    # the chunk-mode prologue at B8 H12 T8192 (scalar gate) and the fused decode token
    "prologue_kernel<bf16,128,128,scalar,silu>": (("prologue.hip", "prologue.h", "gdn_common.h"),
                                                  "1fb5d0b92490e05a", 1307185835),
    "recurrent_step_prologue_kernel<bf16,128,128,channel,silu>": (("prologue.hip", "prologue.h",
                                                                  "gdn_common.h"), "1fb5d0b92490e05a", 1719304713),
}


# bf16 matrix-core work per launch of the headline kernel from rocprofv3
# (SQ_INSTS_VALU_MFMA_MOPS_BF16, in units of 512 flops), keyed like
# MEASURED_TRAFFIC on the kernel's sources.
MEASURED_MFMA_MOPS = {
    "chunk_fwd_ws_kernel<128>": (("chunk_fwd_ws.hip", "ws_common.h", "gdn_common.h",
                                  "mfma_frag.h"),
                                 "34acdf37d6007014", 257949696),
}


def _sources_match(files, digest):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16] == digest


def measured_mfma_flops(kernel):
    """Counter-measured bf16 MFMA flops per launch of ``kernel``, or None when
    its sources changed since the counters were taken."""
    if kernel not in MEASURED_MFMA_MOPS:
        return None
    files, digest, mops = MEASURED_MFMA_MOPS[kernel]
    return mops * 512 if _sources_match(files, digest) else None


def measured_traffic(kernel):
    """Counter-measured HBM bytes per launch of ``kernel``, or None when the
    kernel's sources no longer match the ones the counters were taken on."""
    import hashlib
    if kernel not in MEASURED_TRAFFIC:
        return None
    files, digest, nbytes = MEASURED_TRAFFIC[kernel]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return nbytes if h.hexdigest()[:16] == digest else None


def chunk_bytes(B, T, H, K, V, es, channel, s0, so):
    """Algorithmic HBM bytes of one chunkwise forward: every input read once,
    every output written once."""
    per_ht = 2 * K * es + V * es + V * es + (K if channel else 1) * 4 + 4
    state = B * H * K * V * 4 * ((1 if s0 else 0) + (1 if so else 0))
    return B * T * H * per_ht + state


def chunk_flops(B, T, H, K, V, C=CHUNK):
    """Flops per head-token of the formulation the kernel runs, lower-triangular
    C x C blocks counted at half ("useful") or whole ("dense"):
    Gram K K^T and Q K^T (2 C K), K+ S, Q+ S and K-^T D (6 K V), Tm X and P D (2 C V),
    the triangular inverse (C^2 / 3)."""
    useful = C * (2 * K + 2 * V) + 6 * K * V + C * C / 3
    dense = 2 * C * (2 * K + 2 * V) + 6 * K * V + C * C / 3
    n = B * T * H
    return n * useful, n * dense


def decode_bytes(N, H, K, V, es, channel):
    per = 2 * K * V * 4 + 2 * K * es + V * es + V * es + (K if channel else 1) * 4 + 4
    return N * H * per


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def bench_chunk(torch, gdn, steps, warmup):
    from gdn_inputs import CHUNK_CONFIGS, chunk_inputs
    cfg = CHUNK_CONFIGS["scalar_bf16"]
    d = chunk_inputs(cfg, device="cuda")
    B, T, H, K, V = cfg.B, cfg.T, cfg.H, cfg.K, cfg.V
    o = torch.empty(B, T, H, V, dtype=torch.bfloat16, device="cuda")
    S_T = torch.empty(B, H, K, V, dtype=torch.float32, device="cuda")
    run = lambda: gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], o, S_T)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = _events(torch)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = chunk_bytes(B, T, H, K, V, 2, False, d["S0"] is not None, True)
    useful, dense = chunk_flops(B, T, H, K, V)
    s = ms / 1e3
    return dict(cfg=cfg, ms=ms, tokens=B * T, head_tokens=B * T * H, bytes=nbytes,
                gbs=nbytes / s / 1e9, useful_tflops=useful / s / 1e12,
                dense_tflops=dense / s / 1e12, inputs=d)


def bench_channel(torch, gdn, name, steps, warmup):
    """Per-key-channel-gate chunkwise forward on one of the channel configs, timed
    like the headline case: o and S_T for the batched case, only S_T (from a
    random S0) for the long prefill, which then reads no q."""
    from gdn_inputs import CHUNK_CONFIGS, chunk_inputs
    cfg = CHUNK_CONFIGS[name]
    d = chunk_inputs(cfg, device="cuda")
    B, T, H, K, V = cfg.B, cfg.T, cfg.H, cfg.K, cfg.V
    want_o = d["S0"] is None
    o = torch.empty(B, T, H, V, dtype=torch.bfloat16, device="cuda") if want_o else None
    S_T = torch.empty(B, H, K, V, dtype=torch.float32, device="cuda")
    run = lambda: gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], o, S_T)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = _events(torch)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    es = 2
    # q is read only when o is wanted: the final state does not depend on it
    per_ht = (2 if want_o else 1) * K * es + V * es + (V * es if want_o else 0) + K * 4 + 4
    nbytes = B * T * H * per_ht + B * H * K * V * 4 * ((1 if d["S0"] is not None else 0) + 1)
    del d
    gbs = nbytes / (ms / 1e3) / 1e9
    return {"workload": f"per-key-channel-gate GDN chunkwise forward, B={B} H={H} T={T} "
                        f"d_k=d_v={K} chunk={cfg.chunk}, bf16 " + ("q/k/v/o" if want_o else "k/v (q not read)") +
                        ", fp32 g/beta/state" + (", returns S_T only from a random S0" if not want_o else ", S0=0"),
            "ms": ms, "mtok_s": B * T / (ms / 1e3) / 1e6, "gbs": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
            "bytes_per_launch": nbytes, "kernel": "chunk_fwd_wsc_kernel<128>",
            "traffic": measured_traffic("chunk_fwd_wsc_kernel<128>" + ("" if want_o else "/long")),
            "steps": steps, "warmup": warmup}


def bench_decode(torch, gdn, reps):
    from gdn_inputs import DECODE_CONFIG, decode_inputs
    cfg = DECODE_CONFIG
    d = decode_inputs(cfg, device="cuda")
    N, H, K, V = cfg.N, cfg.H, cfg.K, cfg.V
    S = d["S0"].clone()
    o = torch.empty(cfg.steps, N, H, V, dtype=torch.bfloat16, device="cuda")

    def chain():
        for s in range(cfg.steps):
            gdn.gdn_recurrent_step(d["q"][s], d["k"][s], d["v"][s], d["g"][s], d["beta"][s], S, o[s])

    chain()  # warm-up
    times = []
    for _ in range(reps):
        S.copy_(d["S0"])                      # restore the state (not timed)
        torch.cuda.synchronize()
        e0, e1 = _events(torch)
        e0.record()
        chain()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / cfg.steps)
    ms = sorted(times)[len(times) // 2]
    nbytes = decode_bytes(N, H, K, V, 2, True)
    return dict(cfg=cfg, ms_per_step=ms, bytes=nbytes, gbs=nbytes / (ms / 1e3) / 1e9)


def bench_verify(torch, gdn, M, keep_hist, reps, warmup):
    """M draft tokens per sequence from one state (gdn_recurrent_steps) on the
    decode workload's shape: o of every token plus either the final state or the
    state after every token (rollback).  S0 is left untouched (S_T is a separate
    buffer), so the same call repeats."""
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
    run = lambda: gdn.gdn_recurrent_steps(q, k, v, g, beta, S0, o, S_T, S_hist)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = _events(torch)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    state = K * V * 4
    per_tok = 2 * K * 2 + V * 2 + V * 2 + K * 4 + 4
    nbytes = N * H * (state + (M * state if keep_hist else state) + M * per_tok)
    gbs = nbytes / (ms / 1e3) / 1e9
    return {"workload": f"{M} draft tokens per sequence from one state, N={N} H={H} "
                        f"d_k=d_v={K}, per-channel gate, bf16 q/k/v/o, fp32 state; "
                        + ("state after every token kept" if keep_hist else "final state written"),
            "M": M, "ms": ms, "tokens_per_s": N * M / (ms / 1e3), "gbs": gbs,
            "frac_hbm": gbs / HBM_PEAK_GBS, "bytes_per_call": nbytes,
            "traffic": measured_traffic("recurrent_multi_kernel<bf16,128,128,channel>/"
                                        + ("hist" if keep_hist else "final")),
            "kernel": "recurrent_multi_kernel<bf16,128,128,channel>"}


def bwd_bytes(B, T, H, K, V, es, channel):
    """Algorithmic HBM bytes of one chunkwise backward: q, k, v, g, beta, S0, d_o and
    dS_T read once, dq, dk, dv, dg, dbeta and dS0 written once."""
    gb = (K if channel else 1) * 4
    per_ht = (2 * K + 2 * V) * es + gb + 4          # q, k, v, d_o, g, beta
    per_ht += (2 * K + V) * es + gb + 4             # dq, dk, dv, dg, dbeta
    return B * T * H * per_ht + 3 * B * H * K * V * 4


def bench_bwd(torch, gdn, steps, warmup):
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
    fwd = lambda: gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], o, S_T)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = _events(torch)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms_bwd = timed(bwd)
    ms_fb = timed(lambda: (fwd(), bwd()))
    nbytes = bwd_bytes(B, T, H, K, V, 2, True)
    gbs = nbytes / (ms_bwd / 1e3) / 1e9
    return {"workload": f"chunkwise backward, B={B} H={H} T={T} d_k=d_v={K} chunk=64, per-channel "
                        f"gate, bf16 q/k/v/do and dq/dk/dv, fp32 g/beta/states and their gradients, "
                        f"dL/do and dL/dS_T ~ N(0, 1)",
            "ms": ms_bwd, "ms_fwd_bwd": ms_fb, "mtok_s_fwd_bwd": B * T / (ms_fb / 1e3) / 1e6,
            "gbs": gbs, "frac_hbm": gbs / HBM_PEAK_GBS, "bytes_per_call": nbytes,
            "workspace_bytes": nws, "steps": steps, "warmup": warmup,
            "kernels": ["bwd_prep_kernel", "bwd_sweeps_kernel", "bwd_vgrad_kernel",
                        "bwd_kgrad2_kernel"]}


def prologue_bytes(B, T, H, K, V, es, channel):
    """Algorithmic HBM bytes of gdn_prologue: raw q, k, v, g, b read once, q, k, v,
    g, beta written once, the taps and the carried states once."""
    gb = (K if channel else 1) * 4
    per_ht = 2 * ((2 * K + V) * es + gb + 4)
    return B * T * H * per_ht + H * (2 * K + V) * 16 + 2 * B * 3 * H * (2 * K + V) * es


def bench_prologue(torch, gdn, steps, warmup):
    """gdn_prologue on the headline forward's shape (B=8 H=12 T=8192, d_k=d_v=128,
    scalar gate, bf16, SiLU) and, on the decode shape (N=256 H=48, per-channel
    gate), the fused decode token against the prologue and the step as two launches."""
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
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = _events(torch)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = prologue_bytes(B, T, H, K, V, 2, False)
    out["chunk"] = {"workload": f"gdn_prologue, B={B} T={T} H={H} d_k=d_v={K}, scalar gate, bf16, "
                                f"SiLU, carried states in and out",
                    "ms": ms, "gbs": nbytes / (ms / 1e3) / 1e9,
                    "frac_hbm": nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, "bytes_per_call": nbytes,
                    "traffic": measured_traffic("prologue_kernel<bf16,128,128,scalar,silu>"),
                    "kernel": "prologue_kernel<bf16,128,128,scalar,silu>"}
    del d, r, cso
    # the decode token: fused against two launches
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

    def fused(j):
        a, b = cs[j % 2], cs[(j + 1) % 2]
        gdn.gdn_recurrent_step_prologue(d["q_raw"], d["k_raw"], d["v_raw"], d["g_raw"], d["b_raw"],
                                        d["w_q"], d["w_k"], d["w_v"], a[0], a[1], a[2], b[0], b[1],
                                        b[2], S, o)

    def two(j):
        a, b = cs[j % 2], cs[(j + 1) % 2]
        gdn.gdn_prologue(raw1["q_raw"], raw1["k_raw"], raw1["v_raw"], raw1["g_raw"], raw1["b_raw"],
                         d["w_q"], d["w_k"], d["w_v"], a[0], a[1], a[2], pro["q_raw"], pro["k_raw"],
                         pro["v_raw"], pro["g_raw"], pro["b_raw"], b[0], b[1], b[2])
        gdn.gdn_recurrent_step(pro["q_raw"][:, 0], pro["k_raw"][:, 0], pro["v_raw"][:, 0],
                               pro["g_raw"][:, 0], pro["b_raw"][:, 0], S, o)

    res = {}
    for name, fn in (("fused", fused), ("two_launches", two)):
        for j in range(warmup):
            fn(j)
        torch.cuda.synchronize()
        e0, e1 = _events(torch)
        e0.record()
        for j in range(steps):
            fn(j)
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / steps
    state = N * H * K * V * 4
    nb = 2 * state + N * H * ((2 * K + V) * 2 + K * 4 + 4 + V * 2) + H * (2 * K + V) * 16 \
        + 2 * N * 3 * H * (2 * K + V) * 2
    out["decode"] = {"workload": f"decode token from the raw projections, N={N} H={H} "
                                 f"d_k=d_v={K}, per-channel gate, bf16, SiLU, state in place",
                     "ms_fused": res["fused"], "ms_two_launches": res["two_launches"],
                     "gbs_fused": nb / (res["fused"] / 1e3) / 1e9,
                     "frac_hbm_fused": nb / (res["fused"] / 1e3) / 1e9 / HBM_PEAK_GBS,
                     "bytes_per_step": nb,
                     "traffic": measured_traffic("recurrent_step_prologue_kernel<bf16,128,128,channel,silu>"),
                     "kernel": "recurrent_step_prologue_kernel<bf16,128,128,channel,silu>"}
    return out


def cpu_baseline(chunk_inputs_dev, cfg, target_s=15.0):
    """fp64 oracle on a bounded sample of the prefill workload: whole sequences of
    some (b, h) slices, one OpenMP thread per slice."""
    import oracle
    threads = oracle.max_threads()
    d = chunk_inputs_dev
    # time one slice alone to size the sample (target_s of CPU thread-time)
    one = [t[:1, :, :1].cpu().contiguous() for t in (d["q"], d["k"], d["v"], d["g"], d["beta"])]
    t0 = time.perf_counter()
    oracle.forward(*one, None, want_o=True, nthreads=1)
    t_one = time.perf_counter() - t0
    nb = int(round(target_s / max(t_one, 1e-3) / cfg.H))
    nb = max(1, min(cfg.B, nb))
    args = [t[:nb].cpu().contiguous() for t in (d["q"], d["k"], d["v"], d["g"], d["beta"])]
    nsl = nb * cfg.H
    t0 = time.perf_counter()
    oracle.forward(*args, None, want_o=True)
    wall = time.perf_counter() - t0
    head_tokens = nsl * cfg.T
    used = min(threads, nsl)
    return dict(value=head_tokens / cfg.H / wall / 1e6, unit="Mtok/s", cores=used,
                kind="oracle",
                sample=(f"fp64 oracle on {nsl} of {cfg.B * cfg.H} (b,h) slices (batch rows "
                        f"0..{nb - 1}), T={cfg.T}, same inputs: {head_tokens} head-tokens in "
                        f"{wall:.2f} s wall on {used} threads; Mtok/s = head-tokens/s / H"),
                wall_s=wall, head_tokens_per_s=head_tokens / wall,
                host_cpus=len(os.sched_getaffinity(0)))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", choices=["all", "chunk", "decode", "channel", "verify", "bwd",
                                       "prologue"], default="all")
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

    out = {
        "metric": "GDN chunk fwd Mtok/s + %bf16 MFMA peak; decode step GB/s + %HBM peak",
        "value": None, "unit": "Mtok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; q,k unit-norm, v~N(0,1), beta=sigmoid(N(0,1)), g=-softplus(N(0,1)))",
    }
    ch = None
    if args.only in ("all", "chunk"):
        ch = bench_chunk(torch, gdn, args.steps, args.warmup)
        cfg = ch["cfg"]
        out["value"] = ch["tokens"] / (ch["ms"] / 1e3) / 1e6
        out["ms_per_step"] = ch["ms"]
        out["config"] = {
            "workload": f"scalar-gate GDN chunkwise forward, B={cfg.B} H={cfg.H} T={cfg.T} "
                        f"d_k=d_v={cfg.K} chunk={cfg.chunk}, bf16 q/k/v/o, fp32 g/beta/state, S0=0",
            "global_batch": cfg.B, "seq_len": cfg.T, "heads": cfg.H, "d_k": cfg.K, "d_v": cfg.V,
            "parallelism": "single GPU"}
        kname = "chunk_fwd_ws_kernel<128>"
        out["roofline"] = {
            "bound": "hbm", "achieved": ch["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": ch["gbs"] / HBM_PEAK_GBS, "traffic": measured_traffic(kname),
            "kernel": kname, "algorithmic_bytes_per_launch": ch["bytes"]}
        out["mfma"] = {
            "useful_tflops": ch["useful_tflops"], "dense_tile_tflops": ch["dense_tflops"],
            "peak_tflops": BF16_PEAK_TFLOPS,
            "frac_useful": ch["useful_tflops"] / BF16_PEAK_TFLOPS}
        cfl = measured_mfma_flops(kname)
        out["mfma"]["counter_flops_per_launch"] = cfl
        out["mfma"]["counter_frac_issued"] = (None if cfl is None else
                                              cfl / (ch["ms"] / 1e3) / (BF16_PEAK_TFLOPS * 1e12))
        out["head_tokens_per_s"] = ch["head_tokens"] / (ch["ms"] / 1e3)
    if args.only in ("all", "decode"):
        dc = bench_decode(torch, gdn, reps=max(3, min(args.steps, 10)))
        c = dc["cfg"]
        dec = {"workload": f"fused recurrent decode, N={c.N} H={c.H} d_k=d_v={c.K}, per-channel "
                           f"gate, bf16 q/k/v/o, fp32 state in place, {c.steps} chained steps",
               "ms_per_step": dc["ms_per_step"], "gbs": dc["gbs"],
               "frac_hbm": dc["gbs"] / HBM_PEAK_GBS, "bytes_per_step": dc["bytes"],
               "traffic": measured_traffic("recurrent_step_kernel<bf16,128,128,channel>")}
        out["decode"] = dec
        if ch is None:
            out["value"] = dc["gbs"]
            out["unit"] = "GB/s"
            out["ms_per_step"] = dc["ms_per_step"]
            out["config"] = {"workload": dec["workload"]}
            out["roofline"] = {"bound": "hbm", "achieved": dc["gbs"], "peak": HBM_PEAK_GBS,
                               "unit": "GB/s", "frac": dc["gbs"] / HBM_PEAK_GBS,
                               "traffic": dec["traffic"],
                               "kernel": "recurrent_step_kernel<bf16,128,128,channel>"}
    if args.only in ("all", "verify"):
        reps = max(3, min(args.steps, 50))
        ver = [bench_verify(torch, gdn, 4, False, reps, 5), bench_verify(torch, gdn, 4, True, reps, 5)]
        if "decode" in out:
            for x in ver:   # the same tokens as M one-token decode steps
                x["vs_single_steps"] = x["M"] * out["decode"]["ms_per_step"] / x["ms"]
        out["verify"] = ver
    if args.only in ("all", "channel"):
        out["channel"] = [bench_channel(torch, gdn, "channel_bf16", args.steps, min(args.warmup, 20)),
                          bench_channel(torch, gdn, "channel_long", max(2, min(args.steps, 5)),
                                        max(1, min(args.warmup, 3)))]
        if ch is None and args.only == "channel":
            first = out["channel"][0]
            out["value"] = first["mtok_s"]
            out["ms_per_step"] = first["ms"]
            out["config"] = {"workload": first["workload"]}
    if args.only in ("all", "bwd"):
        out["backward"] = bench_bwd(torch, gdn, max(2, min(args.steps, 20)), max(1, min(args.warmup, 5)))
        if ch is None and args.only == "bwd":
            out["value"] = out["backward"]["mtok_s_fwd_bwd"]
            out["ms_per_step"] = out["backward"]["ms_fwd_bwd"]
            out["config"] = {"workload": out["backward"]["workload"]}
    if args.only in ("all", "prologue"):
        # the chunk-mode launch settles only after a few dozen launches on fresh
        # buffers: warm up as long as the headline forward does
        out["prologue"] = bench_prologue(torch, gdn, max(3, min(args.steps, 50)), max(1, min(args.warmup, 50)))
        if ch is None and args.only == "prologue":
            out["value"] = out["prologue"]["chunk"]["gbs"]
            out["unit"] = "GB/s"
            out["ms_per_step"] = out["prologue"]["chunk"]["ms"]
            out["config"] = {"workload": out["prologue"]["chunk"]["workload"]}
    if ch is not None and not args.no_cpu:
        torch.cuda.synchronize()
        cb = cpu_baseline(ch["inputs"], ch["cfg"])
        cb["cpu_model"] = platform.processor() or _cpu_model()
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
