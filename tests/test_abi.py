"""C-ABI library: loads, exports every declared symbol, rejects bad arguments on
the host before touching the GPU (CPU only: every call here fails validation or
is an empty no-op, so no kernel is launched)."""
import os
import re

import pytest

import gated_deltanet_layer_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(gdn.LIB_PATH):
        from gated_deltanet_layer_amd import build
        build.build()
    return gdn.lib()


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "gdn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = _declared_functions()
    assert set(names) == set(gdn.SYMBOLS)
    for n in names:
        assert hasattr(L, n), n


def test_only_declared_symbols_are_exported():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", gdn.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert {s for s in exported if s.startswith("gdn_")} == set(gdn.SYMBOLS)


def test_version_and_status_strings(L):
    assert gdn.abi_version() == 7
    assert gdn.status_str(0) == "ok"
    assert "invalid" in gdn.status_str(1)
    assert "unsupported" in gdn.status_str(2)
    assert "HIP" in gdn.status_str(3)
    assert gdn.status_str(99) == "unknown status"


# Fake, well-separated, 16-byte aligned device addresses: validation only looks
# at their values, and every call below returns before any HIP call.
BASE = 1 << 44
SEP = 1 << 36


def _ptrs(n=8):
    return [BASE + i * SEP for i in range(n)]


def _chunk(L, **kw):
    q, k, v, g, beta, S0, o, S_T = _ptrs()
    a = dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0, o=o, S_T=S_T,
             B=2, T=100, H=3, K=128, V=128, chunk=64, dtype=1, gate=0)
    a.update(kw)
    return L.gdn_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["o"],
                           a["S_T"], a["B"], a["T"], a["H"], a["K"], a["V"], a["chunk"],
                           a["dtype"], a["gate"], None)


def _step(L, **kw):
    q, k, v, g, beta, S, o = _ptrs(7)
    a = dict(q=q, k=k, v=v, g=g, beta=beta, S=S, o=o, N=4, H=3, K=128, V=128,
             dtype=1, gate=1)
    a.update(kw)
    return L.gdn_recurrent_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S"], a["o"],
                                a["N"], a["H"], a["K"], a["V"], a["dtype"], a["gate"], None)


@pytest.mark.parametrize("kw", [
    dict(dtype=2), dict(dtype=-1), dict(gate=2), dict(B=-1), dict(T=-1), dict(H=-1),
    dict(K=0), dict(V=-5), dict(chunk=0), dict(q=None), dict(g=None), dict(beta=None),
    dict(o=None, S_T=None), dict(q=BASE + 8), dict(v=BASE + 2 * SEP + 4),
    dict(g=BASE + 3 * SEP + 4, gate=1), dict(g=BASE + 3 * SEP + 2),
    dict(beta=BASE + 4 * SEP + 2), dict(S_T=BASE + 7 * SEP + 2), dict(o=BASE + 6 * SEP + 1),
    dict(o=BASE),                       # o aliases q
    dict(o=BASE + 2 * SEP + 64),        # o overlaps v
    dict(S_T=BASE + 3 * SEP),           # S_T aliases g
    dict(S_T=BASE + 5 * SEP + 16),      # S_T partially overlaps S0
    dict(B=1 << 30, T=1 << 30, H=1 << 30),  # size overflow
])
def test_chunk_rejects_invalid(L, kw):
    assert _chunk(L, **kw) == gdn.GDN_EINVAL


@pytest.mark.parametrize("kw", [
    dict(K=96), dict(V=32), dict(K=256), dict(chunk=32), dict(chunk=128),
    dict(dtype=0, K=128),               # fp32 chunk path: K = 64 only
])
def test_chunk_unsupported(L, kw):
    assert _chunk(L, **kw) == gdn.GDN_ENOTSUP


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(T=0, S_T=None)])
def test_chunk_empty_is_a_noop(L, kw):
    assert _chunk(L, **kw) == gdn.GDN_OK


def test_chunk_empty_batch_needs_no_pointers(L):
    assert _chunk(L, B=0, q=None, k=None, v=None, g=None, beta=None) == gdn.GDN_OK


@pytest.mark.parametrize("kw", [
    dict(dtype=3), dict(gate=-1), dict(N=-1), dict(H=-2), dict(K=0), dict(S=None),
    dict(q=None), dict(o=BASE + 5 * SEP), dict(o=BASE), dict(S=BASE + 1 * SEP),
    dict(v=BASE + 2 * SEP + 1), dict(S=BASE + 5 * SEP + 8), dict(beta=BASE + 4 * SEP + 2),
    dict(q=BASE + 1), dict(g=BASE + 3 * SEP + 2),
])
def test_step_rejects_invalid(L, kw):
    assert _step(L, **kw) == gdn.GDN_EINVAL


@pytest.mark.parametrize("kw", [dict(K=32), dict(V=256), dict(K=100)])
def test_step_unsupported(L, kw):
    assert _step(L, **kw) == gdn.GDN_ENOTSUP


def test_step_empty_is_a_noop(L):
    assert _step(L, N=0) == gdn.GDN_OK


def _steps(L, **kw):
    q, k, v, g, beta, S0, o, S_T, S_hist = _ptrs(9)
    a = dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0, o=o, S_T=S_T, S_hist=S_hist,
             N=4, M=3, H=3, K=128, V=128, dtype=1, gate=1)
    a.update(kw)
    return L.gdn_recurrent_steps(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["o"],
                                 a["S_T"], a["S_hist"], a["N"], a["M"], a["H"], a["K"], a["V"],
                                 a["dtype"], a["gate"], None)


@pytest.mark.parametrize("kw", [
    dict(dtype=2), dict(gate=3), dict(N=-1), dict(M=-1), dict(H=-1), dict(K=0), dict(V=-1),
    dict(o=None, S_T=None, S_hist=None), dict(q=None), dict(v=None), dict(g=None),
    dict(beta=None), dict(q=BASE + 1), dict(o=BASE + 6 * SEP + 1), dict(g=BASE + 3 * SEP + 2),
    dict(S0=BASE + 5 * SEP + 8), dict(S_T=BASE + 7 * SEP + 4), dict(S_hist=BASE + 8 * SEP + 8),
    dict(o=BASE + 5 * SEP),             # o aliases S0
    dict(S_hist=BASE + 7 * SEP),        # S_hist aliases S_T
    dict(S_hist=BASE + 2 * SEP + 64),   # S_hist overlaps v
    dict(S_T=BASE),                     # S_T aliases q
    dict(S_T=BASE + 5 * SEP + 16),      # S_T partially overlaps S0
    dict(N=1 << 30, M=1 << 30, H=1 << 30),  # size overflow
])
def test_steps_rejects_invalid(L, kw):
    assert _steps(L, **kw) == gdn.GDN_EINVAL


@pytest.mark.parametrize("kw", [dict(K=32), dict(V=256), dict(K=96, dtype=0)])
def test_steps_unsupported(L, kw):
    assert _steps(L, **kw) == gdn.GDN_ENOTSUP


@pytest.mark.parametrize("kw", [dict(N=0), dict(H=0), dict(M=0, S_T=None),
                                dict(N=0, q=None, k=None, v=None, g=None, beta=None, S0=None)])
def test_steps_empty_is_a_noop(L, kw):
    assert _steps(L, **kw) == gdn.GDN_OK


def test_steps_in_place_state_passes_validation(L):
    # S_T == S0 is allowed; an unsupported K stops the call right after the checks
    assert _steps(L, S_T=BASE + 5 * SEP, K=32) == gdn.GDN_ENOTSUP


def _bwd(L, ws_bytes=None, **kw):
    p = _ptrs(16)
    a = dict(q=p[0], k=p[1], v=p[2], g=p[3], beta=p[4], S0=p[5], d_o=p[6], dS_T=p[7],
             dq=p[8], dk=p[9], dv=p[10], dg=p[11], dbeta=p[12], dS0=p[13], ws=p[14],
             B=2, T=100, H=3, K=128, V=128, chunk=64, dtype=1, gate=1)
    a.update(kw)
    if ws_bytes is None:
        ws_bytes = SEP   # large enough for these sizes
    return L.gdn_chunk_bwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["d_o"],
                           a["dS_T"], a["dq"], a["dk"], a["dv"], a["dg"], a["dbeta"], a["dS0"],
                           a["ws"], ws_bytes, a["B"], a["T"], a["H"], a["K"], a["V"],
                           a["chunk"], a["dtype"], a["gate"], None)


def _ws_size(L, B, T, H, K, V, chunk=64):
    import ctypes
    n = ctypes.c_size_t(12345)
    rc = L.gdn_chunk_bwd_workspace_size(B, T, H, K, V, chunk, ctypes.byref(n))
    return rc, n.value


@pytest.mark.parametrize("kw", [
    dict(dtype=2), dict(gate=2), dict(B=-1), dict(T=-1), dict(H=-1), dict(K=0), dict(V=-1),
    dict(chunk=0), dict(q=None), dict(d_o=None), dict(dq=None), dict(dg=None), dict(dbeta=None),
    dict(ws=None), dict(q=BASE + 1), dict(k=BASE + SEP + 8), dict(d_o=BASE + 6 * SEP + 2),
    dict(S0=BASE + 5 * SEP + 4), dict(dS_T=BASE + 7 * SEP + 8), dict(g=BASE + 3 * SEP + 4),
    dict(dv=BASE + 10 * SEP + 1), dict(g=BASE + 3 * SEP + 2),
    dict(dS0=BASE + 13 * SEP + 2), dict(ws=BASE + 14 * SEP + 64),
    dict(dq=BASE),                      # dq aliases q
    dict(dv=BASE + 6 * SEP + 64),       # dv overlaps d_o
    dict(dg=BASE + 12 * SEP),           # dg aliases dbeta
    dict(dS0=BASE + 5 * SEP),           # dS0 aliases S0
    dict(ws=BASE + 13 * SEP),           # workspace over dS0
    dict(dbeta=BASE + 14 * SEP + 256),  # an output inside the workspace
    dict(B=1 << 30, T=1 << 30, H=1 << 30),
])
def test_bwd_rejects_invalid(L, kw):
    assert _bwd(L, **kw) == gdn.GDN_EINVAL


def test_bwd_rejects_small_workspace(L):
    rc, need = _ws_size(L, 2, 100, 3, 128, 128)
    assert rc == gdn.GDN_OK and need > 0
    assert _bwd(L, ws_bytes=need - 1) == gdn.GDN_EINVAL


@pytest.mark.parametrize("kw", [dict(K=96), dict(V=32), dict(chunk=32), dict(K=256, dtype=0)])
def test_bwd_unsupported(L, kw):
    assert _bwd(L, **kw) == gdn.GDN_ENOTSUP


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(T=0, dS0=None),
                                dict(B=0, q=None, k=None, v=None, g=None, beta=None, d_o=None,
                                     dq=None, dk=None, dv=None, dg=None, dbeta=None, ws=None)])
def test_bwd_empty_is_a_noop(L, kw):
    assert _bwd(L, **kw) == gdn.GDN_OK


def test_bwd_workspace_size(L):
    import ctypes
    assert L.gdn_chunk_bwd_workspace_size(1, 64, 1, 128, 128, 64, None) == gdn.GDN_EINVAL
    assert _ws_size(L, 1, 64, 1, 96, 128)[0] == gdn.GDN_ENOTSUP
    assert _ws_size(L, 1, 64, 1, 128, 128, chunk=32)[0] == gdn.GDN_ENOTSUP
    assert _ws_size(L, -1, 64, 1, 128, 128)[0] == gdn.GDN_EINVAL
    assert _ws_size(L, 3, 0, 2, 128, 128) == (gdn.GDN_OK, 0)
    # twenty-four arrays over the chunks (the last three half-size), each
    # rounded up to 256 bytes
    for B, T, H, K, V in [(1, 1, 1, 64, 64), (2, 100, 3, 128, 64), (4, 4096, 6, 128, 128)]:
        nch = B * H * ((T + 63) // 64)
        per = [64 * K] + [64 * 64] * 4 + [K * V] * 2 + [64 * V] * 2 + [64 * K] * 3 + \
              [64 * 64] * 2 + [K] + [64 * K] * 5 + [K] + [32 * K, 32 * 64, 32 * 64]
        want = sum((nch * x * 4 + 255) // 256 * 256 for x in per)
        assert _ws_size(L, B, T, H, K, V) == (gdn.GDN_OK, want)
        assert gdn.gdn_chunk_bwd_workspace_size(B, T, H, K, V) == want
    assert ctypes.sizeof(ctypes.c_size_t) == 8


def _pro(L, **kw):
    p = _ptrs(20)
    a = dict(q_raw=p[0], k_raw=p[1], v_raw=p[2], g_raw=p[3], b_raw=p[4], w_q=p[5], w_k=p[6],
             w_v=p[7], cs_q=p[8], cs_k=p[9], cs_v=p[10], q=p[11], k=p[12], v=p[13], g=p[14],
             beta=p[15], cs_q_out=p[16], cs_k_out=p[17], cs_v_out=p[18],
             B=2, T=50, H=3, K=128, V=128, cap=5.0, act=1, dtype=1, gate=1)
    a.update(kw)
    return L.gdn_prologue(*[a[n] for n in ("q_raw", "k_raw", "v_raw", "g_raw", "b_raw", "w_q",
                                           "w_k", "w_v", "cs_q", "cs_k", "cs_v", "q", "k", "v",
                                           "g", "beta", "cs_q_out", "cs_k_out", "cs_v_out", "B",
                                           "T", "H", "K", "V", "cap", "act", "dtype", "gate")],
                          None)


@pytest.mark.parametrize("kw", [
    dict(dtype=2), dict(gate=2), dict(act=2), dict(B=-1), dict(T=-1), dict(K=0), dict(V=-1),
    dict(cap=0.0), dict(cap=-1.0), dict(cap=float("nan")), dict(q_raw=None), dict(w_v=None),
    dict(beta=None), dict(q=BASE + 11 * SEP + 8), dict(w_k=BASE + 6 * SEP + 4),
    dict(cs_v=BASE + 10 * SEP + 2), dict(g_raw=BASE + 3 * SEP + 4), dict(b_raw=BASE + 4 * SEP + 2),
    dict(q=BASE),                       # q over q_raw
    dict(v=BASE + 7 * SEP),             # v over the v taps
    dict(g=BASE + 15 * SEP),            # g over beta
    dict(cs_q_out=BASE + 8 * SEP + 16), # partial overlap with its own input
    dict(cs_k_out=BASE + 8 * SEP),      # over another state input
    dict(cs_v_out=BASE + 16 * SEP),     # two outputs on one buffer
])
def test_prologue_rejects_invalid(L, kw):
    assert _pro(L, **kw) == gdn.GDN_EINVAL


@pytest.mark.parametrize("kw", [dict(K=96), dict(V=32)])
def test_prologue_unsupported(L, kw):
    assert _pro(L, **kw) == gdn.GDN_ENOTSUP


def test_prologue_state_in_place_and_no_cap_pass_validation(L):
    assert _pro(L, cs_q_out=BASE + 8 * SEP, cs_k_out=BASE + 9 * SEP, cs_v_out=BASE + 10 * SEP,
                cap=float("inf"), K=96) == gdn.GDN_ENOTSUP


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(T=0, cs_q_out=None, cs_k_out=None,
                                                           cs_v_out=None)])
def test_prologue_empty_is_a_noop(L, kw):
    assert _pro(L, **kw) == gdn.GDN_OK


def _stp(L, **kw):
    p = _ptrs(20)
    a = dict(q_raw=p[0], k_raw=p[1], v_raw=p[2], g_raw=p[3], b_raw=p[4], w_q=p[5], w_k=p[6],
             w_v=p[7], cs_q=p[8], cs_k=p[9], cs_v=p[10], cs_q_out=p[11], cs_k_out=p[12],
             cs_v_out=p[13], S=p[14], o=p[15], N=4, H=3, K=128, V=128, cap=5.0, act=1, dtype=1,
             gate=1)
    a.update(kw)
    return L.gdn_recurrent_step_prologue(*[a[n] for n in (
        "q_raw", "k_raw", "v_raw", "g_raw", "b_raw", "w_q", "w_k", "w_v", "cs_q", "cs_k", "cs_v",
        "cs_q_out", "cs_k_out", "cs_v_out", "S", "o", "N", "H", "K", "V", "cap", "act", "dtype",
        "gate")], None)


@pytest.mark.parametrize("kw", [
    dict(dtype=2), dict(act=-1), dict(N=-1), dict(cap=0.0), dict(S=None), dict(w_q=None),
    dict(S=BASE + 14 * SEP + 8), dict(w_v=BASE + 7 * SEP + 4), dict(q_raw=BASE + 1),
    dict(cs_q_out=BASE + 8 * SEP),      # a state output on its input: not allowed here
    dict(o=BASE + 14 * SEP),            # o on S
    dict(cs_v_out=BASE + 2 * SEP),      # over v_raw
])
def test_step_prologue_rejects_invalid(L, kw):
    assert _stp(L, **kw) == gdn.GDN_EINVAL


def test_step_prologue_unsupported_and_empty(L):
    assert _stp(L, K=32) == gdn.GDN_ENOTSUP
    assert _stp(L, N=0) == gdn.GDN_OK


def test_element_aligned_vectors_are_accepted_by_validation(L):
    # per-step slices of [steps, N, H] beta / scalar g are 4-byte aligned only;
    # validation must pass them (the call then fails later only for lack of a GPU,
    # so this uses an unsupported K to stop right after the pointer checks)
    assert _step(L, beta=BASE + 4 * SEP + 4, g=BASE + 3 * SEP + 4, gate=0, K=32) == gdn.GDN_ENOTSUP
    assert _chunk(L, beta=BASE + 4 * SEP + 4, S0=BASE + 5 * SEP + 4, K=32) == gdn.GDN_ENOTSUP


def test_python_binding_rejects_cpu_tensors(L):
    import torch
    q = torch.zeros(1, 4, 1, 64)
    with pytest.raises(ValueError):
        gdn.gdn_chunk_fwd(q, q, q, torch.zeros(1, 4, 1), torch.zeros(1, 4, 1), None, q, None)


def test_status_error_carries_code(L):
    e = gdn.GDNError(2, "gdn_chunk_fwd")
    assert e.status == 2 and "unsupported" in str(e)


# ---------------------------------------------------------------- chunkwise forward with workspace
def _fws_size(L, B=1, T=262144, H=48, K=128, V=128, chunk=64, dtype=1, gate=1, want_o=0):
    import ctypes
    n = ctypes.c_size_t(12345)
    rc = L.gdn_chunk_fwd_workspace_size(B, T, H, K, V, chunk, dtype, gate, want_o, ctypes.byref(n))
    return rc, n.value


def test_fwd_workspace_size_values(L):
    # final state only, bf16, per-channel gate, 48 heads of 262144 tokens: 16 segments of
    # 256 chunks, an fp32 M (128 x 128) and N (128 x 128) and four int flags (which
    # column blocks of M are all zero) for each of the 15 after the first
    assert _fws_size(L) == (gdn.GDN_OK, 48 * 15 * (2 * 128 * 128 + 4) * 4)
    # two heads of 2048 tokens: four segments of 8 chunks
    assert _fws_size(L, B=1, H=2, T=2048) == (gdn.GDN_OK, 1 * 2 * 3 * (2 * 128 * 128 + 4) * 4)
    # 48 heads of 16 chunks: two segments of 8
    assert _fws_size(L, T=1000) == (gdn.GDN_OK, 48 * 1 * (2 * 128 * 128 + 4) * 4)
    # with o: the incoming state of each later segment as well
    assert _fws_size(L, want_o=1) == (gdn.GDN_OK, 48 * 15 * (3 * 128 * 128 + 4) * 4)
    # no sequence-parallel form: scalar gate, fp32, K = 64, enough heads, short T
    for kw in (dict(gate=0), dict(dtype=0, K=64, V=64), dict(K=64), dict(K=64, want_o=1),
               dict(B=16, H=8, T=2048), dict(T=500), dict(T=0), dict(B=0)):
        assert _fws_size(L, **kw) == (gdn.GDN_OK, 0), kw


def test_fwd_workspace_size_errors(L):
    import ctypes
    assert L.gdn_chunk_fwd_workspace_size(1, 64, 1, 128, 128, 64, 1, 1, 0, None) == gdn.GDN_EINVAL
    for kw in (dict(dtype=2), dict(gate=3), dict(B=-1), dict(T=-1), dict(K=0), dict(chunk=0)):
        assert _fws_size(L, **kw)[0] == gdn.GDN_EINVAL, kw
    for kw in (dict(K=96), dict(V=32), dict(chunk=32), dict(dtype=0, K=128), dict(H=70000)):
        assert _fws_size(L, **kw)[0] == gdn.GDN_ENOTSUP, kw


def _chunk_ws(L, **kw):
    q, k, v, g, beta, S0, o, S_T, ws = _ptrs(9)
    a = dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0, o=None, S_T=S_T, ws=ws, nbytes=1 << 30,
             B=1, T=262144, H=48, K=128, V=128, chunk=64, dtype=1, gate=1)
    a.update(kw)
    return L.gdn_chunk_fwd_ws(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["o"],
                              a["S_T"], a["ws"], a["nbytes"], a["B"], a["T"], a["H"], a["K"],
                              a["V"], a["chunk"], a["dtype"], a["gate"], None)


@pytest.mark.parametrize("kw", [
    dict(ws=None),                        # the segment form needs its workspace
    dict(nbytes=48 * 15 * 2 * 128 * 128 * 4 - 1),
    dict(ws=BASE + 8 * SEP + 128),        # misaligned
    dict(ws=BASE + 1 * SEP),              # over k
    dict(ws=BASE + 7 * SEP - 4096),       # runs into S_T
    dict(dtype=5), dict(S_T=None),        # o and S_T both absent
    dict(q=BASE + 4),
])
def test_fwd_ws_rejects_invalid(L, kw):
    assert _chunk_ws(L, **kw) == gdn.GDN_EINVAL


def test_fwd_ws_unsupported(L):
    assert _chunk_ws(L, K=96) == gdn.GDN_ENOTSUP
    assert _chunk_ws(L, T=64, H=70000) == gdn.GDN_ENOTSUP


def test_fwd_ws_empty_is_a_noop(L):
    assert _chunk_ws(L, B=0) == gdn.GDN_OK
    assert _chunk_ws(L, H=0, ws=None) == gdn.GDN_OK


def test_chunk_paths_reject_shapes_past_32bit_offsets(L):
    # 64 rows of H * 128 fp32 values past 2^31 bytes: the kernels' per-lane
    # offsets would overflow, so the host refuses the shape
    assert _chunk(L, B=1, T=64, H=65536) == gdn.GDN_ENOTSUP
    import ctypes
    n = ctypes.c_size_t(0)
    assert L.gdn_chunk_bwd_workspace_size(1, 64, 65536, 128, 128, 64, ctypes.byref(n)) == gdn.GDN_ENOTSUP
    assert L.gdn_chunk_bwd_workspace_size(1, 64, 65535, 128, 128, 64, ctypes.byref(n)) == gdn.GDN_OK


def test_chunk_bwd_rejects_grids_past_2_23_chunks(L):
    # one 512-thread workgroup per 64-token chunk: 2^23 chunks would make the
    # grid 2^32 threads
    import ctypes
    n = ctypes.c_size_t(0)
    assert L.gdn_chunk_bwd_workspace_size(1, 64 * (1 << 23), 1, 128, 128, 64, ctypes.byref(n)) == gdn.GDN_ENOTSUP
    assert L.gdn_chunk_bwd_workspace_size(1, 64 * ((1 << 23) - 1), 1, 128, 128, 64, ctypes.byref(n)) == gdn.GDN_OK


def test_prologue_channel_cap_above_five_is_unsupported(L):
    # the per-channel chunk kernels need g >= -5: a larger cap (or none) for the
    # per-channel gate is refused; the scalar gate takes any cap
    assert _pro(L, gate=1, cap=5.5) == gdn.GDN_ENOTSUP
    assert _pro(L, gate=1, cap=float("inf")) == gdn.GDN_ENOTSUP
    assert _pro(L, gate=0, cap=float("inf"), K=96) == gdn.GDN_ENOTSUP   # stops at K, not the cap


# --- decoupled erase/write gates ----------------------------------------------------
def _chunk_dg(L, **kw):
    q, k, v, g, e, w, S0, o, S_T = _ptrs(9)
    a = dict(q=q, k=k, v=v, g=g, e=e, w=w, S0=S0, o=o, S_T=S_T,
             B=2, T=100, H=3, K=128, V=128, chunk=64, dtype=1, gate=1)
    a.update(kw)
    return L.gdn_chunk_fwd_decoupled(a["q"], a["k"], a["v"], a["g"], a["e"], a["w"], a["S0"],
                                     a["o"], a["S_T"], a["B"], a["T"], a["H"], a["K"], a["V"],
                                     a["chunk"], a["dtype"], a["gate"], None)


def _step_dg(L, **kw):
    q, k, v, g, e, w, S, o = _ptrs(8)
    a = dict(q=q, k=k, v=v, g=g, e=e, w=w, S=S, o=o, N=4, H=3, K=128, V=128, dtype=1, gate=1)
    a.update(kw)
    return L.gdn_recurrent_step_decoupled(a["q"], a["k"], a["v"], a["g"], a["e"], a["w"],
                                          a["S"], a["o"], a["N"], a["H"], a["K"], a["V"],
                                          a["dtype"], a["gate"], None)


@pytest.mark.parametrize("kw", [
    dict(e=None), dict(w=None), dict(w=BASE + 5 * SEP + 2), dict(e=BASE + 4 * SEP + 2),
    dict(o=BASE + 5 * SEP),             # o aliases the write gate
    dict(S_T=BASE + 5 * SEP + 64),      # S_T overlaps the write gate
    dict(dtype=2), dict(gate=3), dict(T=-1), dict(o=None, S_T=None),
])
def test_chunk_decoupled_rejects_invalid(L, kw):
    assert _chunk_dg(L, **kw) == gdn.GDN_EINVAL


@pytest.mark.parametrize("kw", [dict(K=96), dict(chunk=32), dict(dtype=0, K=128)])
def test_chunk_decoupled_unsupported(L, kw):
    assert _chunk_dg(L, **kw) == gdn.GDN_ENOTSUP


def test_chunk_decoupled_empty_is_a_noop(L):
    assert _chunk_dg(L, B=0, q=None, k=None, v=None, g=None, e=None, w=None) == gdn.GDN_OK
    assert _chunk_dg(L, T=0, S_T=None) == gdn.GDN_OK


@pytest.mark.parametrize("kw", [
    dict(e=None), dict(w=None), dict(w=BASE + 5 * SEP + 1), dict(o=BASE + 5 * SEP),
    dict(S=BASE + 5 * SEP),             # S aliases the write gate
    dict(dtype=3), dict(N=-1),
])
def test_step_decoupled_rejects_invalid(L, kw):
    assert _step_dg(L, **kw) == gdn.GDN_EINVAL


def test_step_decoupled_unsupported_and_empty(L):
    assert _step_dg(L, K=32) == gdn.GDN_ENOTSUP
    assert _step_dg(L, N=0) == gdn.GDN_OK
    assert _step_dg(L, N=0, w=None, e=None) == gdn.GDN_OK


# --- the prologue fused into the chunkwise forward ----------------------------------------
def _cpro(L, **kw):
    names = ["q", "k", "v", "g", "b", "wq", "wk", "wv", "csq", "csk", "csv", "oq", "ok", "ov",
             "S0", "o", "S_T"]
    a = dict(zip(names, _ptrs(len(names))))
    a.update(B=2, T=100, H=3, K=128, V=128, chunk=64, cap=5.0, act=1, dtype=1, gate=1)
    a.update(kw)
    return L.gdn_chunk_fwd_prologue(*(a[n] for n in names), a["B"], a["T"], a["H"], a["K"],
                                    a["V"], a["chunk"], a["cap"], a["act"], a["dtype"], a["gate"],
                                    None)


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(wq=None), dict(b=None), dict(act=2), dict(cap=0.0), dict(cap=-1.0),
    dict(cap=float("nan")), dict(dtype=2), dict(gate=3), dict(T=-1), dict(o=None, S_T=None),
    dict(oq=BASE + 8 * SEP),            # a carried state out that is its own input
    dict(ov=BASE + 10 * SEP + 16),      # overlaps the incoming v state
    dict(o=BASE + 5 * SEP),             # o overlaps the q taps
    dict(S_T=BASE + 9 * SEP),           # S_T overlaps an incoming state
    dict(ok=BASE + 15 * SEP),           # a carried state out overlaps o
    dict(wk=BASE + 6 * SEP + 4), dict(csv=BASE + 10 * SEP + 8),
])
def test_chunk_prologue_rejects_invalid(L, kw):
    assert _cpro(L, **kw) == gdn.GDN_EINVAL


@pytest.mark.parametrize("kw", [dict(cap=5.5), dict(cap=float("inf")), dict(K=96), dict(chunk=32),
                                dict(dtype=0, K=128)])
def test_chunk_prologue_unsupported(L, kw):
    assert _cpro(L, **kw) == gdn.GDN_ENOTSUP


def test_chunk_prologue_valid_edges(L):
    # an uncapped scalar gate passes validation (then enqueues work: not called here)
    assert _cpro(L, B=0, gate=0, cap=float("inf")) == gdn.GDN_OK
    assert _cpro(L, B=0, q=None, k=None, v=None, g=None, b=None, wq=None, wk=None, wv=None) == gdn.GDN_OK
    assert _cpro(L, T=0, S_T=None, oq=None, ok=None, ov=None) == gdn.GDN_OK
