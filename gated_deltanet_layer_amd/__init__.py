"""Gated DeltaNet mixer on MI355X (gfx950): Python binding of libgdn.so.

The work runs in the HIP kernels behind the C ABI declared in ``include/gdn.h``;
this module only checks tensors, marshals pointers and sizes, and passes the
current torch stream.  PyTorch provides device memory and streams.  There is no
fallback: if ``libgdn.so`` has not been built, every call raises.

Entry points (same names as the C ABI):
    gdn_chunk_fwd(q, k, v, g, beta, S0, o, S_T, chunk=64)
    gdn_chunk_fwd_ws(q, k, v, g, beta, S0, o, S_T, workspace, chunk=64)
    gdn_chunk_fwd_workspace_size(B, T, H, K, V, dtype, gate, want_o) -> bytes
    gdn_chunk_fwd_noalloc(q, k, v, g, beta, S0, o, S_T, chunk=64)
    gdn_recurrent_step(q, k, v, g, beta, S, o)
    gdn_recurrent_steps(q, k, v, g, beta, S0, o, S_T, S_hist)
    gdn_chunk_fwd_decoupled(q, k, v, g, erase, write, S0, o, S_T, chunk=64)
    gdn_recurrent_step_decoupled(q, k, v, g, erase, write, S, o)
    gdn_chunk_bwd(q, k, v, g, beta, S0, d_o, dS_T, dq, dk, dv, dg, dbeta, dS0, workspace)
    gdn_chunk_bwd_workspace_size(B, T, H, K, V, chunk=64) -> bytes
    gdn_prologue(q_raw, k_raw, v_raw, g_raw, b_raw, w_q, w_k, w_v, cs_q, cs_k, cs_v,
                 q, k, v, g, beta, cs_q_out, cs_k_out, cs_v_out, g_cap=5.0, act="silu")
    gdn_recurrent_step_prologue(q_raw, k_raw, v_raw, g_raw, b_raw, w_q, w_k, w_v,
                 cs_q, cs_k, cs_v, cs_q_out, cs_k_out, cs_v_out, S, o, g_cap=5.0, act="silu")
    gdn_chunk_fwd_prologue(q_raw, k_raw, v_raw, g_raw, b_raw, w_q, w_k, w_v, cs_q, cs_k, cs_v,
                 cs_q_out, cs_k_out, cs_v_out, S0, o, S_T, chunk=64, g_cap=5.0, act="silu")
Conveniences that allocate the outputs:
    chunk_fwd(q, k, v, g, beta, S0=None, want_o=True) -> (o, S_T)
    recurrent_step_(q, k, v, g, beta, S) -> o      (S updated in place)
    chunk_fwd_decoupled(q, k, v, g, erase, write, S0=None, want_o=True) -> (o, S_T)
    recurrent_step_decoupled_(q, k, v, g, erase, write, S) -> o
    chunk_bwd(q, k, v, g, beta, S0, d_o, dS_T) -> dict of dq, dk, dv, dg, dbeta, dS0
    prologue(q_raw, k_raw, v_raw, g_raw, b_raw, w_q, w_k, w_v, state=None) -> dict
    chunk_fwd_prologue(q_raw, k_raw, v_raw, g_raw, b_raw, w_q, w_k, w_v, state=None, S0=None)
        -> (o, S_T, state)
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_OK, GDN_EINVAL, GDN_ENOTSUP, GDN_EHIP = 0, 1, 2, 3
GDN_F32, GDN_BF16 = 0, 1
GDN_GATE_HEAD, GDN_GATE_CHANNEL = 0, 1
GDN_ACT_NONE, GDN_ACT_SILU = 0, 1
_ACTS = {"none": GDN_ACT_NONE, "silu": GDN_ACT_SILU}
SYMBOLS = ("gdn_chunk_fwd", "gdn_chunk_fwd_workspace_size", "gdn_chunk_fwd_ws",
           "gdn_chunk_fwd_noalloc", "gdn_recurrent_step", "gdn_recurrent_steps",
           "gdn_chunk_bwd_workspace_size", "gdn_chunk_bwd", "gdn_prologue",
           "gdn_recurrent_step_prologue", "gdn_chunk_fwd_decoupled",
           "gdn_recurrent_step_decoupled", "gdn_chunk_fwd_prologue", "gdn_status_str",
           "gdn_abi_version")

_lock = threading.Lock()
_lib = None


class GDNError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded libgdn.so, with argument types set.  Raises if it is not built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m gated_deltanet_layer_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        vp, fp, i = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int
        L.gdn_chunk_fwd.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp,
                                    i, i, i, i, i, i, i, i, vp]
        L.gdn_chunk_fwd.restype = i
        L.gdn_recurrent_step.argtypes = [vp, vp, vp, fp, fp, fp, vp,
                                         i, i, i, i, i, i, vp]
        L.gdn_recurrent_step.restype = i
        L.gdn_recurrent_steps.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, fp,
                                          i, i, i, i, i, i, i, vp]
        L.gdn_recurrent_steps.restype = i
        sz = ctypes.c_size_t
        L.gdn_chunk_fwd_workspace_size.argtypes = [i, i, i, i, i, i, i, i, i, ctypes.POINTER(sz)]
        L.gdn_chunk_fwd_workspace_size.restype = i
        L.gdn_chunk_fwd_ws.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, vp, sz,
                                       i, i, i, i, i, i, i, i, vp]
        L.gdn_chunk_fwd_ws.restype = i
        L.gdn_chunk_fwd_noalloc.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp,
                                            i, i, i, i, i, i, i, i, vp]
        L.gdn_chunk_fwd_noalloc.restype = i
        L.gdn_chunk_bwd_workspace_size.argtypes = [i, i, i, i, i, i, ctypes.POINTER(sz)]
        L.gdn_chunk_bwd_workspace_size.restype = i
        L.gdn_chunk_bwd.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, vp, vp, vp, fp, fp, fp,
                                    vp, sz, i, i, i, i, i, i, i, i, vp]
        L.gdn_chunk_bwd.restype = i
        f = ctypes.c_float
        L.gdn_prologue.argtypes = [vp, vp, vp, fp, fp, fp, fp, fp, vp, vp, vp, vp, vp, vp, fp, fp,
                                   vp, vp, vp, i, i, i, i, i, f, i, i, i, vp]
        L.gdn_prologue.restype = i
        L.gdn_recurrent_step_prologue.argtypes = [vp, vp, vp, fp, fp, fp, fp, fp, vp, vp, vp,
                                                  vp, vp, vp, fp, vp, i, i, i, i, f, i, i, i, vp]
        L.gdn_recurrent_step_prologue.restype = i
        L.gdn_chunk_fwd_decoupled.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp, fp,
                                              i, i, i, i, i, i, i, i, vp]
        L.gdn_chunk_fwd_decoupled.restype = i
        L.gdn_recurrent_step_decoupled.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp,
                                                   i, i, i, i, i, i, vp]
        L.gdn_recurrent_step_decoupled.restype = i
        L.gdn_chunk_fwd_prologue.argtypes = [vp, vp, vp, fp, fp, fp, fp, fp, vp, vp, vp, vp, vp,
                                             vp, fp, vp, fp, i, i, i, i, i, i, f, i, i, i, vp]
        L.gdn_chunk_fwd_prologue.restype = i
        L.gdn_status_str.argtypes = [i]
        L.gdn_status_str.restype = ctypes.c_char_p
        L.gdn_abi_version.argtypes = []
        L.gdn_abi_version.restype = i
        _lib = L
        return L


def status_str(s: int) -> str:
    return lib().gdn_status_str(int(s)).decode()


def abi_version() -> int:
    return int(lib().gdn_abi_version())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError(f"q/k/v/o must be float32 or bfloat16, got {t.dtype}")


def _check(t, name, shape=None, dtype=None, device=None):
    if t is None:
        return
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _chunk_fwd_args(q, k, v, g, beta, S0, o, S_T):
    """Check the tensors of a chunkwise forward; returns (B, T, H, K, V, gate)."""
    import torch
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, T, H, D]")
    B, T, H, K = q.shape
    V = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    dt = q.dtype
    _check(q, "q", dtype=dt)
    _check(k, "k", (B, T, H, K), dt, dev)
    _check(v, "v", (B, T, H, V), dt, dev)
    if g.dim() == 4:
        gate = GDN_GATE_CHANNEL
        _check(g, "g", (B, T, H, K), torch.float32, dev)
    else:
        gate = GDN_GATE_HEAD
        _check(g, "g", (B, T, H), torch.float32, dev)
    _check(beta, "beta", (B, T, H), torch.float32, dev)
    _check(S0, "S0", (B, H, K, V), torch.float32, dev)
    _check(o, "o", (B, T, H, V), dt, dev)
    _check(S_T, "S_T", (B, H, K, V), torch.float32, dev)
    return B, T, H, K, V, gate


def gdn_chunk_fwd(q, k, v, g, beta, S0, o, S_T, chunk: int = 64, stream=None) -> None:
    """Chunkwise forward; writes o [B,T,H,V] and/or S_T [B,H,K,V] (either may be None).

    q, k [B,T,H,K] and v [B,T,H,V] share a dtype (fp32 or bf16); g is [B,T,H] (scalar
    gate) or [B,T,H,K] (per key channel), fp32; beta [B,T,H] fp32; S0 [B,H,K,V] fp32
    or None.  S_T may be S0 (in place).  Enqueued on the current torch stream.
    """
    B, T, H, K, V, gate = _chunk_fwd_args(q, k, v, g, beta, S0, o, S_T)
    rc = lib().gdn_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0),
                             _ptr(o), _ptr(S_T), B, T, H, K, V, int(chunk),
                             _dtype_code(q), gate, _stream(stream))
    if rc != GDN_OK:
        raise GDNError(rc, "gdn_chunk_fwd")


def gdn_chunk_fwd_workspace_size(B: int, T: int, H: int, K: int, V: int, dtype, gate: int,
                                 want_o: bool, chunk: int = 64) -> int:
    """Bytes of workspace gdn_chunk_fwd_ws needs (0: none).  dtype is a torch dtype
    or GDN_F32 / GDN_BF16; gate GDN_GATE_HEAD or GDN_GATE_CHANNEL."""
    if not isinstance(dtype, int):
        import torch
        dtype = GDN_BF16 if dtype == torch.bfloat16 else GDN_F32
    n = ctypes.c_size_t(0)
    rc = lib().gdn_chunk_fwd_workspace_size(int(B), int(T), int(H), int(K), int(V), int(chunk),
                                            int(dtype), int(gate), int(bool(want_o)),
                                            ctypes.byref(n))
    if rc != GDN_OK:
        raise GDNError(rc, "gdn_chunk_fwd_workspace_size")
    return int(n.value)


def gdn_chunk_fwd_ws(q, k, v, g, beta, S0, o, S_T, workspace, chunk: int = 64,
                     stream=None) -> None:
    """gdn_chunk_fwd with a workspace (a uint8 device tensor, or None when
    gdn_chunk_fwd_workspace_size is 0): a call may then run the
    sequence-parallel form (with o as well, unless S_T is S0)."""
    B, T, H, K, V, gate = _chunk_fwd_args(q, k, v, g, beta, S0, o, S_T)
    if workspace is not None:
        _check(workspace, "workspace", device=q.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().gdn_chunk_fwd_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0),
                                _ptr(o), _ptr(S_T), _ptr(workspace), nbytes, B, T, H, K, V,
                                int(chunk), _dtype_code(q), gate, _stream(stream))
    if rc != GDN_OK:
        raise GDNError(rc, "gdn_chunk_fwd_ws")


def gdn_recurrent_step(q, k, v, g, beta, S, o, stream=None) -> None:
    """One decode step for N sequences: S [N,H,K,V] fp32 updated in place, o [N,H,V].

    q, k [N,H,K], v [N,H,V] (fp32 or bf16), g [N,H] or [N,H,K] fp32, beta [N,H] fp32.
    """
    N, H, K, V, gate = _step_args(q, k, v, g, beta, S, o)
    rc = lib().gdn_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S),
                                  _ptr(o), N, H, K, V, _dtype_code(q), gate, _stream(stream))
    if rc != GDN_OK:
        raise GDNError(rc, "gdn_recurrent_step")


def gdn_recurrent_step_decoupled(q, k, v, g, erase, write, S, o, stream=None) -> None:
    """gdn_recurrent_step with separate erase and write gates (erase, write [N,H]
    fp32): S' = (I - e k k^T) Diag(alpha) S + w k v^T."""
    import torch
    N, H, K, V, gate = _step_args(q, k, v, g, erase, S, o)
    _check(write, "write", (N, H), torch.float32, q.device)
    rc = lib().gdn_recurrent_step_decoupled(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(erase),
                                            _ptr(write), _ptr(S), _ptr(o), N, H, K, V,
                                            _dtype_code(q), gate, _stream(stream))
    if rc != GDN_OK:
        raise GDNError(rc, "gdn_recurrent_step_decoupled")


def gdn_chunk_fwd_decoupled(q, k, v, g, erase, write, S0, o, S_T, chunk: int = 64,
                            stream=None) -> None:
    """gdn_chunk_fwd with separate erase and write gates (erase, write [B,T,H] fp32):
    S_t = (I - e_t k_t k_t^T) Diag(alpha_t) S_{t-1} + w_t k_t v_t^T."""
    import torch
    B, T, H, K, V, gate = _chunk_fwd_args(q, k, v, g, erase, S0, o, S_T)
    _check(write, "write", (B, T, H), torch.float32, q.device)
    rc = lib().gdn_chunk_fwd_decoupled(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(erase),
                                       _ptr(write), _ptr(S0), _ptr(o), _ptr(S_T), B, T, H, K,
                                       V, int(chunk), _dtype_code(q), gate, _stream(stream))
    if rc != GDN_OK:
        raise GDNError(rc, "gdn_chunk_fwd_decoupled")


def _step_args(q, k, v, g, beta, S, o):
    """Check the tensors of a decode step; returns (N, H, K, V, gate)."""
    import torch
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [N, H, D]")
    N, H, K = q.shape
    V = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    dt = q.dtype
    _check(q, "q", dtype=dt)
    _check(k, "k", (N, H, K), dt, dev)
    _check(v, "v", (N, H, V), dt, dev)
    if g.dim() == 3:
        gate = GDN_GATE_CHANNEL
        _check(g, "g", (N, H, K), torch.float32, dev)
    else:
        gate = GDN_GATE_HEAD
        _check(g, "g", (N, H), torch.float32, dev)
    _check(beta, "beta", (N, H), torch.float32, dev)
    _check(S, "S", (N, H, K, V), torch.float32, dev)
    _check(o, "o", (N, H, V), dt, dev)
    return N, H, K, V, gate


def gdn_recurrent_steps(q, k, v, g, beta, S0, o, S_T, S_hist=None, stream=None) -> None:
    """M tokens per sequence from one state (speculative-decoding verification).

    q, k [N,M,H,K], v [N,M,H,V] (fp32 or bf16); g [N,M,H] or [N,M,H,K] fp32; beta
    [N,M,H] fp32; S0 [N,H,K,V] fp32 or None (zeros).  Writes o [N,M,H,V], S_T
    [N,H,K,V] (may be S0) and S_hist [N,M,H,K,V] (state after each token); any of
    them may be None, not all.  Enqueued on the current torch stream.
    """
    import torch
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [N, M, H, D]")
    N, M, H, K = q.shape
    V = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    dt = q.dtype
    _check(q, "q", dtype=dt)
    _check(k, "k", (N, M, H, K), dt, dev)
    _check(v, "v", (N, M, H, V), dt, dev)
    if g.dim() == 4:
        gate = GDN_GATE_CHANNEL
        _check(g, "g", (N, M, H, K), torch.float32, dev)
    else:
        gate = GDN_GATE_HEAD
        _check(g, "g", (N, M, H), torch.float32, dev)
    _check(beta, "beta", (N, M, H), torch.float32, dev)
    _check(S0, "S0", (N, H, K, V), torch.float32, dev)
    _check(o, "o", (N, M, H, V), dt, dev)
    _check(S_T, "S_T", (N, H, K, V), torch.float32, dev)
    _check(S_hist, "S_hist", (N, M, H, K, V), torch.float32, dev)
    rc = lib().gdn_recurrent_steps(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0),
                                   _ptr(o), _ptr(S_T), _ptr(S_hist), N, M, H, K, V,
                                   _dtype_code(q), gate, _stream(stream))
    if rc != GDN_OK:
        raise GDNError(rc, "gdn_recurrent_steps")


def gdn_chunk_bwd_workspace_size(B: int, T: int, H: int, K: int, V: int, chunk: int = 64) -> int:
    """Bytes of device workspace gdn_chunk_bwd needs for these sizes."""
    n = ctypes.c_size_t(0)
    rc = lib().gdn_chunk_bwd_workspace_size(B, T, H, K, V, int(chunk), ctypes.byref(n))
    if rc != GDN_OK:
        raise GDNError(rc, "gdn_chunk_bwd_workspace_size")
    return int(n.value)


def gdn_chunk_bwd(q, k, v, g, beta, S0, d_o, dS_T, dq, dk, dv, dg, dbeta, dS0, workspace,
                  chunk: int = 64, stream=None) -> None:
    """Chunkwise backward: gradients of a loss through gdn_chunk_fwd's operation.

    Inputs as for gdn_chunk_fwd plus d_o [B,T,H,V] (q's dtype) and dS_T [B,H,K,V] fp32
    (or None).  Writes dq, dk [B,T,H,K] and dv [B,T,H,V] (q's dtype), dg (g's shape)
    and dbeta [B,T,H] fp32, and dS0 [B,H,K,V] fp32 (or None).  ``workspace`` is a
    device tensor of at least gdn_chunk_bwd_workspace_size(...) bytes.
    """
    import torch
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, T, H, D]")
    B, T, H, K = q.shape
    V = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    dt = q.dtype
    _check(q, "q", dtype=dt)
    for t, name in ((k, "k"), (dq, "dq"), (dk, "dk")):
        _check(t, name, (B, T, H, K), dt, dev)
    for t, name in ((v, "v"), (d_o, "d_o"), (dv, "dv")):
        _check(t, name, (B, T, H, V), dt, dev)
    gshape = (B, T, H, K) if g.dim() == 4 else (B, T, H)
    gate = GDN_GATE_CHANNEL if g.dim() == 4 else GDN_GATE_HEAD
    _check(g, "g", gshape, torch.float32, dev)
    _check(dg, "dg", gshape, torch.float32, dev)
    _check(beta, "beta", (B, T, H), torch.float32, dev)
    _check(dbeta, "dbeta", (B, T, H), torch.float32, dev)
    for t, name in ((S0, "S0"), (dS_T, "dS_T"), (dS0, "dS0")):
        _check(t, name, (B, H, K, V), torch.float32, dev)
    _check(workspace, "workspace", device=dev)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().gdn_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0),
                             _ptr(d_o), _ptr(dS_T), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
                             _ptr(dbeta), _ptr(dS0), _ptr(workspace), nbytes,
                             B, T, H, K, V, int(chunk), _dtype_code(q), gate, _stream(stream))
    if rc != GDN_OK:
        raise GDNError(rc, "gdn_chunk_bwd")


def chunk_bwd(q, k, v, g, beta, S0, d_o, dS_T, want_dS0: bool = True, workspace=None,
              chunk: int = 64, stream=None):
    """Allocate the gradients (and the workspace unless one is given), run
    gdn_chunk_bwd, return a dict with dq, dk, dv, dg, dbeta, dS0."""
    import torch
    B, T, H, K = q.shape
    V = v.shape[-1]
    dev = q.device
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
               dg=torch.empty_like(g), dbeta=torch.empty_like(beta),
               dS0=torch.empty((B, H, K, V), dtype=torch.float32, device=dev) if want_dS0 else None)
    if workspace is None:
        n = gdn_chunk_bwd_workspace_size(B, T, H, K, V, chunk)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    gdn_chunk_bwd(q, k, v, g, beta, S0, d_o, dS_T, out["dq"], out["dk"], out["dv"], out["dg"],
                  out["dbeta"], out["dS0"], workspace, chunk=chunk, stream=stream)
    return out


def gdn_chunk_fwd_noalloc(q, k, v, g, beta, S0, o, S_T, chunk: int = 64, stream=None) -> None:
    """gdn_chunk_fwd_ws with the segment maps in the library's static device
    buffer (no allocation in the call; calls sharing a GPU must not overlap)."""
    B, T, H, K, V, gate = _chunk_fwd_args(q, k, v, g, beta, S0, o, S_T)
    rc = lib().gdn_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0),
                                     _ptr(o), _ptr(S_T), B, T, H, K, V, int(chunk),
                                     _dtype_code(q), gate, _stream(stream))
    if rc != GDN_OK:
        raise GDNError(rc, "gdn_chunk_fwd_noalloc")


def chunk_fwd(q, k, v, g, beta, S0=None, want_o: bool = True, chunk: int = 64, stream=None,
              workspace=None):
    """Allocate o (if wanted), S_T and, when the call can use one, a workspace;
    run gdn_chunk_fwd_ws; return (o, S_T).  workspace=False forces gdn_chunk_fwd
    (no workspace, the sequential kernels)."""
    import torch
    B, T, H, K = q.shape
    V = v.shape[-1]
    o = torch.empty((B, T, H, V), dtype=q.dtype, device=q.device) if want_o else None
    S_T = torch.empty((B, H, K, V), dtype=torch.float32, device=q.device)
    if workspace is False:
        gdn_chunk_fwd(q, k, v, g, beta, S0, o, S_T, chunk=chunk, stream=stream)
        return o, S_T
    if workspace is None:
        gate = GDN_GATE_CHANNEL if g.dim() == 4 else GDN_GATE_HEAD
        n = gdn_chunk_fwd_workspace_size(B, T, H, K, V, q.dtype, gate, want_o, chunk)
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device) if n > 0 else None
    gdn_chunk_fwd_ws(q, k, v, g, beta, S0, o, S_T, workspace, chunk=chunk, stream=stream)
    return o, S_T


def chunk_fwd_decoupled(q, k, v, g, erase, write, S0=None, want_o: bool = True,
                        chunk: int = 64, stream=None):
    """Allocate o (if wanted) and S_T, run gdn_chunk_fwd_decoupled, return (o, S_T)."""
    import torch
    B, T, H, K = q.shape
    V = v.shape[-1]
    o = torch.empty((B, T, H, V), dtype=q.dtype, device=q.device) if want_o else None
    S_T = torch.empty((B, H, K, V), dtype=torch.float32, device=q.device)
    gdn_chunk_fwd_decoupled(q, k, v, g, erase, write, S0, o, S_T, chunk=chunk, stream=stream)
    return o, S_T


def recurrent_step_decoupled_(q, k, v, g, erase, write, S, o=None, stream=None):
    """One decode step with separate erase and write gates; S is updated in
    place.  Returns o [N,H,V]."""
    import torch
    if o is None:
        o = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    gdn_recurrent_step_decoupled(q, k, v, g, erase, write, S, o, stream=stream)
    return o


def recurrent_step_(q, k, v, g, beta, S, o=None, stream=None):
    """One decode step; S is updated in place.  Returns o [N,H,V]."""
    import torch
    if o is None:
        o = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    gdn_recurrent_step(q, k, v, g, beta, S, o, stream=stream)
    return o


def gdn_prologue(q_raw, k_raw, v_raw, g_raw, b_raw, w_q, w_k, w_v, cs_q, cs_k, cs_v, q, k, v, g,
                 beta, cs_q_out, cs_k_out, cs_v_out, g_cap: float = 5.0, act: str = "silu",
                 stream=None) -> None:
    """The prologue of a chunk-mode call (convolution, activation, q/k norm, gates).

    Raw q_raw, k_raw [B,T,H,K] and v_raw [B,T,H,V] (fp32 or bf16), g_raw [B,T,H(,K)] and
    b_raw [B,T,H] fp32, taps w_q, w_k [H*K,4] and w_v [H*V,4] fp32, carried states
    cs_* [B,3,H*D] (raw dtype) or None.  Writes q, k, v, g, beta and, if given, the
    states after the sequence (each may be its own input).
    """
    import torch
    if q_raw.dim() != 4 or v_raw.dim() != 4:
        raise ValueError("q_raw, k_raw, v_raw must be [B, T, H, D]")
    B, T, H, K = q_raw.shape
    V = v_raw.shape[-1]
    dev = q_raw.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    dt = q_raw.dtype
    for t, name in ((q_raw, "q_raw"), (k_raw, "k_raw"), (q, "q"), (k, "k")):
        _check(t, name, (B, T, H, K), dt, dev)
    for t, name in ((v_raw, "v_raw"), (v, "v")):
        _check(t, name, (B, T, H, V), dt, dev)
    gshape = (B, T, H, K) if g_raw.dim() == 4 else (B, T, H)
    gate = GDN_GATE_CHANNEL if g_raw.dim() == 4 else GDN_GATE_HEAD
    for t, name in ((g_raw, "g_raw"), (g, "g")):
        _check(t, name, gshape, torch.float32, dev)
    for t, name in ((b_raw, "b_raw"), (beta, "beta")):
        _check(t, name, (B, T, H), torch.float32, dev)
    for t, name, D in ((w_q, "w_q", H * K), (w_k, "w_k", H * K), (w_v, "w_v", H * V)):
        _check(t, name, (D, 4), torch.float32, dev)
    for t, name, D in ((cs_q, "cs_q", H * K), (cs_k, "cs_k", H * K), (cs_v, "cs_v", H * V),
                       (cs_q_out, "cs_q_out", H * K), (cs_k_out, "cs_k_out", H * K),
                       (cs_v_out, "cs_v_out", H * V)):
        _check(t, name, (B, 3, D), dt, dev)
    rc = lib().gdn_prologue(_ptr(q_raw), _ptr(k_raw), _ptr(v_raw), _ptr(g_raw), _ptr(b_raw),
                            _ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(cs_q), _ptr(cs_k), _ptr(cs_v),
                            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cs_q_out),
                            _ptr(cs_k_out), _ptr(cs_v_out), B, T, H, K, V, float(g_cap),
                            _ACTS[act], _dtype_code(q_raw), gate, _stream(stream))
    if rc != GDN_OK:
        raise GDNError(rc, "gdn_prologue")


def prologue(q_raw, k_raw, v_raw, g_raw, b_raw, w_q, w_k, w_v, state=None, g_cap: float = 5.0,
             act: str = "silu", want_state: bool = True, stream=None):
    """Allocate the outputs (and the states after the sequence if wanted), run
    gdn_prologue; ``state`` is a (cs_q, cs_k, cs_v) tuple or None.  Returns a dict
    with q, k, v, g, beta and state (a tuple, or None)."""
    import torch
    B, T, H, K = q_raw.shape
    V = v_raw.shape[-1]
    dev, dt = q_raw.device, q_raw.dtype
    cs = state if state is not None else (None, None, None)
    outs = None
    if want_state:
        outs = (torch.empty(B, 3, H * K, dtype=dt, device=dev), torch.empty(B, 3, H * K, dtype=dt, device=dev),
                torch.empty(B, 3, H * V, dtype=dt, device=dev))
    r = dict(q=torch.empty_like(q_raw), k=torch.empty_like(k_raw), v=torch.empty_like(v_raw),
             g=torch.empty_like(g_raw), beta=torch.empty_like(b_raw))
    o3 = outs if outs is not None else (None, None, None)
    gdn_prologue(q_raw, k_raw, v_raw, g_raw, b_raw, w_q, w_k, w_v, cs[0], cs[1], cs[2], r["q"],
                 r["k"], r["v"], r["g"], r["beta"], o3[0], o3[1], o3[2], g_cap=g_cap, act=act,
                 stream=stream)
    r["state"] = outs
    return r


def gdn_chunk_fwd_prologue(q_raw, k_raw, v_raw, g_raw, b_raw, w_q, w_k, w_v, cs_q, cs_k, cs_v,
                           cs_q_out, cs_k_out, cs_v_out, S0, o, S_T, chunk: int = 64,
                           g_cap: float = 5.0, act: str = "silu", stream=None) -> None:
    """The prologue of gdn_prologue and the chunkwise forward of gdn_chunk_fwd in
    one launch: raw projections in (layouts of gdn_prologue), o [B,T,H,V] and/or
    S_T [B,H,K,V] out, the carried states after the sequence in cs_*_out (never
    the incoming ones) or None."""
    import torch
    B, T, H, K, V, gate = _chunk_fwd_args(q_raw, k_raw, v_raw, g_raw, b_raw, S0, o, S_T)
    dev, dt = q_raw.device, q_raw.dtype
    for t, name, D in ((w_q, "w_q", H * K), (w_k, "w_k", H * K), (w_v, "w_v", H * V)):
        _check(t, name, (D, 4), torch.float32, dev)
    for t, name, D in ((cs_q, "cs_q", H * K), (cs_k, "cs_k", H * K), (cs_v, "cs_v", H * V),
                       (cs_q_out, "cs_q_out", H * K), (cs_k_out, "cs_k_out", H * K),
                       (cs_v_out, "cs_v_out", H * V)):
        _check(t, name, (B, 3, D), dt, dev)
    rc = lib().gdn_chunk_fwd_prologue(_ptr(q_raw), _ptr(k_raw), _ptr(v_raw), _ptr(g_raw),
                                      _ptr(b_raw), _ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(cs_q),
                                      _ptr(cs_k), _ptr(cs_v), _ptr(cs_q_out), _ptr(cs_k_out),
                                      _ptr(cs_v_out), _ptr(S0), _ptr(o), _ptr(S_T), B, T, H, K, V,
                                      int(chunk), float(g_cap), _ACTS[act], _dtype_code(q_raw),
                                      gate, _stream(stream))
    if rc != GDN_OK:
        raise GDNError(rc, "gdn_chunk_fwd_prologue")


def chunk_fwd_prologue(q_raw, k_raw, v_raw, g_raw, b_raw, w_q, w_k, w_v, state=None, S0=None,
                       want_o: bool = True, want_state: bool = True, g_cap: float = 5.0,
                       act: str = "silu", chunk: int = 64, stream=None):
    """Allocate o (if wanted), S_T and the carried states after the sequence (if
    wanted); run gdn_chunk_fwd_prologue.  ``state`` is a (cs_q, cs_k, cs_v) tuple
    or None.  Returns (o, S_T, state)."""
    import torch
    B, T, H, K = q_raw.shape
    V = v_raw.shape[-1]
    dev, dt = q_raw.device, q_raw.dtype
    cs = state if state is not None else (None, None, None)
    outs = None
    if want_state:
        outs = (torch.empty(B, 3, H * K, dtype=dt, device=dev),
                torch.empty(B, 3, H * K, dtype=dt, device=dev),
                torch.empty(B, 3, H * V, dtype=dt, device=dev))
    o3 = outs if outs is not None else (None, None, None)
    o = torch.empty((B, T, H, V), dtype=dt, device=dev) if want_o else None
    S_T = torch.empty((B, H, K, V), dtype=torch.float32, device=dev)
    gdn_chunk_fwd_prologue(q_raw, k_raw, v_raw, g_raw, b_raw, w_q, w_k, w_v, cs[0], cs[1], cs[2],
                           o3[0], o3[1], o3[2], S0, o, S_T, chunk=chunk, g_cap=g_cap, act=act,
                           stream=stream)
    return o, S_T, outs


def gdn_recurrent_step_prologue(q_raw, k_raw, v_raw, g_raw, b_raw, w_q, w_k, w_v, cs_q, cs_k,
                                cs_v, cs_q_out, cs_k_out, cs_v_out, S, o, g_cap: float = 5.0,
                                act: str = "silu", stream=None) -> None:
    """One decode token from the raw projections: prologue and recurrence in one
    kernel.  q_raw, k_raw [N,H,K], v_raw [N,H,V]; g_raw [N,H(,K)], b_raw [N,H] fp32;
    cs_* [N,3,H*D] or None; cs_*_out the states after the token (never the inputs)
    or None; S [N,H,K,V] fp32 updated in place; o [N,H,V] or None."""
    import torch
    if q_raw.dim() != 3 or v_raw.dim() != 3:
        raise ValueError("q_raw, k_raw, v_raw must be [N, H, D]")
    N, H, K = q_raw.shape
    V = v_raw.shape[-1]
    dev = q_raw.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    dt = q_raw.dtype
    _check(k_raw, "k_raw", (N, H, K), dt, dev)
    _check(v_raw, "v_raw", (N, H, V), dt, dev)
    gate = GDN_GATE_CHANNEL if g_raw.dim() == 3 else GDN_GATE_HEAD
    _check(g_raw, "g_raw", (N, H, K) if gate == GDN_GATE_CHANNEL else (N, H), torch.float32, dev)
    _check(b_raw, "b_raw", (N, H), torch.float32, dev)
    for t, name, D in ((w_q, "w_q", H * K), (w_k, "w_k", H * K), (w_v, "w_v", H * V)):
        _check(t, name, (D, 4), torch.float32, dev)
    for t, name, D in ((cs_q, "cs_q", H * K), (cs_k, "cs_k", H * K), (cs_v, "cs_v", H * V),
                       (cs_q_out, "cs_q_out", H * K), (cs_k_out, "cs_k_out", H * K),
                       (cs_v_out, "cs_v_out", H * V)):
        _check(t, name, (N, 3, D), dt, dev)
    _check(S, "S", (N, H, K, V), torch.float32, dev)
    _check(o, "o", (N, H, V), dt, dev)
    rc = lib().gdn_recurrent_step_prologue(
        _ptr(q_raw), _ptr(k_raw), _ptr(v_raw), _ptr(g_raw), _ptr(b_raw), _ptr(w_q), _ptr(w_k),
        _ptr(w_v), _ptr(cs_q), _ptr(cs_k), _ptr(cs_v), _ptr(cs_q_out), _ptr(cs_k_out),
        _ptr(cs_v_out), _ptr(S), _ptr(o), N, H, K, V, float(g_cap), _ACTS[act],
        _dtype_code(q_raw), gate, _stream(stream))
    if rc != GDN_OK:
        raise GDNError(rc, "gdn_recurrent_step_prologue")
