"""fp64 CPU oracle for the Gated DeltaNet mixer forward.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this package.  It shares no code with the HIP
library under ``gated_deltanet_layer_amd``; neither imports the other.

The arithmetic lives in ``gdn_oracle.c`` (plain C, double precision, OpenMP over
independent (batch, head) slices).  This module only builds it with gcc, loads it
with ctypes, and converts the stored inputs to float32 host arrays (an exact
upcast for bf16 and fp32) before the call.

Functions
---------
forward(q, k, v, g, beta, S0=None, want_o=True)  -> (o, S_T)   float64
decode(q, k, v, g, beta, S)                       -> (o, S')    float64
slice_run(q, k, v, g, beta, S0=None)              -> (o, S_T)   one slice, fp64 S0

``chunked`` (numpy) holds the chunkwise form used to pin the oracle.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math). Returns the .so path."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        i, l = ctypes.c_int, ctypes.c_long
        lib.gdn_oracle_slice.argtypes = [i, i, i, i,
                                         f32p, l, f32p, l, f32p, l, f32p, l, f32p, l,
                                         f64p, f64p, l]
        lib.gdn_oracle_slice.restype = i
        lib.gdn_oracle_forward.argtypes = [i, i, i, i, i, i,
                                           f32p, f32p, f32p, f32p, f32p, f32p,
                                           f64p, f64p, i]
        lib.gdn_oracle_forward.restype = i
        lib.gdn_oracle_decode.argtypes = [i, i, i, i, i, i,
                                          f32p, f32p, f32p, f32p, f32p,
                                          f64p, f64p, i]
        lib.gdn_oracle_decode.restype = i
        lib.gdn_oracle_max_threads.argtypes = []
        lib.gdn_oracle_max_threads.restype = i
        _lib = lib
        return lib


def _f32(x) -> np.ndarray:
    """Host float32 copy of a numpy array or torch tensor (exact for bf16/fp32)."""
    if x is None:
        return None
    if not isinstance(x, np.ndarray):  # torch tensor
        x = x.detach().to("cpu").float().numpy()
    return np.ascontiguousarray(x, dtype=np.float32)


def _p32(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _p64(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads() -> int:
    return int(_load().gdn_oracle_max_threads())


def _gate(g: np.ndarray, lead: int, K: int) -> int:
    """1 for a per-key-channel gate (g has a trailing K axis), 0 for a scalar gate."""
    if g.ndim == lead + 1:
        if g.shape[-1] != K:
            raise ValueError("channel gate must have a trailing axis of size K")
        return 1
    if g.ndim == lead:
        return 0
    raise ValueError(f"gate has {g.ndim} dims, expected {lead} or {lead + 1}")


def forward(q, k, v, g, beta, S0=None, want_o: bool = True, nthreads: int = 0):
    """Token-by-token fp64 recurrence over q,k [B,T,H,K], v [B,T,H,V].

    Returns (o [B,T,H,V] or None, S_T [B,H,K,V]) as float64 arrays.
    """
    q, k, v, g, beta, S0 = (_f32(x) for x in (q, k, v, g, beta, S0))
    B, T, H, K = q.shape
    V = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, T, H) and beta.shape == (B, T, H)
    gate = _gate(g, 3, K)
    assert g.shape[:3] == (B, T, H)
    if S0 is not None:
        assert S0.shape == (B, H, K, V)
    o = np.zeros((B, T, H, V), np.float64) if want_o else None
    S_T = np.zeros((B, H, K, V), np.float64)
    rc = _load().gdn_oracle_forward(B, T, H, K, V, gate, _p32(q), _p32(k), _p32(v),
                                    _p32(g), _p32(beta), _p32(S0), _p64(o), _p64(S_T),
                                    int(nthreads))
    if rc != 0:
        raise RuntimeError("gdn_oracle_forward failed")
    return o, S_T


def slice_run(q, k, v, g, beta, S0=None):
    """One slice: q,k [T,K], v [T,V], g [T] or [T,K], beta [T], S0 [K,V] (float64, may be None).

    Returns (o [T,V], S_T [K,V]) float64.  S0 is taken in double precision so that
    states can be carried from one call to the next without rounding.
    """
    q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
    T, K = q.shape
    V = v.shape[1]
    gate = _gate(g, 1, K)
    S = np.zeros((K, V), np.float64) if S0 is None else np.array(S0, np.float64, copy=True)
    S = np.ascontiguousarray(S)
    o = np.zeros((T, V), np.float64)
    gs = K if gate else 1
    rc = _load().gdn_oracle_slice(T, K, V, gate, _p32(q), K, _p32(k), K, _p32(v), V,
                                  _p32(g), gs, _p32(beta), 1, _p64(S), _p64(o), V)
    if rc != 0:
        raise RuntimeError("gdn_oracle_slice failed")
    return o, S


def decode(q, k, v, g, beta, S, nthreads: int = 0):
    """Chained decode steps: q,k [steps,N,H,K], v [steps,N,H,V], g [steps,N,H(,K)],
    beta [steps,N,H]; S [N,H,K,V] initial state (any float dtype).

    Returns (o [steps,N,H,V], S_final [N,H,K,V]) float64.
    """
    q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
    steps, N, H, K = q.shape
    V = v.shape[-1]
    gate = _gate(g, 3, K)
    if not isinstance(S, np.ndarray):
        S = S.detach().to("cpu").double().numpy()
    S = np.ascontiguousarray(np.array(S, np.float64, copy=True))
    assert S.shape == (N, H, K, V)
    o = np.zeros((steps, N, H, V), np.float64)
    rc = _load().gdn_oracle_decode(steps, N, H, K, V, gate, _p32(q), _p32(k), _p32(v),
                                   _p32(g), _p32(beta), _p64(S), _p64(o), int(nthreads))
    if rc != 0:
        raise RuntimeError("gdn_oracle_decode failed")
    return o, S
