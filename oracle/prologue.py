"""fp64 prologue of the gated delta rule: the steps between the projections and
the recurrence (numpy).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): only the tests may use it.
It shares no code with the HIP library.

What the pages fix:
  * DeltaNet layers carry a kernel-4 convolution ("Hybrid layouts: three DeltaNet,
    one attention", 01 Concept); a recurrent layer's convolution is causal.
  * g = -min(softplus(g_raw), 160 / bs2) with bs2 = 32, i.e. a cap of 5, and
    alpha = exp(g) (Atomic-GDN2 card, section 2.1).
  * beta is a per-token update gate (same section).
Readings where they are silent: the convolution is depthwise (one 4-tap filter
per channel) over each of q, k and v, with tap j multiplying token t - 3 + j;
it may be followed by SiLU (the pages name no activation, so both are offered);
q and k are divided by their L2 norm over the K channels of their head (floor
1e-12); beta = sigmoid(b_raw).  The convolution of the first tokens reads a
carried state: the last three raw inputs before the sequence (zeros if absent),
and returns the last three raw inputs of the sequence for the next call.

Layouts: q_raw, k_raw [B,T,H,K]; v_raw [B,T,H,V]; g_raw [B,T,H] or [B,T,H,K];
b_raw [B,T,H]; filter weights [H*K, 4] / [H*V, 4] (channel c = h * K + x);
convolution states [B, 3, H*K] / [B, 3, H*V] (row j = token j - 3).
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    if x is None:
        return None
    if not isinstance(x, np.ndarray):
        x = x.detach().to("cpu").double().numpy()
    return np.array(x, np.float64)


def conv4(x, w, state=None):
    """Causal depthwise 4-tap convolution along time.  x [B,T,D], w [D,4],
    state [B,3,D] or None.  Returns (y [B,T,D], state_out [B,3,D])."""
    x, w = _f64(x), _f64(w)
    B, T, D = x.shape
    prev = np.zeros((B, 3, D)) if state is None else _f64(state)
    ext = np.concatenate([prev, x], axis=1)          # token t sits at ext[:, t + 3]
    y = np.zeros((B, T, D))
    for j in range(4):                               # tap j reads token t - 3 + j
        y += w[None, None, :, j] * ext[:, j:j + T]
    return y, ext[:, T:T + 3].copy()


def silu(x):
    return x / (1.0 + np.exp(-x))


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def softplus(x):
    """log(1 + e^x), evaluated without overflow."""
    return np.logaddexp(0.0, x)


def l2norm(x, axis=-1, floor=1e-12):
    return x / np.maximum(np.linalg.norm(x, axis=axis, keepdims=True), floor)


def prologue(q_raw, k_raw, v_raw, g_raw, b_raw, wq, wk, wv, silu_act=True, cap=5.0,
             state_q=None, state_k=None, state_v=None):
    """The prologue of one chunk-mode call.  Returns a dict with q, k [B,T,H,K],
    v [B,T,H,V], g (shape of g_raw), beta [B,T,H] and the convolution states
    state_q, state_k, state_v after the sequence, all float64."""
    q_raw, k_raw, v_raw, g_raw, b_raw = (_f64(x) for x in (q_raw, k_raw, v_raw, g_raw, b_raw))
    B, T, H, K = q_raw.shape
    V = v_raw.shape[-1]
    act = silu if silu_act else (lambda x: x)
    cq, sq = conv4(q_raw.reshape(B, T, H * K), wq, state_q)
    ck, sk = conv4(k_raw.reshape(B, T, H * K), wk, state_k)
    cv, sv = conv4(v_raw.reshape(B, T, H * V), wv, state_v)
    q = l2norm(act(cq).reshape(B, T, H, K))
    k = l2norm(act(ck).reshape(B, T, H, K))
    v = act(cv).reshape(B, T, H, V)
    g = -np.minimum(softplus(g_raw), cap)
    beta = sigmoid(b_raw)
    return dict(q=q, k=k, v=v, g=g, beta=beta, state_q=sq, state_k=sk, state_v=sv)
