"""fp64 gradients of the gated delta rule, token by token in reverse (numpy).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): only the tests may use it.
It shares no code with the HIP library.

The Atomic-GDN2 model card times its kernel forward and backward together
(section 5.1) and trains with the chunk mode; this module is the definition
that a backward kernel has to reproduce: the gradients of a scalar loss L with
respect to every input of the recurrence of section 2.1, given dL/do_t for every
token and dL/dS_T for the final state.

Forward, one (batch, head) slice, token t (alpha_t = exp(g_t), a scalar per
token for the scalar gate and a K-vector for the per-key-channel gate):
    Sd  = Diag(alpha_t) S_{t-1}
    u   = Sd^T k_t
    d   = beta_t (v_t - u)
    S_t = Sd + k_t d^T
    o_t = S_t^T q_t
This is (I - beta k k^T) Diag(alpha) S + beta k v^T read after the write, the
same rank-1 form the forward oracle uses.

Reverse mode, t = T-1 .. 0, carrying G = dL/dS_t (G = dL/dS_T at the start),
each line the derivative of one forward line above:
    from o_t = S_t^T q_t:        dq_t = S_t do_t;      G <- G + q_t do_t^T
    from S_t = Sd + k_t d^T:     dSd = G;  dk_t = G d;  dd = G^T k_t
    from d = beta (v - u):       dv_t = beta dd;  dbeta_t = (v_t - u) . dd;  du = -beta dd
    from u = Sd^T k_t:           dk_t += Sd du;        dSd += k_t du^T
    from Sd = Diag(alpha) S:     dL/dS_{t-1} = Diag(alpha) dSd;
                                 dalpha = rowsum(S_{t-1} * dSd);  dg = alpha * dalpha
For the scalar gate dg_t is the sum of that vector over the K channels.  The
states S_{t-1} are kept from a forward sweep; nothing is approximated.

Layouts as in the forward: q, k [B,T,H,K]; v, do [B,T,H,V]; g [B,T,H] or
[B,T,H,K]; beta [B,T,H]; S0, dS_T [B,H,K,V] (either may be None = zeros).
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    """float64 host copy of a numpy array or torch tensor (exact upcast)."""
    if x is None:
        return None
    if not isinstance(x, np.ndarray):
        x = x.detach().to("cpu").double().numpy()
    return np.array(x, np.float64)


def backward(q, k, v, g, beta, S0, do, dS_T):
    """Gradients of L given do = dL/do [B,T,H,V] and dS_T = dL/dS_T [B,H,K,V].

    Returns a dict of float64 arrays: dq, dk [B,T,H,K]; dv [B,T,H,V]; dg in the
    shape of g; dbeta [B,T,H]; dS0 [B,H,K,V].
    """
    q, k, v, g, beta, S0, do, dS_T = (_f64(x) for x in (q, k, v, g, beta, S0, do, dS_T))
    B, T, H, K = q.shape
    V = v.shape[-1]
    channel = g.ndim == 4
    assert k.shape == q.shape and v.shape == (B, T, H, V) and beta.shape == (B, T, H)
    assert do.shape == (B, T, H, V)
    # slice-major views: [B, H, T, ...]
    Q = q.transpose(0, 2, 1, 3)
    Kk = k.transpose(0, 2, 1, 3)
    Vv = v.transpose(0, 2, 1, 3)
    dO = do.transpose(0, 2, 1, 3)
    Be = beta.transpose(0, 2, 1)
    if channel:
        Al = np.exp(g.transpose(0, 2, 1, 3))                     # [B,H,T,K]
    else:
        Al = np.repeat(np.exp(g.transpose(0, 2, 1))[..., None], K, axis=-1)

    S = np.zeros((B, H, K, V)) if S0 is None else S0.copy()
    before = np.empty((T, B, H, K, V))
    for t in range(T):
        before[t] = S
        Sd = Al[:, :, t, :, None] * S
        u = np.einsum("bhkv,bhk->bhv", Sd, Kk[:, :, t])
        d = Be[:, :, t, None] * (Vv[:, :, t] - u)
        S = Sd + Kk[:, :, t, :, None] * d[:, :, None, :]

    G = np.zeros((B, H, K, V)) if dS_T is None else dS_T.copy()
    dq = np.zeros((B, H, T, K))
    dk = np.zeros((B, H, T, K))
    dv = np.zeros((B, H, T, V))
    dbeta = np.zeros((B, H, T))
    dg = np.zeros((B, H, T, K))
    for t in range(T - 1, -1, -1):
        kt, qt, vt, bt, at = Kk[:, :, t], Q[:, :, t], Vv[:, :, t], Be[:, :, t], Al[:, :, t]
        Sd = at[..., None] * before[t]
        u = np.einsum("bhkv,bhk->bhv", Sd, kt)
        d = bt[..., None] * (vt - u)
        St = Sd + kt[..., None] * d[:, :, None, :]
        # o_t = S_t^T q_t
        dq[:, :, t] = np.einsum("bhkv,bhv->bhk", St, dO[:, :, t])
        G = G + qt[..., None] * dO[:, :, t][:, :, None, :]
        # S_t = Sd + k_t d^T
        dk[:, :, t] = np.einsum("bhkv,bhv->bhk", G, d)
        dd = np.einsum("bhkv,bhk->bhv", G, kt)
        # d = beta (v - u)
        dv[:, :, t] = bt[..., None] * dd
        dbeta[:, :, t] = np.sum((vt - u) * dd, axis=-1)
        du = -bt[..., None] * dd
        # u = Sd^T k_t
        dk[:, :, t] += np.einsum("bhkv,bhv->bhk", Sd, du)
        dSd = G + kt[..., None] * du[:, :, None, :]
        # Sd = Diag(alpha) S_{t-1}
        dg[:, :, t] = at * np.sum(before[t] * dSd, axis=-1)
        G = at[..., None] * dSd

    back = lambda x: x.transpose(0, 2, 1, 3)
    return dict(dq=back(dq), dk=back(dk), dv=back(dv),
                dg=back(dg) if channel else dg.sum(-1).transpose(0, 2, 1),
                dbeta=dbeta.transpose(0, 2, 1), dS0=G)
