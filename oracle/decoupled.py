"""fp64 oracle of the gated delta rule with decoupled erase and write gates (numpy).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): only the tests, the smoke
check and the bench's CPU-baseline leg may import it.  It shares no code with the
HIP library.

Source.  The MindPattern "Gated DeltaNet" page (its corpus finding of 2026-05-22,
the follow-up paper on decoupling the memory's edit operations) names a variant
in which the one scalar beta of the delta rule, which scales both the removal of
the old association of k and the writing of the new one, is split into two
separate gates.  The page gives no formula.  The reading taken here is the
plainest one that keeps the rest of the card's recurrence (Atomic-GDN2 model
card, section 2.1) unchanged: beta's place in the removal term goes to an erase
gate e_t, its place in the write term to a write gate w_t, one of each per
(token, head):

    S_t = (I - e_t k_t k_t^T) Diag(alpha_t) S_{t-1} + w_t k_t v_t^T,
    o_t = S_t^T q_t,          alpha_t = exp(g_t)  (scalar or per key channel).

With e = w = beta this is the card's recurrence.  With e = 0 the memory only
adds (a gated linear-attention memory); with w = 0 it only forgets.

Functions
---------
forward(q, k, v, g, erase, write, S0=None, want_o=True) -> (o, S_T)   float64
    the token recurrence above, all (batch, head) slices at once.
chunk_step / slice_chunked
    the chunkwise form of the same recurrence for one slice, used to pin
    ``forward`` (derivation in ``chunk_step``).
decode(q, k, v, g, erase, write, S) -> (o, S')
    chained single-token steps from a given state.

Inputs may be numpy arrays or torch tensors of any float dtype; they are upcast
to float64 (exact for bf16 and fp32) before any arithmetic.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    if x is None:
        return None
    if not isinstance(x, np.ndarray):  # torch tensor
        x = x.detach().to("cpu").double().numpy()
    return np.array(x, dtype=np.float64, copy=True)


def _alpha(g_t, K):
    """exp(g) for one token over [B, H] (scalar gate) or [B, H, K] (channel gate),
    returned as [B, H, K]."""
    a = np.exp(g_t)
    if a.ndim == 2:
        a = np.repeat(a[..., None], K, axis=-1)
    return a


def forward(q, k, v, g, erase, write, S0=None, want_o: bool = True):
    """Token recurrence over q, k [B,T,H,K], v [B,T,H,V], g [B,T,H] or [B,T,H,K],
    erase, write [B,T,H]; S0 [B,H,K,V] or None (zeros).

    Returns (o [B,T,H,V] or None, S_T [B,H,K,V]) as float64 arrays.
    """
    q, k, v, g, e, w, S0 = (_f64(x) for x in (q, k, v, g, erase, write, S0))
    B, T, H, K = k.shape
    V = v.shape[-1]
    assert q.shape == k.shape and v.shape[:3] == (B, T, H)
    assert e.shape == (B, T, H) and w.shape == (B, T, H)
    assert g.shape in ((B, T, H), (B, T, H, K))
    S = np.zeros((B, H, K, V)) if S0 is None else S0.reshape(B, H, K, V).copy()
    o = np.zeros((B, T, H, V)) if want_o else None
    for t in range(T):
        kt = k[:, t]                                          # [B,H,K]
        S = _alpha(g[:, t], K)[..., None] * S                 # Diag(alpha_t) S_{t-1}
        u = np.einsum("bhk,bhkv->bhv", kt, S)                 # k^T (Diag(alpha) S)
        # (I - e k k^T) (Diag(alpha) S) = Diag(alpha) S - e k u^T
        S = S - e[:, t, :, None, None] * kt[..., :, None] * u[..., None, :]
        S = S + w[:, t, :, None, None] * kt[..., :, None] * v[:, t, :, None, :]
        if want_o:
            o[:, t] = np.einsum("bhk,bhkv->bhv", q[:, t], S)
    return o, S


def decode(q, k, v, g, erase, write, S):
    """Chained decode steps: q, k [steps,N,H,K], v [steps,N,H,V], g [steps,N,H(,K)],
    erase, write [steps,N,H]; S [N,H,K,V] the state before the first step.

    Returns (o [steps,N,H,V], S after the last step) as float64 arrays.  A chain of
    steps over N sequences is the recurrence with the step axis as time.
    """
    q, k, v, g, e, w = (_f64(x) for x in (q, k, v, g, erase, write))
    S = _f64(S)
    tr = lambda x: None if x is None else np.ascontiguousarray(np.swapaxes(x, 0, 1))
    o, S_T = forward(tr(q), tr(k), tr(v), tr(g), tr(e), tr(w), S)
    return np.ascontiguousarray(np.swapaxes(o, 0, 1)), S_T


def chunk_step(q, k, v, g, erase, write, S):
    """One chunk of n tokens of one slice entering with state S [K,V]:
    q, k [n,K]; v [n,V]; g [n] or [n,K]; erase, write [n].  Returns (o [n,V], S').

    Derivation (the card's chunkwise algebra with beta split in two).  With
    gamma_t the running sum of g inside the chunk (per key channel) and
    d_t = w_t v_t - e_t (Diag(alpha_t) S_{t-1})^T k_t, every state is
        S_t = Diag(e^{gamma_t}) S + sum_{s<=t} Diag(e^{gamma_t - gamma_s}) k_s d_s^T.
    Putting S_{t-1} into d_t:
        d_t + e_t sum_{s<t} G_ts d_s = w_t v_t - e_t (e^{gamma_t} * k_t)^T S,
        G_ts = sum_c k_tc k_sc e^{gamma_tc - gamma_sc},
    i.e. (I + diag(e) G_<) D = diag(w) V - diag(e) K+ S, a unit lower triangular
    system.  Then o_t = (e^{gamma_t} * q_t)^T S + sum_{s<=t} P_ts d_s with
    P_ts = sum_c q_tc k_sc e^{gamma_tc - gamma_sc}, and
    S' = Diag(e^{gamma_n}) S + sum_t Diag(e^{gamma_n - gamma_t}) k_t d_t^T.
    """
    q, k, v, g, e, w, S = (np.asarray(x, np.float64) for x in (q, k, v, g, erase, write, S))
    n, K = k.shape
    gam = np.cumsum(g if g.ndim == 2 else np.repeat(g[:, None], K, axis=1), axis=0)   # [n,K]
    # decayed inner products: X_ts = sum_c x_tc k_sc e^{gamma_tc - gamma_sc}
    # (only s <= t is used; the rest is set to 0 rather than exponentiated)
    causal = (np.arange(n)[:, None] >= np.arange(n)[None, :])[..., None]
    dec = np.exp(np.where(causal, gam[:, None, :] - gam[None, :, :], -np.inf))   # [t, s, c]
    G = np.einsum("tc,sc,tsc->ts", k, k, dec)
    P = np.einsum("tc,sc,tsc->ts", q, k, dec)
    lower = np.tril(np.ones((n, n)), -1)
    Kp = np.exp(gam) * k
    Qp = np.exp(gam) * q
    A = np.eye(n) + e[:, None] * G * lower
    D = np.linalg.solve(A, w[:, None] * v - e[:, None] * (Kp @ S))
    o = Qp @ S + (P * (lower + np.eye(n))) @ D
    Km = np.exp(gam[-1][None, :] - gam) * k
    S_next = np.exp(gam[-1])[:, None] * S + Km.T @ D
    return o, S_next


def slice_chunked(q, k, v, g, erase, write, S0=None, chunk: int = 64):
    """The chunkwise form over a whole slice: q, k [T,K], v [T,V], g [T] or [T,K],
    erase, write [T]; S0 [K,V] or None.  Returns (o [T,V], S_T [K,V])."""
    q, k, v, g, e, w = (_f64(x) for x in (q, k, v, g, erase, write))
    T, K = k.shape
    V = v.shape[1]
    S = np.zeros((K, V)) if S0 is None else _f64(S0)
    o = np.zeros((T, V))
    for t0 in range(0, T, chunk):
        sl = slice(t0, min(T, t0 + chunk))
        o[sl], S = chunk_step(q[sl], k[sl], v[sl], g[sl], e[sl], w[sl], S)
    return o, S
