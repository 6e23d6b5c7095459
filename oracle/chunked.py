"""Chunkwise fp64 form of the gated delta rule (numpy), used to pin the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The MindPattern "Gated DeltaNet" page (finding of 2026-07-29, the derivation from
softmax attention to KDA) says the chunkwise (training) mode and the fused
recurrent (decode) mode compute the same mathematics.  This module writes the
chunkwise mode out, for one (batch, head) slice, directly from the recurrence of
the Atomic-GDN2 card section 2.1, so that a test can check that both modes agree.

Derivation, for one chunk of n tokens t = 1..n entering with state S (K x V):

* gamma_t = sum_{s<=t} g_s  (per key channel; a scalar gate is broadcast).
* Unrolling S_t = Diag(a_t) S_{t-1} + k_t d_t^T with the delta
  d_t = beta_t (v_t - (Diag(a_t) S_{t-1})^T k_t) gives
      S_t = Diag(e^{gamma_t}) S + sum_{s<=t} Diag(e^{gamma_t - gamma_s}) k_s d_s^T.
* Putting that S_{t-1} into d_t:
      d_t + beta_t sum_{s<t} (sum_c k_tc k_sc e^{gamma_tc - gamma_sc}) d_s
          = beta_t (v_t - (e^{gamma_t} * k_t)^T S),
  i.e. (I + A) D = diag(beta) (V - Kp S) with A strictly lower triangular,
  A_ts = beta_t sum_c k_tc k_sc e^{gamma_tc - gamma_sc}, and Kp_t = e^{gamma_t} * k_t.
  I + A is unit lower triangular, so it is always invertible.
* Outputs: o_t = S_t^T q_t = (e^{gamma_t} * q_t)^T S + sum_{s<=t} P_ts d_s with
  P_ts = sum_c q_tc k_sc e^{gamma_tc - gamma_sc} (lower triangular, diagonal kept).
* Outgoing state: S' = Diag(e^{gamma_n}) S + Km^T D with Km_t = e^{gamma_n - gamma_t} * k_t.

Library primitives (matmul, a linear solve) serve as steps; nothing else is
blocked, fused or reordered.
"""
from __future__ import annotations

import numpy as np


def chunk_step(q, k, v, g, beta, S):
    """One chunk.  q,k [n,K]; v [n,V]; g [n] or [n,K]; beta [n]; S [K,V] (float64).

    Returns (o [n,V], S_next [K,V]).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    beta = np.asarray(beta, np.float64)
    n, K = k.shape
    g = np.asarray(g, np.float64)
    if g.ndim == 1:
        g = np.repeat(g[:, None], K, axis=1)
    gamma = np.cumsum(g, axis=0)                         # [n, K]
    # exponent of the decay between token s and a later token t, per channel
    diff = gamma[:, None, :] - gamma[None, :, :]          # [t, s, K]
    lower_strict = np.tril(np.ones((n, n), bool), -1)
    lower_incl = np.tril(np.ones((n, n), bool), 0)
    # only t >= s is ever used; the upper part is masked before exponentiating
    decay = np.exp(np.where(lower_incl[:, :, None], diff, 0.0))
    A = np.where(lower_strict, beta[:, None] * np.einsum("tc,sc,tsc->ts", k, k, decay), 0.0)
    P = np.where(lower_incl, np.einsum("tc,sc,tsc->ts", q, k, decay), 0.0)
    Kp = np.exp(gamma) * k
    Qp = np.exp(gamma) * q
    Km = np.exp(gamma[-1][None, :] - gamma) * k
    rhs = beta[:, None] * (v - Kp @ S)
    D = np.linalg.solve(np.eye(n) + A, rhs)
    o = Qp @ S + P @ D
    S_next = np.exp(gamma[-1])[:, None] * S + Km.T @ D
    return o, S_next


def slice_forward(q, k, v, g, beta, S0=None, chunk: int = 64):
    """Whole slice in chunks of ``chunk`` tokens (the last one may be partial).

    q,k [T,K]; v [T,V]; g [T] or [T,K]; beta [T]; S0 [K,V] or None.
    Returns (o [T,V], S_T [K,V]) float64.
    """
    q = np.asarray(q, np.float64)
    T, K = q.shape
    V = np.asarray(v).shape[1]
    S = np.zeros((K, V)) if S0 is None else np.array(S0, np.float64, copy=True)
    o = np.zeros((T, V))
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        o[t0:t1], S = chunk_step(q[t0:t1], k[t0:t1], v[t0:t1], g[t0:t1], beta[t0:t1], S)
    return o, S
