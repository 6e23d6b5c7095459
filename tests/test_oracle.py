"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every check here compares the oracle with something other than itself: a special
case with a closed form, exact rational arithmetic on tiny inputs, the literal
matrix form printed on the Atomic-GDN2 card (section 2.1), an invariant, or the
independently written chunkwise form.  A plausible mistake in the oracle (a
dropped term, a wrong sign, decay on the wrong axis, readout before the write,
a transposed operand) fails at least one of them; ``test_planted_mistakes``
checks that claim on mutated copies of the recurrence.
"""
from fractions import Fraction
import math

import numpy as np
import pytest

import oracle
from oracle import chunked

RNG = np.random.default_rng(1234)


def _rand_inputs(T, K, V, gate="head", rng=RNG, g_scale=1.0, unit=True, s0=True):
    q = rng.standard_normal((T, K))
    k = rng.standard_normal((T, K))
    if unit:
        q /= np.linalg.norm(q, axis=1, keepdims=True)
        k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, V))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    graw = rng.standard_normal((T, K) if gate == "channel" else T)
    g = -np.log1p(np.exp(graw)) * g_scale
    S0 = 0.3 * rng.standard_normal((K, V)) if s0 else None
    f = lambda a: None if a is None else a.astype(np.float32)
    return dict(q=f(q), k=f(k), v=f(v), g=f(g), beta=f(beta),
                S0=None if S0 is None else S0.astype(np.float32).astype(np.float64))


def _dense_reference(q, k, v, g, beta, S0):
    """The matrix form exactly as printed: S_t = (I - b k k^T) Diag(a) S + b k v^T,
    o_t = S_t^T q_t, with explicit K x K matrices."""
    T, K = q.shape
    V = v.shape[1]
    S = np.zeros((K, V)) if S0 is None else np.array(S0, np.float64)
    o = np.zeros((T, V))
    for t in range(T):
        kt = k[t].astype(np.float64)[:, None]
        gt = np.asarray(g[t], np.float64)
        a = np.exp(gt) * np.ones(K)
        E = np.eye(K) - float(beta[t]) * (kt @ kt.T)
        S = E @ np.diag(a) @ S + float(beta[t]) * kt @ v[t].astype(np.float64)[None, :]
        o[t] = S.T @ q[t].astype(np.float64)
    return o, S


def _rel(x, ref):
    return np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300)


# --- pin 1: beta = 0 and g = 0 leave the state alone; o_t = S0^T q_t ----------
def test_identity_update_keeps_state_and_reads_S0():
    T, K, V = 20, 16, 12
    d = _rand_inputs(T, K, V)
    d["beta"][:] = 0
    d["g"][:] = 0
    o, S = oracle.slice_run(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    assert np.array_equal(S, d["S0"])  # bitwise: every update is an exact identity
    ref = d["q"].astype(np.float64) @ d["S0"]  # row t = (S0^T q_t)^T
    assert _rel(o, ref) < 1e-14


# --- pin 2: delta rule recalls exactly with orthonormal keys -------------------
def _hadamard(n):
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H / math.sqrt(n)


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_orthonormal_keys_recall_exactly(gate):
    K, V = 16, 8
    rng = np.random.default_rng(7)
    keys = _hadamard(K)[rng.permutation(K)] * rng.choice([-1.0, 1.0], size=(K, 1))
    T = K
    v = rng.standard_normal((T, V)).astype(np.float32)
    S0 = rng.standard_normal((K, V))  # any initial memory is overwritten
    g = np.zeros((T, K) if gate == "channel" else T, np.float32)
    beta = np.ones(T, np.float32)
    kf = keys.astype(np.float32)  # +-1/4 entries: exact in fp32
    o, S = oracle.slice_run(kf, kf, v, g, beta, S0)
    # reading with q_t = k_t right after writing (k_t, v_t) returns v_t
    assert np.max(np.abs(o - v)) < 1e-14
    # and every key still retrieves its own value at the end
    assert np.max(np.abs(kf.astype(np.float64) @ S - v)) < 1e-14


def test_orthonormal_keys_from_qr_recall_to_input_precision():
    K, V, T = 32, 16, 24
    rng = np.random.default_rng(3)
    Qm, _ = np.linalg.qr(rng.standard_normal((K, K)))
    kf = Qm[:T].astype(np.float32)
    v = rng.standard_normal((T, V)).astype(np.float32)
    o, S = oracle.slice_run(kf, kf, v, np.zeros(T, np.float32), np.ones(T, np.float32),
                            rng.standard_normal((K, V)))
    # keys are orthonormal only to fp32 rounding (~1e-7)
    assert np.max(np.abs(o - v)) < 1e-5


def test_rewriting_a_key_replaces_its_value():
    """Delta rule overwrites; a purely additive (linear-attention) write would sum."""
    K, V = 8, 4
    e0 = np.zeros(K, np.float32)
    e0[0] = 1
    e1 = np.zeros(K, np.float32)
    e1[1] = 1
    k = np.stack([e0, e1, e0])
    v = np.array([[1, 2, 3, 4], [5, 6, 7, 8], [-1, 0.5, 2, -3]], np.float32)
    o, S = oracle.slice_run(k, k, v, np.zeros(3, np.float32), np.ones(3, np.float32))
    assert np.array_equal(S[0], v[2].astype(np.float64))
    assert np.array_equal(S[1], v[1].astype(np.float64))
    assert np.array_equal(o[2], v[2].astype(np.float64))


# --- pin 3: channel gate replicated across K == scalar gate --------------------
def test_replicated_channel_gate_equals_scalar_gate():
    T, K, V = 50, 16, 8
    d = _rand_inputs(T, K, V)
    gch = np.repeat(d["g"][:, None], K, axis=1)
    o1, S1 = oracle.slice_run(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    o2, S2 = oracle.slice_run(d["q"], d["k"], d["v"], gch, d["beta"], d["S0"])
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


# --- pin 4: chunkwise form == token recurrence ----------------------------------
@pytest.mark.parametrize("gate", ["head", "channel"])
@pytest.mark.parametrize("T", [1, 5, 37, 64, 100, 130])
@pytest.mark.parametrize("C", [1, 4, 16, 64])
def test_chunked_form_matches_recurrence(gate, T, C):
    K, V = 8, 6
    d = _rand_inputs(T, K, V, gate=gate, rng=np.random.default_rng(T * 100 + C))
    o1, S1 = oracle.slice_run(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    o2, S2 = chunked.slice_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], chunk=C)
    assert _rel(o2, o1) < 1e-12
    assert _rel(S2, S1) < 1e-12


# --- pin 5: rank-1 evaluation == the printed dense matrix form ------------------
@pytest.mark.parametrize("gate", ["head", "channel"])
def test_matches_printed_dense_form(gate):
    T, K, V = 40, 12, 7
    d = _rand_inputs(T, K, V, gate=gate)
    o1, S1 = oracle.slice_run(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    o2, S2 = _dense_reference(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    assert _rel(o1, o2) < 1e-13
    assert _rel(S1, S2) < 1e-13


def test_exact_rational_brute_force():
    """Tiny case in exact rational arithmetic (decay factors taken as the exact
    rationals of the doubles exp(g) returns)."""
    K, V, T = 3, 2, 4
    rng = np.random.default_rng(11)
    # dyadic inputs: exactly representable in fp32
    q = (rng.integers(-8, 9, (T, K)) / 8).astype(np.float32)
    k = (rng.integers(-8, 9, (T, K)) / 8).astype(np.float32)
    v = (rng.integers(-8, 9, (T, V)) / 4).astype(np.float32)
    beta = (rng.integers(1, 8, T) / 8).astype(np.float32)
    g = (-rng.integers(0, 5, (T, K)) / 4).astype(np.float32)
    S0 = rng.integers(-4, 5, (K, V)) / 2.0
    o, S = oracle.slice_run(q, k, v, g, beta, S0)
    F = Fraction
    Sx = [[F(float(S0[c, j])) for j in range(V)] for c in range(K)]
    for t in range(T):
        a = [F(math.exp(float(g[t, c]))) for c in range(K)]
        b = F(float(beta[t]))
        kt = [F(float(x)) for x in k[t]]
        DS = [[a[c] * Sx[c][j] for j in range(V)] for c in range(K)]
        # (I - b k k^T) DS + b k v^T, entry by entry
        kDS = [sum(kt[c] * DS[c][j] for c in range(K)) for j in range(V)]
        Sx = [[DS[c][j] - b * kt[c] * kDS[j] + b * kt[c] * F(float(v[t, j]))
               for j in range(V)] for c in range(K)]
        ot = [sum(Sx[c][j] * F(float(q[t, c])) for c in range(K)) for j in range(V)]
        for j in range(V):
            assert abs(float(ot[j]) - o[t, j]) <= 1e-14 * (1 + abs(float(ot[j])))
    for c in range(K):
        for j in range(V):
            assert abs(float(Sx[c][j]) - S[c, j]) <= 1e-14 * (1 + abs(float(Sx[c][j])))


# --- pin 6: with beta = 0, the channel gate decays the rows of S ------------------
def test_decay_only_closed_form():
    T, K, V = 30, 10, 5
    d = _rand_inputs(T, K, V, gate="channel")
    d["beta"][:] = 0
    o, S = oracle.slice_run(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    gam = np.cumsum(d["g"].astype(np.float64), axis=0)
    assert _rel(S, np.exp(gam[-1])[:, None] * d["S0"]) < 1e-14
    ref_o = np.stack([(np.exp(gam[t])[:, None] * d["S0"]).T @ d["q"][t].astype(np.float64)
                      for t in range(T)])
    assert _rel(o, ref_o) < 1e-13


# --- pin 7: linear in (S0, v) for fixed q, k, g, beta ----------------------------
def test_linearity_in_state_and_values():
    T, K, V = 25, 8, 6
    rng = np.random.default_rng(5)
    d = _rand_inputs(T, K, V, gate="channel", rng=rng)
    # values on a 1/64 grid, so that the combined v below is stored exactly in fp32
    d["v"] = (np.round(d["v"].astype(np.float64) * 64) / 64).astype(np.float32)
    v2 = (np.round(rng.standard_normal((T, V)) * 64) / 64).astype(np.float32)
    S2 = rng.standard_normal((K, V))
    a, b = 0.75, -1.5  # exact in fp32, so the combined v is stored exactly
    vc = (a * d["v"].astype(np.float64) + b * v2.astype(np.float64)).astype(np.float32)
    assert np.array_equal(vc.astype(np.float64), a * d["v"].astype(np.float64) + b * v2)
    o1, S1 = oracle.slice_run(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    o2, Sb = oracle.slice_run(d["q"], d["k"], v2, d["g"], d["beta"], S2)
    oc, Sc = oracle.slice_run(d["q"], d["k"], vc, d["g"], d["beta"], a * d["S0"] + b * S2)
    assert _rel(oc, a * o1 + b * o2) < 1e-12
    assert _rel(Sc, a * S1 + b * Sb) < 1e-12


# --- pin 8: value columns never mix ------------------------------------------------
def test_value_columns_are_separable():
    T, K, V = 33, 8, 10
    d = _rand_inputs(T, K, V, gate="channel")
    o, S = oracle.slice_run(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    for lo, hi in [(0, 3), (3, 10), (5, 6)]:
        oo, SS = oracle.slice_run(d["q"], d["k"], np.ascontiguousarray(d["v"][:, lo:hi]),
                                  d["g"], d["beta"], np.ascontiguousarray(d["S0"][:, lo:hi]))
        assert np.array_equal(oo, o[:, lo:hi]) and np.array_equal(SS, S[:, lo:hi])


# --- pin 9: state passing -------------------------------------------------------------
def test_state_passing_split_equals_one_call():
    T, K, V = 70, 8, 6
    d = _rand_inputs(T, K, V, gate="channel")
    o, S = oracle.slice_run(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    S_mid = d["S0"]
    outs = []
    for lo, hi in [(0, 13), (13, 64), (64, 70)]:
        sl = slice(lo, hi)
        oo, S_mid = oracle.slice_run(d["q"][sl], d["k"][sl], d["v"][sl], d["g"][sl],
                                     d["beta"][sl], S_mid)
        outs.append(oo)
    assert np.array_equal(np.concatenate(outs), o) and np.array_equal(S_mid, S)


# --- pin 10: non-expansion with unit keys, beta in [0,1], alpha <= 1 -------------
def test_state_norm_never_grows_more_than_the_write():
    T, K, V = 60, 12, 9
    d = _rand_inputs(T, K, V, gate="channel")
    S = d["S0"]
    for t in range(T):
        sl = slice(t, t + 1)
        _, S_new = oracle.slice_run(d["q"][sl], d["k"][sl], d["v"][sl], d["g"][sl],
                                    d["beta"][sl], S)
        bound = np.linalg.norm(S) + float(d["beta"][t]) * np.linalg.norm(d["v"][t])
        assert np.linalg.norm(S_new) <= bound * (1 + 1e-12)
        S = S_new


# --- batched entry points are the slice routine over the right strides ------------
@pytest.mark.parametrize("gate", ["head", "channel"])
def test_forward_batched_layout(gate):
    B, T, H, K, V = 2, 19, 3, 8, 5
    rng = np.random.default_rng(9)
    q = rng.standard_normal((B, T, H, K)).astype(np.float32)
    k = rng.standard_normal((B, T, H, K)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, V)).astype(np.float32)
    beta = rng.uniform(0, 1, (B, T, H)).astype(np.float32)
    g = -rng.uniform(0, 2, (B, T, H, K) if gate == "channel" else (B, T, H)).astype(np.float32)
    S0 = rng.standard_normal((B, H, K, V)).astype(np.float32)
    o, S = oracle.forward(q, k, v, g, beta, S0)
    for b in range(B):
        for h in range(H):
            oo, SS = _dense_reference(q[b, :, h], k[b, :, h], v[b, :, h], g[b, :, h],
                                      beta[b, :, h], S0[b, h].astype(np.float64))
            assert _rel(o[b, :, h], oo) < 1e-13 and _rel(S[b, h], SS) < 1e-13
    # decode over [steps, N, H] is the same recurrence with the time axis first
    od, Sd = oracle.decode(q.transpose(1, 0, 2, 3), k.transpose(1, 0, 2, 3),
                           v.transpose(1, 0, 2, 3),
                           np.ascontiguousarray(np.moveaxis(g, 1, 0)),
                           beta.transpose(1, 0, 2), S0)
    assert np.array_equal(od, o.transpose(1, 0, 2, 3)) and np.array_equal(Sd, S)


def test_empty_sequence_returns_initial_state():
    K, V = 4, 3
    S0 = np.arange(12, dtype=np.float64).reshape(K, V)
    z = np.zeros((0, K), np.float32)
    o, S = oracle.slice_run(z, z, np.zeros((0, V), np.float32), np.zeros(0, np.float32),
                            np.zeros(0, np.float32), S0)
    assert o.shape == (0, V) and np.array_equal(S, S0)


# --- the pins catch planted mistakes ----------------------------------------------
def _mutant(q, k, v, g, beta, S0, bug):
    """A copy of the recurrence with one plausible mistake planted (CPU only)."""
    T, K = q.shape
    V = v.shape[1]
    S = np.array(S0, np.float64)
    o = np.zeros((T, V))
    for t in range(T):
        a = np.exp(np.asarray(g[t], np.float64)) * np.ones(K)
        kt, qt, vt, b = (k[t].astype(np.float64), q[t].astype(np.float64),
                         v[t].astype(np.float64), float(beta[t]))
        S = (S * a[None, :V] if (bug == "decay_cols" and K == V) else S * a[:, None])
        u = S.T @ kt
        if bug == "no_error_term":
            u = 0 * u
        if bug == "sign":
            u = -u
        if bug == "read_before":
            o[t] = S.T @ qt
        S = S + b * np.outer(kt, vt - u)
        if bug != "read_before":
            o[t] = (S @ qt) if (bug == "transposed_read" and K == V) else S.T @ qt
    return o, S


@pytest.mark.parametrize("bug", ["no_error_term", "sign", "read_before", "decay_cols",
                                 "transposed_read"])
def test_planted_mistakes_are_caught(bug):
    T, K, V = 16, 16, 16
    d = _rand_inputs(T, K, V, gate="channel", rng=np.random.default_rng(21))
    mo, mS = _mutant(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], bug)
    ro, rS = _dense_reference(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    assert max(_rel(mo, ro), _rel(mS, rS)) > 1e-3
