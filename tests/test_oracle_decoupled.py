"""Pins of the decoupled-gate oracle (``oracle.decoupled``) against what the pages
and the mathematics fix, not against itself.

The pages name the variant (MindPattern "Gated DeltaNet" page, finding of
2026-05-22: beta split into separate erase and write gates) but print no
formula; the reading pinned here is
    S_t = (I - e_t k_t k_t^T) Diag(alpha_t) S_{t-1} + w_t k_t v_t^T,  o_t = S_t^T q_t.
Pins:
  * e = w = beta is the card's recurrence (Atomic-GDN2 card, section 2.1), as
    computed by the separately pinned C oracle;
  * for e > 0, writing w v is writing e ((w / e) v): the decoupled memory equals
    the card's memory with beta = e and v scaled by w / e (exact in fp32 when the
    ratio is a power of two);
  * e = 0 is an additive (gated linear-attention) memory with a closed form;
  * with orthonormal keys and no decay, the value read back for a key follows
    the scalar recursion r <- (1 - e) r + w v;
  * finite differences: S_T is affine in every gate, with the slopes of the last
    token known in closed form;
  * the chunkwise form (a separate derivation) agrees with the recurrence.
``test_planted_mistakes_are_caught`` checks that a plausible mistake in the
recurrence fails at least one pin.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import decoupled as dg


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _inputs(B, T, H, K, V, gate, seed, s0=True):
    """fp32-representable random inputs (stored as float64 arrays)."""
    rng = np.random.default_rng(seed)
    f = lambda a: a.astype(np.float32).astype(np.float64)
    d = dict(q=f(_unit(rng.standard_normal((B, T, H, K)))),
             k=f(_unit(rng.standard_normal((B, T, H, K)))),
             v=f(rng.standard_normal((B, T, H, V))))
    gs = (B, T, H, K) if gate == "channel" else (B, T, H)
    d["g"] = f(-np.log1p(np.exp(rng.standard_normal(gs))))
    d["e"] = f(1 / (1 + np.exp(-rng.standard_normal((B, T, H)))))
    d["w"] = f(1 / (1 + np.exp(-rng.standard_normal((B, T, H)))))
    d["S0"] = f(0.3 * rng.standard_normal((B, H, K, V))) if s0 else None
    return d


def _rel(x, ref):
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300))


def _run(fwd, d, **over):
    x = dict(d, **over)
    return fwd(x["q"], x["k"], x["v"], x["g"], x["e"], x["w"], x["S0"])


# --- the pins, as functions of a recurrence implementation ---------------------------
def pin_equal_gates(fwd, gate, tol=1e-12):
    """e = w = beta against the C oracle of the card's recurrence."""
    d = _inputs(2, 37, 3, 16, 8, gate, seed=11)
    o, S = _run(fwd, d, w=d["e"])
    ro, rS = oracle.forward(d["q"], d["k"], d["v"], d["g"], d["e"], d["S0"])
    return max(_rel(o, ro), _rel(S, rS)) <= tol


def pin_write_rescaling(fwd, gate, tol=1e-12):
    """For e > 0: decoupled(e, w, v) == card(beta = e, v * w / e).  e is drawn from
    {1/4, 1/2, 3/4, 1} and w = e * 2^j, so v * w / e is exact in fp32."""
    B, T, H, K, V = 2, 29, 2, 16, 8
    d = _inputs(B, T, H, K, V, gate, seed=12)
    rng = np.random.default_rng(13)
    e = rng.choice([0.25, 0.5, 0.75, 1.0], size=(B, T, H))
    r = 2.0 ** rng.integers(-2, 2, size=(B, T, H))
    o, S = _run(fwd, d, e=e, w=e * r)
    ro, rS = oracle.forward(d["q"], d["k"], d["v"] * r[..., None], d["g"], e, d["S0"])
    return max(_rel(o, ro), _rel(S, rS)) <= tol


def pin_no_erase_closed_form(fwd, gate, tol=1e-12):
    """e = 0: S_t = Diag(e^{Gamma_t}) S0 + sum_{s<=t} w_s Diag(e^{Gamma_t - Gamma_s}) k_s v_s^T
    with Gamma the running sum of g from the first token; o_t = S_t^T q_t."""
    B, T, H, K, V = 1, 23, 2, 8, 4
    d = _inputs(B, T, H, K, V, gate, seed=14)
    o, S = _run(fwd, d, e=np.zeros((B, T, H)))
    g = d["g"] if gate == "channel" else np.repeat(d["g"][..., None], K, axis=-1)
    Gam = np.cumsum(g, axis=1)                                      # [B,T,H,K]
    ok = True
    for t in range(T):
        St = np.exp(Gam[:, t])[..., None] * d["S0"]
        for s in range(t + 1):
            St = St + (d["w"][:, s, :, None, None] * np.exp(Gam[:, t] - Gam[:, s])[..., None]
                       * d["k"][:, s, :, :, None] * d["v"][:, s, :, None, :])
        ot = np.einsum("bhk,bhkv->bhv", d["q"][:, t], St)
        ok &= _rel(o[:, t], ot) <= tol
        if t == T - 1:
            ok &= _rel(S, St) <= tol
    return bool(ok)


def _hadamard(n):
    Hm = np.array([[1.0]])
    while Hm.shape[0] < n:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    return Hm / math.sqrt(n)


def pin_orthonormal_recursion(fwd, gate, tol=1e-13):
    """Orthonormal keys (rows of a Hadamard matrix, exact in fp32), g = 0: after
    writing key j the value read back with q = k_j is r_j <- (1 - e) r_j + w v;
    a key not written keeps its r_j."""
    K, V, T = 16, 4, 40
    rng = np.random.default_rng(15)
    keys = _hadamard(K)
    idx = rng.integers(0, K, size=T)
    k = keys[idx][None, :, None, :]
    v = rng.standard_normal((1, T, 1, V)).astype(np.float32).astype(np.float64)
    e = rng.choice([0.0, 0.25, 0.5, 1.0], size=(1, T, 1))
    w = rng.choice([0.0, 0.5, 0.75, 1.0], size=(1, T, 1))
    S0 = rng.standard_normal((1, 1, K, V)).astype(np.float32).astype(np.float64)
    g = np.zeros((1, T, 1, K) if gate == "channel" else (1, T, 1))
    o, S = fwd(k, k, v, g, e, w, S0)
    r = keys @ S0[0, 0]                                              # [K, V]: r_j = S^T k_j
    ok = True
    for t in range(T):
        j = idx[t]
        r[j] = (1 - e[0, t, 0]) * r[j] + w[0, t, 0] * v[0, t, 0]
        ok &= np.max(np.abs(o[0, t, 0] - r[j])) <= tol
    ok &= np.max(np.abs(keys @ S[0, 0] - r)) <= tol
    return bool(ok)


def pin_last_token_slopes(fwd, gate, tol=1e-9):
    """S_T is affine in w_t and e_t for every t.  At the last token the slopes are
    dS_T/dw_T = k_T v_T^T and dS_T/de_T = -k_T u^T with u = (Diag(alpha_T) S_{T-1})^T k_T;
    do_T/dw_T = (q_T . k_T) v_T.  Central differences with h = 1/8 are exact up to
    rounding for an affine map; second differences at an interior token vanish."""
    B, T, H, K, V = 1, 12, 1, 8, 4
    d = _inputs(B, T, H, K, V, gate, seed=16)
    h = 0.125
    ok = True

    def bump(name, t, dh):
        x = d[name].copy()
        x[:, t] += dh
        return _run(fwd, d, **{name: x})

    kT, vT, qT = d["k"][0, -1, 0], d["v"][0, -1, 0], d["q"][0, -1, 0]
    (op, Sp), (om, Sm) = bump("w", T - 1, h), bump("w", T - 1, -h)
    ok &= _rel((Sp - Sm)[0, 0] / (2 * h), np.outer(kT, vT)) <= tol
    ok &= _rel((op - om)[0, -1, 0] / (2 * h), (qT @ kT) * vT) <= tol
    # S_{T-1}: the same call on the first T-1 tokens
    sub = {n: (d[n][:, :-1] if n != "S0" else d[n]) for n in d}
    _, S1 = _run(fwd, sub)
    a = np.exp(d["g"][0, -1, 0]) * np.ones(K)
    u = (a[:, None] * S1[0, 0]).T @ kT
    (_, Sp), (_, Sm) = bump("e", T - 1, h), bump("e", T - 1, -h)
    ok &= _rel((Sp - Sm)[0, 0] / (2 * h), -np.outer(kT, u)) <= tol
    for name in ("e", "w"):
        (_, S2), (_, S1b), (_, S0b) = bump(name, 5, 2 * h), bump(name, 5, h), bump(name, 5, 0.0)
        ok &= np.max(np.abs(S2 - 2 * S1b + S0b)) <= tol * max(1.0, np.max(np.abs(S0b)))
    return bool(ok)


def pin_chunked_form(fwd, gate, tol=1e-11):
    """The chunkwise form (chunk 16, ragged last chunk) against the recurrence."""
    d = _inputs(1, 53, 2, 16, 8, gate, seed=17)
    o, S = _run(fwd, d)
    for h in range(2):
        sl = lambda x: x[0, :, h]
        co, cS = dg.slice_chunked(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]),
                                  sl(d["e"]), sl(d["w"]), d["S0"][0, h], chunk=16)
        if max(_rel(o[0, :, h], co), _rel(S[0, h], cS)) > tol:
            return False
    return True


PINS = [pin_equal_gates, pin_write_rescaling, pin_no_erase_closed_form,
        pin_orthonormal_recursion, pin_last_token_slopes, pin_chunked_form]


@pytest.mark.parametrize("gate", ["head", "channel"])
@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_holds_pin(pin, gate):
    assert pin(dg.forward, gate)


def test_chunked_form_handles_hard_resets():
    """g far below the per-channel clamp (alpha < e^-20): both forms stay finite
    and agree."""
    d = _inputs(1, 40, 1, 8, 4, "head", seed=18)
    g = d["g"].copy()
    g[0, ::7, 0] = -150.0
    o, S = dg.forward(d["q"], d["k"], d["v"], g, d["e"], d["w"], d["S0"])
    co, cS = dg.slice_chunked(d["q"][0, :, 0], d["k"][0, :, 0], d["v"][0, :, 0], g[0, :, 0],
                              d["e"][0, :, 0], d["w"][0, :, 0], d["S0"][0, 0], chunk=16)
    assert np.isfinite(co).all() and np.isfinite(cS).all()
    assert max(_rel(o[0, :, 0], co), _rel(S[0, 0], cS)) < 1e-11


def test_decode_chain_is_the_recurrence():
    d = _inputs(3, 6, 2, 8, 4, "channel", seed=19)          # B=3 sequences, 6 steps
    tr = lambda x: np.ascontiguousarray(np.swapaxes(x, 0, 1))
    o, S = dg.decode(tr(d["q"]), tr(d["k"]), tr(d["v"]), tr(d["g"]), tr(d["e"]), tr(d["w"]),
                     d["S0"])
    ro, rS = dg.forward(d["q"], d["k"], d["v"], d["g"], d["e"], d["w"], d["S0"])
    assert np.array_equal(tr(o), ro) and np.array_equal(S, rS)
    # no steps: the state is returned unchanged
    z = lambda x: x[:0]
    o0, S0 = dg.decode(z(tr(d["q"])), z(tr(d["k"])), z(tr(d["v"])), z(tr(d["g"])),
                       z(tr(d["e"])), z(tr(d["w"])), d["S0"])
    assert o0.shape == (0, 3, 2, 4) and np.array_equal(S0, d["S0"])


def test_empty_sequence_and_absent_state():
    d = _inputs(1, 5, 1, 8, 4, "head", seed=20, s0=False)
    o, S = dg.forward(d["q"][:, :0], d["k"][:, :0], d["v"][:, :0], d["g"][:, :0],
                      d["e"][:, :0], d["w"][:, :0], None)
    assert o.shape == (1, 0, 1, 4) and not S.any()
    # w = 0 and no S0: nothing is ever written, whatever e is
    o, S = dg.forward(d["q"], d["k"], d["v"], d["g"], d["e"], np.zeros_like(d["w"]), None)
    assert not o.any() and not S.any()


# --- planted mistakes ------------------------------------------------------------------
def _mutant(bug):
    """A copy of the recurrence with one plausible mistake planted (CPU only)."""
    def fwd(q, k, v, g, e, w, S0):
        q, k, v, g, e, w = (np.asarray(x, np.float64) for x in (q, k, v, g, e, w))
        B, T, H, K = k.shape
        V = v.shape[-1]
        S = np.zeros((B, H, K, V)) if S0 is None else np.array(S0, np.float64)
        o = np.zeros((B, T, H, V))
        for t in range(T):
            kt = k[:, t]
            a = np.exp(g[:, t])
            a = a if a.ndim == 3 else np.repeat(a[..., None], K, axis=-1)
            et, wt = e[:, t, :, None, None], w[:, t, :, None, None]
            if bug == "swap_gates":
                et, wt = wt, et
            elif bug == "erase_uses_write":
                et = wt
            elif bug == "write_uses_erase":
                wt = et
            elif bug == "write_ungated":
                wt = np.ones_like(wt)
            u_src = S if bug == "erase_before_decay" else a[..., None] * S
            if bug != "decay_after_write":
                S = a[..., None] * S
            u = np.einsum("bhk,bhkv->bhv", kt, u_src)
            S = S - et * kt[..., :, None] * u[..., None, :] + wt * kt[..., :, None] * v[:, t, :, None, :]
            if bug == "decay_after_write":
                S = a[..., None] * S
            o[:, t] = np.einsum("bhk,bhkv->bhv", q[:, t], S)
        return o, S
    return fwd


def test_mutant_copy_without_a_mistake_holds_every_pin():
    fwd = _mutant(None)
    assert all(pin(fwd, gate) for pin in PINS[:-1] for gate in ("head", "channel"))


@pytest.mark.parametrize("bug", ["swap_gates", "erase_uses_write", "write_uses_erase",
                                 "write_ungated", "erase_before_decay", "decay_after_write"])
def test_planted_mistakes_are_caught(bug):
    fwd = _mutant(bug)
    held = [pin(fwd, gate) for pin in PINS[:-1] for gate in ("head", "channel")]
    assert not all(held), f"no pin catches {bug}"
