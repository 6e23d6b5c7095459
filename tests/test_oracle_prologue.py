"""Pins of the fp64 prologue oracle (``oracle.prologue``) against what the pages
and the mathematics fix, independently of its own code:

* the convolution equals numpy's own 1-D convolution per channel (a library
  routine, with the filter reversed as its definition requires), and special
  filters give closed forms: identity, one-token delay, a four-token sum;
* causality: changing a later token leaves every earlier output unchanged;
* the carried state: a sequence cut in two, with the state passed across the
  cut, equals the whole;
* the gate: g = -min(softplus(g_raw), 5) (Atomic-GDN2 card, section 2.1) at
  points with closed forms (softplus(0) = ln 2, the cap reached, g -> 0 from
  below), beta = sigmoid(b_raw) with sigmoid(0) = 1/2 and symmetry;
* q and k leave with unit L2 norm per head, and a positive rescaling of the
  raw input does not change them; SiLU at known points;
* the g and beta outputs of prologue() itself, element by element, for caps
  5, 2.5, 0.75 and none, from raw inputs built as closed-form preimages
  (g_raw = log(e^c - 1), b_raw = logit(p));
* planted mistakes (an anti-causal filter, reversed taps, normalising over the
  wrong axis, no cap, g_raw and b_raw swapped, the cap argument ignored, a
  flipped gate sign, beta = sigmoid(-b_raw)) fail these pins.
"""
import math

import numpy as np
import pytest

from oracle import prologue as P

RNG = np.random.default_rng(77)


def _np_conv(x, w, state=None):
    """Per-channel numpy.convolve over [state; x]: out[t] = sum_j w[j] x[t-3+j]."""
    B, T, D = x.shape
    prev = np.zeros((B, 3, D)) if state is None else state
    ext = np.concatenate([prev, x], axis=1)
    y = np.zeros((B, T, D))
    for b in range(B):
        for c in range(D):
            # np.convolve flips its second argument: pass the taps reversed
            y[b, :, c] = np.convolve(ext[b, :, c], w[c, ::-1], mode="valid")
    return y


def test_conv_matches_numpy_convolve():
    x = RNG.standard_normal((2, 11, 5))
    w = RNG.standard_normal((5, 4))
    st = RNG.standard_normal((2, 3, 5))
    y, s_out = P.conv4(x, w, st)
    assert np.allclose(y, _np_conv(x, w, st), rtol=1e-13, atol=1e-13)
    assert np.array_equal(s_out, x[:, -3:])


def test_conv_special_filters():
    x = RNG.standard_normal((1, 9, 3))
    st = RNG.standard_normal((1, 3, 3))
    ident = np.tile([0.0, 0.0, 0.0, 1.0], (3, 1))
    delay = np.tile([0.0, 0.0, 1.0, 0.0], (3, 1))
    summ = np.ones((3, 4))
    assert np.array_equal(P.conv4(x, ident, st)[0], x)
    d = P.conv4(x, delay, st)[0]
    assert np.array_equal(d[:, 0], st[:, 2]) and np.array_equal(d[:, 1:], x[:, :-1])
    ext = np.concatenate([st, x], axis=1)
    want = np.stack([ext[:, t:t + 4].sum(axis=1) for t in range(9)], axis=1)
    assert np.allclose(P.conv4(x, summ, st)[0], want, rtol=1e-14, atol=1e-14)


def test_conv_is_causal():
    x = RNG.standard_normal((1, 12, 4))
    w = RNG.standard_normal((4, 4))
    y0 = P.conv4(x, w)[0]
    x2 = x.copy()
    x2[:, 7:] += 10.0
    y1 = P.conv4(x2, w)[0]
    assert np.array_equal(y0[:, :7], y1[:, :7]) and not np.allclose(y0[:, 7:], y1[:, 7:])


def test_short_sequences_and_state_passing():
    x = RNG.standard_normal((2, 10, 6))
    w = RNG.standard_normal((6, 4))
    st = RNG.standard_normal((2, 3, 6))
    full, s_full = P.conv4(x, w, st)
    for cut in (0, 1, 2, 3, 7, 10):
        a, sa = P.conv4(x[:, :cut], w, st)
        b, sb = P.conv4(x[:, cut:], w, sa)
        assert np.allclose(np.concatenate([a, b], axis=1), full, rtol=1e-14, atol=1e-14), cut
        assert np.array_equal(sb, s_full), cut
    # fewer than three tokens: the state keeps the older entries
    one, s1 = P.conv4(x[:, :1], w, st)
    assert np.array_equal(s1[:, :2], st[:, 1:]) and np.array_equal(s1[:, 2], x[:, 0])


def test_gate_and_beta_closed_forms():
    g = -np.minimum(P.softplus(np.array([0.0, 100.0, -50.0, math.log(math.e ** 5 - 1)])), 5.0)
    assert math.isclose(g[0], -math.log(2.0), rel_tol=1e-15)
    assert g[1] == -5.0
    assert -1e-21 < g[2] < 0.0
    assert math.isclose(g[3], -5.0, rel_tol=1e-14)     # softplus(x) = 5 exactly at the cap
    assert P.sigmoid(np.array(0.0)) == 0.5
    x = RNG.standard_normal(20)
    assert np.allclose(P.sigmoid(x) + P.sigmoid(-x), 1.0, rtol=0, atol=1e-15)
    assert math.isclose(float(P.silu(np.array(1.0))), 1.0 / (1.0 + math.exp(-1.0)), rel_tol=1e-15)
    assert P.silu(np.array(0.0)) == 0.0


def _raw(B=2, T=9, H=3, K=4, V=5, gate="channel"):
    r = np.random.default_rng(5)
    d = dict(q_raw=r.standard_normal((B, T, H, K)), k_raw=r.standard_normal((B, T, H, K)),
             v_raw=r.standard_normal((B, T, H, V)),
             g_raw=r.standard_normal((B, T, H, K) if gate == "channel" else (B, T, H)) * 3,
             b_raw=r.standard_normal((B, T, H)),
             wq=r.standard_normal((H * K, 4)), wk=r.standard_normal((H * K, 4)),
             wv=r.standard_normal((H * V, 4)))
    return d


@pytest.mark.parametrize("act", [True, False])
@pytest.mark.parametrize("gate", ["channel", "head"])
def test_prologue_shapes_norms_and_gates(act, gate):
    d = _raw(gate=gate)
    out = P.prologue(**d, silu_act=act)
    assert np.allclose(np.linalg.norm(out["q"], axis=-1), 1.0, rtol=0, atol=1e-14)
    assert np.allclose(np.linalg.norm(out["k"], axis=-1), 1.0, rtol=0, atol=1e-14)
    assert np.all(out["g"] <= 0) and np.all(out["g"] >= -5.0)
    assert np.all((out["beta"] > 0) & (out["beta"] < 1))
    # v is the convolution (and activation) of v_raw, channel by channel
    B, T, H, V = d["v_raw"].shape
    cv = _np_conv(d["v_raw"].reshape(B, T, H * V), d["wv"])
    want = P.silu(cv) if act else cv
    assert np.allclose(out["v"].reshape(B, T, H * V), want, rtol=1e-13, atol=1e-13)
    # a positive rescaling of the raw q (no activation) leaves the normalised q alone
    if not act:
        d2 = dict(d)
        d2["q_raw"] = 7.5 * d["q_raw"]
        assert np.allclose(P.prologue(**d2, silu_act=act)["q"], out["q"], rtol=1e-13, atol=1e-14)


def test_planted_mistakes_are_caught():
    x = RNG.standard_normal((1, 10, 3))
    w = RNG.standard_normal((3, 4))
    ref = _np_conv(x, w)
    # taps applied in the opposite order
    assert not np.allclose(P.conv4(x, w[:, ::-1])[0], ref)
    # anti-causal: a filter that reads tokens t .. t+3 (shift the input back by 3)
    xs = np.concatenate([x[:, 3:], np.zeros((1, 3, 3))], axis=1)
    assert not np.allclose(P.conv4(xs, w)[0], ref)
    # normalising over the token axis instead of the key channels
    d = _raw()
    out = P.prologue(**d, silu_act=False)
    B, T, H, K = d["q_raw"].shape
    cq = _np_conv(d["q_raw"].reshape(B, T, H * K), d["wq"]).reshape(B, T, H, K)
    wrong = cq / np.linalg.norm(cq, axis=1, keepdims=True)
    assert not np.allclose(out["q"], wrong)
    assert np.allclose(out["q"], cq / np.linalg.norm(cq, axis=-1, keepdims=True), rtol=1e-13)
    # no cap: large g_raw would fall below -5
    assert np.any(-P.softplus(d["g_raw"]) < -5.0) and np.all(out["g"] >= -5.0)


# ---------------------------------------------------------------------------
# The gate outputs of prologue() itself, element by element.
#
# The raw gate inputs are built from targets with closed-form preimages, so that
# the expected outputs are known without evaluating softplus or the sigmoid:
#   softplus(log(e^c - 1)) = c, so g_raw = log(expm1(c)) must give g = -min(c, cap)
#   (Atomic-GDN2 card, section 2.1: g = -min(softplus(g_raw), cap));
#   sigmoid(log(p / (1 - p))) = p, so b_raw = logit(p) must give beta = p.
# The softplus targets c span [0.05, 9] (many above every finite cap used) and
# the sigmoid targets p span [0.02, 0.98], drawn independently, so that swapping
# g_raw and b_raw, ignoring the cap or flipping a sign changes the outputs.
def _gate_case(gate, cap, B=2, T=7, H=3, K=4, V=4, seed=11):
    r = np.random.default_rng(seed)
    gshape = (B, T, H, K) if gate == "channel" else (B, T, H)
    c = r.uniform(0.05, 9.0, gshape)               # softplus targets, some above any cap used
    p = r.uniform(0.02, 0.98, (B, T, H))           # sigmoid targets
    d = _raw(B, T, H, K, V, gate)
    d["g_raw"] = np.log(np.expm1(c))
    d["b_raw"] = np.log(p) - np.log1p(-p)
    want_g = -np.minimum(c, cap)
    return d, want_g, p


def _gate_pins_hold(fn, gate, cap):
    d, want_g, want_b = _gate_case(gate, cap)
    out = fn(**d, silu_act=True, cap=cap)
    return (np.allclose(out["g"], want_g, rtol=1e-12, atol=1e-12)
            and np.allclose(out["beta"], want_b, rtol=1e-12, atol=1e-12))


@pytest.mark.parametrize("cap", [5.0, 2.5, 0.75, math.inf])
@pytest.mark.parametrize("gate", ["head", "channel"])
def test_prologue_gate_outputs_elementwise(gate, cap):
    d, want_g, want_b = _gate_case(gate, cap)
    out = P.prologue(**d, silu_act=True, cap=cap)
    assert out["g"].shape == want_g.shape and out["beta"].shape == want_b.shape
    assert np.allclose(out["g"], want_g, rtol=1e-12, atol=1e-12)
    assert np.allclose(out["beta"], want_b, rtol=1e-12, atol=1e-12)
    # the cap is reached exactly where the target exceeds it
    if math.isfinite(cap):
        hit = want_g == -cap
        assert hit.any() and np.all(out["g"][hit] == -cap)


def test_prologue_gate_pins_catch_planted_mistakes():
    real = P.prologue
    assert _gate_pins_hold(real, "head", 2.5) and _gate_pins_hold(real, "channel", 2.5)

    def swapped(**kw):            # g_raw and b_raw exchanged (same shape under the scalar gate)
        kw["g_raw"], kw["b_raw"] = kw["b_raw"], kw["g_raw"]
        return real(**kw)

    def cap_ignored(**kw):        # the cap argument dropped in favour of the card's 5
        kw["cap"] = 5.0
        return real(**kw)

    def no_cap(**kw):             # no clamp at all
        kw["cap"] = math.inf
        return real(**kw)

    def sign_flipped(**kw):       # g = +min(softplus, cap)
        out = real(**kw)
        out["g"] = -out["g"]
        return out

    def beta_complement(**kw):    # beta = sigmoid(-b_raw)
        kw["b_raw"] = -np.asarray(kw["b_raw"])
        return real(**kw)

    assert not _gate_pins_hold(swapped, "head", 2.5)
    for gate in ("head", "channel"):
        for mutant in (cap_ignored, no_cap, sign_flipped, beta_complement):
            assert not _gate_pins_hold(mutant, gate, 2.5), (mutant.__name__, gate)
