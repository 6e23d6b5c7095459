"""Pins of the fp64 backward oracle (``oracle.backward``) against what the
mathematics fixes, independently of the oracle's own code:

* central finite differences of the matrix form printed on the Atomic-GDN2 card
  (section 2.1), S_t = (I - beta k k^T) Diag(alpha) S + beta k v^T, o_t = S_t^T q_t,
  for every input element of tiny problems;
* torch autograd in float64 through that same printed matrix form, at sizes with
  several slices;
* closed forms of the decay-only case (beta = 0);
* splitting a sequence in two and chaining dL/dS through the cut;
* planted mistakes in a copy of the reverse sweep, each caught by the pins.
"""
import numpy as np
import pytest
import torch

from oracle.backward import backward
from tests.test_oracle import _dense_reference


def _inputs(B, T, H, K, V, gate, rng, s0=True):
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, V))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    gs = (B, T, H, K) if gate == "channel" else (B, T, H)
    g = -np.log1p(np.exp(rng.standard_normal(gs)))
    S0 = 0.5 * rng.standard_normal((B, H, K, V)) if s0 else None
    do = rng.standard_normal((B, T, H, V))
    dS_T = rng.standard_normal((B, H, K, V))
    return dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0), do, dS_T


def _loss_dense(d, do, dS_T):
    """L = sum(o * do) + sum(S_T * dS_T) through the printed matrix form."""
    B, T, H, K = d["q"].shape
    tot = 0.0
    for b in range(B):
        for h in range(H):
            S0 = None if d["S0"] is None else d["S0"][b, h]
            o, S = _dense_reference(d["q"][b, :, h], d["k"][b, :, h], d["v"][b, :, h],
                                    d["g"][b, :, h], d["beta"][b, :, h], S0)
            tot += float(np.sum(o * do[b, :, h]) + np.sum(S * dS_T[b, h]))
    return tot


def _rel(x, ref):
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300))


def _fd(d, do, dS_T, name, h=1e-6):
    x = d[name]
    out = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        keep = x[idx]
        x[idx] = keep + h
        lp = _loss_dense(d, do, dS_T)
        x[idx] = keep - h
        lm = _loss_dense(d, do, dS_T)
        x[idx] = keep
        out[idx] = (lp - lm) / (2 * h)
    return out


# --- pin 1: finite differences of the printed matrix form ------------------------
@pytest.mark.parametrize("gate", ["head", "channel"])
def test_matches_finite_differences(gate):
    rng = np.random.default_rng(7)
    d, do, dS_T = _inputs(1, 6, 2, 4, 3, gate, rng)
    gr = backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], do, dS_T)
    for name, gname in [("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"),
                        ("beta", "dbeta"), ("S0", "dS0")]:
        ref = _fd(d, do, dS_T, name)
        assert gr[gname].shape == ref.shape, name
        assert _rel(gr[gname], ref) < 1e-7, (name, _rel(gr[gname], ref))


# --- pin 2: torch autograd through the printed matrix form -----------------------
def _torch_dense_loss(t, do, dS_T, channel):
    B, T, H, K = t["q"].shape
    eye = torch.eye(K, dtype=torch.float64)
    L = 0.0
    for b in range(B):
        for h in range(H):
            S = t["S0"][b, h]
            for s in range(T):
                kt = t["k"][b, s, h][:, None]
                a = torch.exp(t["g"][b, s, h]) if channel else torch.exp(t["g"][b, s, h]) * torch.ones(K, dtype=torch.float64)
                bt = t["beta"][b, s, h]
                S = (eye - bt * (kt @ kt.T)) @ torch.diag(a) @ S + bt * kt @ t["v"][b, s, h][None, :]
                L = L + (S.T @ t["q"][b, s, h] * do[b, s, h]).sum()
            L = L + (S * dS_T[b, h]).sum()
    return L


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_matches_autograd_of_the_matrix_form(gate):
    rng = np.random.default_rng(11)
    d, do, dS_T = _inputs(2, 19, 2, 6, 5, gate, rng)
    t = {n: torch.tensor(x, dtype=torch.float64, requires_grad=True) for n, x in d.items()}
    L = _torch_dense_loss(t, torch.tensor(do), torch.tensor(dS_T), gate == "channel")
    L.backward()
    gr = backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], do, dS_T)
    for name in ("q", "k", "v", "g", "beta", "S0"):
        assert _rel(gr["d" + name], t[name].grad.numpy()) < 1e-11, name


# --- pin 3: decay only (beta = 0) has closed forms --------------------------------
def test_decay_only_closed_forms():
    """beta = 0: S_t = D_t S0 with D_t = Diag(exp(sum_{s<=t} g_s)), so
    dS0 = sum_t D_t q_t do_t^T + D_T dS_T, dq_t = D_t S0 do_t, dv = dk = 0."""
    rng = np.random.default_rng(3)
    d, do, dS_T = _inputs(1, 9, 1, 5, 4, "channel", rng)
    d["beta"][:] = 0.0
    gr = backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], do, dS_T)
    S0 = d["S0"][0, 0]
    gam = np.cumsum(d["g"][0, :, 0], axis=0)                  # [T, K]
    dS0 = np.exp(gam[-1])[:, None] * dS_T[0, 0]
    for t in range(9):
        D = np.exp(gam[t])
        dS0 += D[:, None] * np.outer(d["q"][0, t, 0], do[0, t, 0])
        assert np.allclose(gr["dq"][0, t, 0], D * (S0 @ do[0, t, 0]), rtol=1e-13, atol=1e-14)
    assert np.allclose(gr["dS0"][0, 0], dS0, rtol=1e-13, atol=1e-14)
    assert np.all(gr["dv"] == 0) and np.all(gr["dk"] == 0)


# --- pin 4: a cut in the sequence, dL/dS chained through it ----------------------
@pytest.mark.parametrize("gate", ["head", "channel"])
def test_split_sequence_chains_the_state_gradient(gate):
    rng = np.random.default_rng(5)
    d, do, dS_T = _inputs(1, 23, 2, 8, 6, gate, rng)
    full = backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], do, dS_T)
    c = 10
    head = {n: x[:, :c] for n, x in d.items() if n != "S0"}
    tail = {n: x[:, c:] for n, x in d.items() if n != "S0"}
    # state at the cut, from the printed form
    S_mid = np.stack([np.stack([_dense_reference(d["q"][0, :c, h], d["k"][0, :c, h], d["v"][0, :c, h],
                                                 d["g"][0, :c, h], d["beta"][0, :c, h], d["S0"][0, h])[1]
                                for h in range(2)])])
    gt = backward(tail["q"], tail["k"], tail["v"], tail["g"], tail["beta"], S_mid, do[:, c:], dS_T)
    gh = backward(head["q"], head["k"], head["v"], head["g"], head["beta"], d["S0"], do[:, :c], gt["dS0"])
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        assert np.allclose(np.concatenate([gh[n], gt[n]], axis=1), full[n], rtol=1e-12, atol=1e-13), n
    assert np.allclose(gh["dS0"], full["dS0"], rtol=1e-12, atol=1e-13)


def test_no_initial_state_and_no_state_gradient_mean_zeros():
    rng = np.random.default_rng(9)
    d, do, _ = _inputs(1, 7, 1, 4, 4, "head", rng, s0=False)
    a = backward(d["q"], d["k"], d["v"], d["g"], d["beta"], None, do, None)
    z = np.zeros((1, 1, 4, 4))
    b = backward(d["q"], d["k"], d["v"], d["g"], d["beta"], z, do, z)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


# --- the pins catch planted mistakes ---------------------------------------------
def _mutant_backward(q, k, v, g, beta, S0, do, dS_T, bug):
    """One slice (q,k [T,K] ...), the reverse sweep with one plausible mistake."""
    T, K = q.shape
    a_all = np.exp(g) if g.ndim == 2 else np.exp(g)[:, None] * np.ones(K)
    S = S0.copy()
    before = []
    for t in range(T):
        before.append(S)
        Sd = a_all[t][:, None] * S
        d = beta[t] * (v[t] - Sd.T @ k[t])
        S = Sd + np.outer(k[t], d)
    G = dS_T.copy()
    out = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dbeta", beta))}
    out["dg"] = np.zeros((T, K))
    for t in range(T - 1, -1, -1):
        at = a_all[t]
        Sd = at[:, None] * before[t]
        u = Sd.T @ k[t]
        d = beta[t] * (v[t] - u)
        St = Sd + np.outer(k[t], d)
        out["dq"][t] = (Sd if bug == "read_before_write" else St) @ do[t]
        if bug != "drop_readout_into_state":
            G = G + np.outer(q[t], do[t])
        out["dk"][t] = G @ d
        dd = G.T @ k[t]
        out["dv"][t] = beta[t] * dd
        out["dbeta"][t] = (v[t] - u) @ dd
        du = (beta[t] if bug == "sign_du" else -beta[t]) * dd
        if bug != "drop_dk_error_path":
            out["dk"][t] += Sd @ du
        dSd = G + np.outer(k[t], du)
        out["dg"][t] = at * np.sum(before[t] * dSd, axis=1)
        # the decay scales the key rows; the planted mistake scales value columns (K == V here)
        G = dSd * at[None, :] if bug == "decay_on_values" else at[:, None] * dSd
    out["dS0"] = G
    return out


@pytest.mark.parametrize("bug", ["read_before_write", "drop_readout_into_state", "sign_du",
                                 "drop_dk_error_path", "decay_on_values"])
def test_planted_mistakes_are_caught(bug):
    rng = np.random.default_rng(13)
    d, do, dS_T = _inputs(1, 6, 1, 4, 4, "channel", rng)
    sl = {n: (x[0, :, 0] if n != "S0" else x[0, 0]) for n, x in d.items()}
    m = _mutant_backward(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], sl["S0"],
                         do[0, :, 0], dS_T[0, 0], bug)
    worst = 0.0
    for name, gname in [("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"),
                        ("beta", "dbeta"), ("S0", "dS0")]:
        ref = _fd(d, do, dS_T, name)
        got = m[gname][None, :, None] if name != "S0" else m[gname][None, None]
        worst = max(worst, _rel(got.reshape(ref.shape), ref))
    assert worst > 1e-3, bug
    # and the clean sweep passes the same check
    clean = _mutant_backward(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], sl["S0"],
                             do[0, :, 0], dS_T[0, 0], None)
    assert _rel(clean["dk"], _fd(d, do, dS_T, "k")[0, :, 0]) < 1e-7
