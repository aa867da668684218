"""Pins of the fp64 backward oracle (``oracle.delta_rule_bwd_ref``).

The backward equations are derived from the update (the pages give only the
strategy of recomputing states), so they are pinned against things that do
not share that derivation: central finite differences of the forward oracle,
PyTorch autograd through a forward loop written here independently, closed
forms for beta = 0, and structural facts (linearity in the upstream
gradients, the gated rule with g = 0, cutting the sequence).  A dropped
term of dk, a wrong sign or a missing decay factor fails several of them.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import delta_rule_bwd_ref, delta_rule_ref, gated_delta_rule_ref


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand(seed, B=1, T=6, H=2, Dk=3, Dv=4, gated=False, beta_hi=2.0):
    r = np.random.default_rng(seed)
    x = dict(q=r.standard_normal((B, T, H, Dk)), k=_unit(r.standard_normal((B, T, H, Dk))),
             v=r.standard_normal((B, T, H, Dv)), beta=r.uniform(0.1, beta_hi, (B, T, H)),
             S0=0.5 * r.standard_normal((B, H, Dv, Dk)))
    x["g"] = np.log(r.uniform(0.3, 1.0, (B, T, H))) if gated else None
    up = dict(do=r.standard_normal((B, T, H, Dv)), dS_T=r.standard_normal((B, H, Dv, Dk)))
    return x, up


def _loss(x, up):
    if x["g"] is None:
        o, st = delta_rule_ref(x["q"], x["k"], x["v"], x["beta"], x["S0"])
    else:
        o, st = gated_delta_rule_ref(x["q"], x["k"], x["v"], x["beta"], x["g"], x["S0"])
    return float(np.sum(up["do"] * o) + np.sum(up["dS_T"] * st))


def _bwd(x, up, **kw):
    return delta_rule_bwd_ref(x["q"], x["k"], x["v"], x["beta"], up["do"], x["S0"], up["dS_T"],
                              g=x["g"], **kw)


NAMES = {"q": "dq", "k": "dk", "v": "dv", "beta": "dbeta", "S0": "dS0", "g": "dg"}


# Central differences of L = <do, o> + <dS_T, S_T> through the forward oracle
# (its own pins fix the forward): every entry of every gradient.
@pytest.mark.parametrize("gated", [False, True])
def test_gradients_match_finite_differences(gated):
    x, up = _rand(1, gated=gated)
    grads = _bwd(x, up)
    h = 1e-6
    for name, gname in NAMES.items():
        if x.get(name) is None:
            continue
        base = x[name]
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            xp = dict(x)
            xp[name] = base.copy()
            xp[name][idx] += h
            lp = _loss(xp, up)
            xp[name][idx] -= 2 * h
            lm = _loss(xp, up)
            num[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(num - grads[gname])) / max(np.max(np.abs(num)), 1e-12)
        assert err < 1e-7, f"{gname}: relative error {err:.2e} against finite differences"


def _torch_forward(x):
    """The recurrence written with plain torch ops (fp64), for autograd."""
    q, k, v, beta, S = x["q"], x["k"], x["v"], x["beta"], x["S0"]
    B, T, H, _ = q.shape
    outs = []
    for t in range(T):
        if x.get("g") is not None:
            S = torch.exp(x["g"][:, t])[..., None, None] * S
        pred = torch.einsum("bhij,bhj->bhi", S, k[:, t])
        err = beta[:, t][..., None] * (v[:, t] - pred)
        S = S + err[..., :, None] * k[:, t][..., None, :]
        outs.append(torch.einsum("bhij,bhj->bhi", S, q[:, t]))
    return torch.stack(outs, dim=1), S


# PyTorch autograd through an independently written forward loop, at a size
# where every chunk-free path of the recurrence is exercised.
@pytest.mark.parametrize("gated", [False, True])
def test_gradients_match_autograd(gated):
    x, up = _rand(2, B=2, T=40, H=2, Dk=8, Dv=6, gated=gated)
    grads = _bwd(x, up)
    tx = {n: (None if a is None else torch.tensor(a, requires_grad=True)) for n, a in x.items()}
    o, st = _torch_forward(tx)
    L = (o * torch.tensor(up["do"])).sum() + (st * torch.tensor(up["dS_T"])).sum()
    L.backward()
    for name, gname in NAMES.items():
        if tx.get(name) is None:
            continue
        ref = tx[name].grad.numpy()
        err = np.max(np.abs(ref - grads[gname])) / np.max(np.abs(ref))
        assert err < 1e-12, f"{gname}: relative error {err:.2e} against autograd"


# beta = 0 leaves the state at S0 (decayed by the gates): o_t = S0 q_t, so
# dq_t = S0^T do_t, dS0 = dS_T + sum_t do_t q_t^T, and v, k get no gradient.
def test_beta_zero_closed_form():
    x, up = _rand(3, T=7)
    x["beta"] = np.zeros_like(x["beta"])
    gr = _bwd(x, up)
    S0 = x["S0"]
    assert np.array_equal(gr["dv"], np.zeros_like(gr["dv"]))
    assert np.array_equal(gr["dk"], np.zeros_like(gr["dk"]))
    dq = np.einsum("bhij,bthi->bthj", S0, up["do"])
    assert np.max(np.abs(gr["dq"] - dq)) < 1e-13
    dS0 = up["dS_T"] + np.einsum("bthi,bthj->bhij", up["do"], x["q"])
    assert np.max(np.abs(gr["dS0"] - dS0)) < 1e-13
    # dbeta_t = u_t . (D_t k_t) with u_t = v_t - S0 k_t and D_t = dS_T + sum_{s>=t} do_s q_s^T
    u = x["v"] - np.einsum("bhij,bthj->bthi", S0, x["k"])
    rev = np.cumsum(np.einsum("bthi,bthj->bthij", up["do"], x["q"])[:, ::-1], axis=1)[:, ::-1]
    D = rev + up["dS_T"][:, None]
    db = np.einsum("bthi,bthij,bthj->bth", u, D, x["k"])
    assert np.max(np.abs(gr["dbeta"] - db)) < 1e-12


def test_gated_with_zero_gate_is_the_plain_backward():
    x, up = _rand(4, B=2, T=9)
    plain = _bwd(x, up)
    x["g"] = np.zeros_like(x["beta"])
    gated = _bwd(x, up)
    for n in ("dq", "dk", "dv", "dbeta", "dS0"):
        assert np.array_equal(plain[n], gated[n]), n


def test_gradients_are_linear_in_the_upstream_gradients():
    x, up1 = _rand(5, T=8, gated=True)
    _, up2 = _rand(6, T=8, gated=True)
    mix = {n: 2.0 * up1[n] - 0.5 * up2[n] for n in up1}
    g1, g2, gm = _bwd(x, up1), _bwd(x, up2), _bwd(x, mix)
    for n in g1:
        assert np.max(np.abs(gm[n] - (2.0 * g1[n] - 0.5 * g2[n]))) < 1e-12 * max(
            1.0, np.max(np.abs(gm[n]))), n


# Cutting the sequence: the second half's dS0 is the first half's dS_T, and
# the gradients of both halves together are those of the whole, bit for bit.
@pytest.mark.parametrize("gated", [False, True])
def test_cut_sequence_backward_is_bit_identical(gated):
    x, up = _rand(7, B=1, T=12, gated=gated)
    whole = _bwd(x, up)
    cut = 5
    sl = lambda d, a, b: {n: (None if v is None else (v if n in ("S0", "dS_T") else v[:, a:b]))
                          for n, v in d.items()}
    x1 = sl(x, 0, cut)
    if gated:
        _, s_mid = gated_delta_rule_ref(x1["q"], x1["k"], x1["v"], x1["beta"], x1["g"], x["S0"])
    else:
        _, s_mid = delta_rule_ref(x1["q"], x1["k"], x1["v"], x1["beta"], x["S0"])
    x2 = sl(x, cut, 12)
    x2["S0"] = s_mid
    g2 = _bwd(x2, sl(up, cut, 12))
    up1 = sl(up, 0, cut)
    up1["dS_T"] = g2["dS0"]
    g1 = _bwd(x1, up1)
    for n in ("dq", "dk", "dv", "dbeta") + (("dg",) if gated else ()):
        assert np.array_equal(np.concatenate([g1[n], g2[n]], axis=1), whole[n]), n
    assert np.array_equal(g1["dS0"], whole["dS0"])


def test_empty_sequence_passes_the_state_gradient_through():
    x, up = _rand(8, T=0)
    g = _bwd(x, up)
    assert np.array_equal(g["dS0"], up["dS_T"])
    gz = delta_rule_bwd_ref(x["q"], x["k"], x["v"], x["beta"], up["do"], x["S0"], None)
    assert np.array_equal(gz["dS0"], np.zeros_like(up["dS_T"]))
