"""Pins of the fp64 backward oracle of the per-channel-decay rule
(``oracle.kda_bwd_ref``, Kimi Delta Attention: column j of the state decays by
exp(gk_t[j]) before token t's prediction; hada.io digest, section "Kimi Delta
Attention : attenuation par canal").

Its equations are derived from the update, so they are pinned against things
that do not share the derivation: central finite differences of the forward
oracle ``kda_ref`` (pinned in ``test_kda_oracle.py``), PyTorch autograd
through a forward loop written here, the reduction to the gated rule when
every channel shares one decay (its backward is pinned separately), the
plain rule at gk = 0, and an erased channel, whose state column carries no
gradient back past the erasing token.  A dgk summed over the wrong axis, a
decay applied to rows instead of columns or a missing factor fails several
of them.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import delta_rule_bwd_ref, kda_bwd_ref, kda_ref


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand(seed, B=1, T=6, H=2, Dk=3, Dv=4, gk_lo=-3.0):
    r = np.random.default_rng(seed)
    x = dict(q=r.standard_normal((B, T, H, Dk)), k=_unit(r.standard_normal((B, T, H, Dk))),
             v=r.standard_normal((B, T, H, Dv)), beta=r.uniform(0.1, 2.0, (B, T, H)),
             gk=r.uniform(gk_lo, 0.0, (B, T, H, Dk)),
             S0=0.5 * r.standard_normal((B, H, Dv, Dk)))
    up = dict(do=r.standard_normal((B, T, H, Dv)), dS_T=r.standard_normal((B, H, Dv, Dk)))
    return x, up


def _loss(x, up):
    o, st = kda_ref(x["q"], x["k"], x["v"], x["beta"], x["gk"], x["S0"])
    return float(np.sum(up["do"] * o) + np.sum(up["dS_T"] * st))


def _bwd(x, up, **kw):
    return kda_bwd_ref(x["q"], x["k"], x["v"], x["beta"], x["gk"], up["do"], x["S0"],
                       up["dS_T"], **kw)


NAMES = {"q": "dq", "k": "dk", "v": "dv", "beta": "dbeta", "gk": "dgk", "S0": "dS0"}


def test_gradients_match_finite_differences():
    x, up = _rand(1)
    grads = _bwd(x, up)
    h = 1e-6
    for name, gname in NAMES.items():
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
    """The per-channel-decay recurrence with plain torch ops (fp64): scale the
    state's key columns, predict, correct, write, read."""
    q, k, v, beta, gk, S = x["q"], x["k"], x["v"], x["beta"], x["gk"], x["S0"]
    outs = []
    for t in range(q.shape[1]):
        S = S * torch.exp(gk[:, t])[:, :, None, :]
        pred = (S * k[:, t][:, :, None, :]).sum(-1)
        err = beta[:, t][..., None] * (v[:, t] - pred)
        S = S + err[..., :, None] * k[:, t][..., None, :]
        outs.append((S * q[:, t][:, :, None, :]).sum(-1))
    return torch.stack(outs, dim=1), S


@pytest.mark.parametrize("gk_lo", [-3.0, -16.0])
def test_gradients_match_autograd(gk_lo):
    x, up = _rand(2, B=2, T=40, H=2, Dk=8, Dv=6, gk_lo=gk_lo)
    grads = _bwd(x, up, nthreads=3)
    tx = {n: torch.tensor(a, requires_grad=True) for n, a in x.items()}
    o, st = _torch_forward(tx)
    L = (o * torch.tensor(up["do"])).sum() + (st * torch.tensor(up["dS_T"])).sum()
    L.backward()
    for name, gname in NAMES.items():
        ref = tx[name].grad.numpy()
        err = np.max(np.abs(ref - grads[gname])) / np.max(np.abs(ref))
        assert err < 1e-12, f"{gname}: relative error {err:.2e} against autograd"


# One decay shared by every channel is the gated rule: the same dq, dk, dv,
# dbeta, dS0 bit for bit, and dg_t = sum_j dgk_t[j].
def test_shared_decay_is_the_gated_backward():
    x, up = _rand(3, B=2, T=11, Dk=5)
    g = x["gk"][..., 0].copy()
    x["gk"] = np.repeat(g[..., None], 5, axis=-1)
    kda = _bwd(x, up)
    gated = delta_rule_bwd_ref(x["q"], x["k"], x["v"], x["beta"], up["do"], x["S0"],
                               up["dS_T"], g=g)
    for n in ("dq", "dk", "dv", "dbeta", "dS0"):
        assert np.array_equal(kda[n], gated[n]), n
    dg = kda["dgk"].sum(-1)
    assert np.max(np.abs(dg - gated["dg"])) <= 1e-12 * max(1.0, np.max(np.abs(gated["dg"])))


def test_zero_decay_is_the_plain_backward():
    x, up = _rand(4, B=2, T=9)
    x["gk"] = np.zeros_like(x["gk"])
    kda = _bwd(x, up)
    plain = delta_rule_bwd_ref(x["q"], x["k"], x["v"], x["beta"], up["do"], x["S0"],
                               up["dS_T"])
    for n in ("dq", "dk", "dv", "dbeta", "dS0"):
        assert np.array_equal(kda[n], plain[n]), n


# Erasing key channel j at token e (gk = -1e4, exp underflows to 0) clears
# column j of the state there: S0's column j reaches nothing from token e on,
# so dS0[..., j] only holds what tokens before e saw.  Erasing it at token 0
# leaves it no gradient at all; every gradient stays finite.
def test_erased_channel_blocks_the_state_gradient():
    x, up = _rand(5, B=1, T=8, Dk=4)
    x["gk"][:, 0, :, 2] = -1e4
    g = _bwd(x, up)
    assert np.array_equal(g["dS0"][..., 2], np.zeros_like(g["dS0"][..., 2]))
    assert np.all(np.isfinite(g["dgk"]))
    # dgk at the erasing token: <dP, P> over column 2 with P's column 2 = 0
    assert np.array_equal(g["dgk"][:, 0, :, 2], np.zeros_like(g["dgk"][:, 0, :, 2]))
    # erased at token 3 instead: the first three tokens' reads still reach S0
    x2, _ = _rand(5, B=1, T=8, Dk=4)
    x2["gk"][:, 3, :, 2] = -1e4
    g2 = _bwd(x2, up)
    assert np.any(g2["dS0"][..., 2] != 0)
    # the tokens from 3 on, run alone from the state after token 2, give that
    # incoming state's column 2 no gradient
    x3 = {n: (a if n == "S0" else a[:, :3]) for n, a in x2.items()}
    _, s_mid = kda_ref(x3["q"], x3["k"], x3["v"], x3["beta"], x3["gk"], x3["S0"])
    x4 = {n: (s_mid if n == "S0" else a[:, 3:]) for n, a in x2.items()}
    g4 = kda_bwd_ref(x4["q"], x4["k"], x4["v"], x4["beta"], x4["gk"], up["do"][:, 3:],
                     x4["S0"], up["dS_T"])
    assert np.array_equal(g4["dS0"][..., 2], np.zeros_like(g4["dS0"][..., 2]))


def test_gradients_are_linear_in_the_upstream_gradients():
    x, up1 = _rand(6, T=8)
    _, up2 = _rand(7, T=8)
    mix = {n: 2.0 * up1[n] - 0.5 * up2[n] for n in up1}
    g1, g2, gm = _bwd(x, up1), _bwd(x, up2), _bwd(x, mix)
    for n in g1:
        assert np.max(np.abs(gm[n] - (2.0 * g1[n] - 0.5 * g2[n]))) < 1e-12 * max(
            1.0, np.max(np.abs(gm[n]))), n


def test_thread_count_does_not_change_the_result():
    x, up = _rand(8, B=3, T=10, H=3)
    a, b = _bwd(x, up, nthreads=1), _bwd(x, up, nthreads=4)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


def test_empty_sequence_passes_the_state_gradient_through():
    x, up = _rand(9, T=0)
    g = _bwd(x, up)
    assert np.array_equal(g["dS0"], up["dS_T"])
    assert g["dgk"].shape == (1, 0, 2, 3)
