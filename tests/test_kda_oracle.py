"""Pins of the fp64 KDA oracle (per-key-channel decay, ``oracle.kda_ref``).

hada.io digest, section "Kimi Delta Attention : attenuation par canal": the
scalar gate of Gated DeltaNet becomes a vector over the key channels, which
are the columns of the state; the order is decay, predict, correct, write,
read.  The tests check the reductions to the gated and plain rules, closed
forms (pure decay, one token, keys along coordinate axes), the resume
property and the pages' chunkwise form ("Chunkwise KDA").  Decaying rows
instead of columns, predicting before the decay, or an exponent off by one
token each fail at least one of them.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import chunk_algebra as CA
from oracle import delta_rule_ref, gated_delta_rule_ref, kda_ref


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand(seed, B=2, T=20, H=2, Dk=5, Dv=4, beta_hi=1.0, lo=0.4):
    r = np.random.default_rng(seed)
    q = _unit(r.standard_normal((B, T, H, Dk)))
    k = _unit(r.standard_normal((B, T, H, Dk)))
    v = r.standard_normal((B, T, H, Dv))
    beta = r.uniform(0.0, beta_hi, (B, T, H))
    gk = np.log(r.uniform(lo, 1.0, (B, T, H, Dk)))
    S0 = 0.3 * r.standard_normal((B, H, Dv, Dk))
    return q, k, v, beta, gk, S0


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# A decay that is the same on every channel is the gated rule's scalar gate
# (bit for bit: the same factor multiplies every element); zero is the plain
# rule.
def test_equal_channels_is_the_gated_rule_and_zero_is_the_plain_rule():
    q, k, v, beta, gk, S0 = _rand(1)
    g = gk[..., 0]
    o1, s1 = kda_ref(q, k, v, beta, np.repeat(g[..., None], 5, axis=-1), S0)
    o2, s2 = gated_delta_rule_ref(q, k, v, beta, g, S0)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
    o3, s3 = kda_ref(q, k, v, beta, np.zeros_like(gk), S0)
    o4, s4 = delta_rule_ref(q, k, v, beta, S0)
    assert np.array_equal(o3, o4) and np.array_equal(s3, s4)


# beta = 0 is a pure per-channel decay of the columns:
# S_T = S0 Diag(exp(sum_t gk_t)), o_t = S0 Diag(exp(sum_{s<=t} gk_s)) q_t.
def test_zero_beta_decays_each_column():
    q, k, v, beta, gk, S0 = _rand(2)
    o, st = kda_ref(q, k, v, np.zeros_like(beta), gk, S0)
    cum = np.cumsum(gk, axis=1)                                 # [B,T,H,Dk]
    o_ref = np.einsum("bhij,bthj->bthi", S0, np.exp(cum) * q)
    s_ref = S0 * np.exp(cum[:, -1])[:, :, None, :]
    assert _rel(o, o_ref) < 1e-14 and _rel(st, s_ref) < 1e-14


# One token written out: S1 = S0 D + beta (v - S0 D k) k^T, o = S1 q.
def test_one_token_by_hand():
    r = np.random.default_rng(3)
    Dk, Dv = 6, 4
    q, k = _unit(r.standard_normal((2, Dk)))
    v = r.standard_normal(Dv)
    S0 = r.standard_normal((Dv, Dk))
    gk = np.log(r.uniform(0.2, 1.0, Dk))
    b = 0.7
    o, st = kda_ref(q[None, None, None], k[None, None, None], v[None, None, None],
                    np.array([[[b]]]), gk[None, None, None], S0[None, None])
    P = S0 @ np.diag(np.exp(gk))
    S1 = P + b * np.outer(v - P @ k, k)
    assert _rel(st[0, 0], S1) < 1e-15 and _rel(o[0, 0, 0], S1 @ q) < 1e-15
    rows = S0 * np.exp(gk[:Dv])[:, None]   # decaying rows instead of columns differs
    assert _rel(rows + b * np.outer(v - rows @ k, k), S1) > 1e-2


# Keys along coordinate axes, beta = 1, S0 = 0: token i writes v_i into
# column j_i; later tokens only decay it with their channel-j_i factor, as
# long as no later key shares the axis.
def test_axis_keys_keep_their_column_decay():
    r = np.random.default_rng(4)
    T, Dk, Dv = 5, 5, 3
    K = np.eye(Dk)[:T]
    v = r.standard_normal((T, Dv))
    q = _unit(r.standard_normal((T, Dk)))
    gk = np.log(r.uniform(0.3, 1.0, (T, Dk)))
    _, st = kda_ref(q[None, :, None], K[None, :, None], v[None, :, None], np.ones((1, T, 1)),
                    gk[None, :, None])
    S = st[0, 0]
    for i in range(T):
        keep = np.exp(np.sum(gk[i + 1:, i]))
        assert np.max(np.abs(S[:, i] - keep * v[i])) < 1e-14


def test_resume_at_any_cut_is_bit_identical():
    q, k, v, beta, gk, S0 = _rand(5, T=17)
    o, st = kda_ref(q, k, v, beta, gk, S0)
    for cut in (1, 9, 16):
        o1, s1 = kda_ref(q[:, :cut], k[:, :cut], v[:, :cut], beta[:, :cut], gk[:, :cut], S0)
        o2, s2 = kda_ref(q[:, cut:], k[:, cut:], v[:, cut:], beta[:, cut:], gk[:, cut:], s1)
        assert np.array_equal(np.concatenate([o1, o2], axis=1), o) and np.array_equal(s2, st)


# The pages' chunked form (cumulative per-channel decays, couplings through
# D_{j+1:i}, the triangular solve, S D_{0:C-1} + E^T K_end) equals the
# recurrence for every chunk size, with ragged tails and beta up to 2.
@pytest.mark.parametrize("chunk", [1, 3, 16, 64, 100])
def test_kda_chunk_form_equals_recurrence(chunk):
    q, k, v, beta, gk, S0 = _rand(6, B=1, T=100, H=2, Dk=6, Dv=5, beta_hi=2.0, lo=0.5)
    o, st = kda_ref(q, k, v, beta, gk, S0)
    o2, st2 = CA.kda_chunk_forward(q, k, v, beta, gk, S0, chunk)
    assert _rel(o2, o) < 1e-12 and _rel(st2, st) < 1e-12


# With a decay equal on every channel the KDA chunk step is the gated one.
def test_kda_chunk_step_reduces_to_gated():
    q, k, v, beta, gk, S0 = _rand(7, B=1, T=16, H=1, Dk=6, Dv=4)
    g = gk[0, :, 0, 0]
    a = CA.gated_chunk_step(S0[0, 0], q[0, :, 0], k[0, :, 0], v[0, :, 0], beta[0, :, 0], g)
    b = CA.kda_chunk_step(S0[0, 0], q[0, :, 0], k[0, :, 0], v[0, :, 0], beta[0, :, 0],
                          np.repeat(g[:, None], 6, axis=1))
    for x, y in zip(a, b):
        assert _rel(y, x) < 1e-13
