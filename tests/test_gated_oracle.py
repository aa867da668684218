"""Pins of the gated fp64 oracle (scalar forget gate alpha_t = exp(g_t)).

Each test names the passage it rests on.  They check the gated recurrence
against the ungated oracle, closed forms (pure decay, one token, orthonormal
keys), the order the pages insist on (forget, then predict), a gate of zero
as a reset, an invariant (no growth for a contraction), the resume property
and the pages' chunkwise form with cumulative decay.  A prediction taken
before the decay, a decay applied after the write, a missing or doubled
decay, or a decay exponent off by one token each fails at least one of them.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import chunk_algebra as CA
from oracle import delta_rule_ref, gated_delta_rule_ref


def _unit(x, axis=-1):
    return x / np.linalg.norm(x, axis=axis, keepdims=True)


def _rand(seed, B=2, T=24, H=3, Dk=5, Dv=4, beta_hi=1.0, s0=True, alpha_lo=0.5):
    r = np.random.default_rng(seed)
    q = _unit(r.standard_normal((B, T, H, Dk)))
    k = _unit(r.standard_normal((B, T, H, Dk)))
    v = r.standard_normal((B, T, H, Dv))
    beta = r.uniform(0.0, beta_hi, (B, T, H))
    g = np.log(r.uniform(alpha_lo, 1.0, (B, T, H)))
    S0 = r.standard_normal((B, H, Dv, Dk)) * 0.3 if s0 else None
    return q, k, v, beta, g, S0


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# houmin.site "infra/delta-net", section "Gated DeltaNet": with alpha_t = 1 the
# gated update is the DeltaNet update.  exp(0) = 1 exactly, so bit for bit.
def test_gate_of_one_is_the_ungated_rule():
    q, k, v, beta, g, S0 = _rand(1)
    o0, s0 = delta_rule_ref(q, k, v, beta, S0)
    o1, s1 = gated_delta_rule_ref(q, k, v, beta, np.zeros_like(g), S0)
    assert np.array_equal(o0, o1) and np.array_equal(s0, s1)


# houmin.site, section "Gated DeltaNet": with beta = 0 the update is the
# Mamba2-style pure decay S_t = alpha_t S_{t-1}, so S_t = exp(sum g) S0 and
# o_t = exp(sum_{s<=t} g_s) S0 q_t.
def test_zero_beta_is_pure_decay():
    q, k, v, beta, g, S0 = _rand(2)
    o, st = gated_delta_rule_ref(q, k, v, np.zeros_like(beta), g, S0)
    cum = np.cumsum(g, axis=1)  # [B,T,H]
    o_ref = np.exp(cum)[..., None] * np.einsum("bhij,bthj->bthi", S0, q)
    s_ref = np.exp(cum[:, -1])[..., None, None] * S0
    assert _rel(o, o_ref) < 1e-14 and _rel(st, s_ref) < 1e-14


# hada.io digest, section "Gated DeltaNet : oublier d'abord l'etat entier":
# forget, predict from the decayed state, correct, write -- in that order.
# One token, written out: S_1 = a S0 + b (v - a S0 k) k^T, o = S_1 q.  The
# other order (predict from S0, then decay) gives a different state here.
def test_one_token_forgets_before_predicting():
    r = np.random.default_rng(3)
    Dk, Dv = 6, 5
    q, k = _unit(r.standard_normal((2, Dk)))
    v = r.standard_normal(Dv)
    S0 = r.standard_normal((Dv, Dk))
    a, b = 0.6, 0.8
    o, st = gated_delta_rule_ref(q[None, None, None], k[None, None, None], v[None, None, None],
                                 np.array([[[b]]]), np.array([[[np.log(a)]]]), S0[None, None])
    S1 = a * S0 + b * np.outer(v - a * S0 @ k, k)
    assert _rel(st[0, 0], S1) < 1e-15 and _rel(o[0, 0, 0], S1 @ q) < 1e-15
    wrong = a * (S0 + b * np.outer(v - S0 @ k, k))  # predict before the decay
    assert _rel(wrong, S1) > 1e-2


# hada.io digest, sections "Gated DeltaNet" (locality of the delta write) and
# "Transition d'etat structuree": with orthonormal keys, beta = 1 and S0 = 0,
# token i stores v_i k_i^T and every later token only decays it (its write is
# orthogonal), so S_T k_i = (prod_{s>i} alpha_s) v_i.
def test_orthonormal_keys_recall_with_decay():
    r = np.random.default_rng(4)
    T, Dk, Dv = 7, 7, 4
    K = np.linalg.qr(r.standard_normal((Dk, Dk)))[0][:T]
    v = r.standard_normal((T, Dv))
    q = _unit(r.standard_normal((T, Dk)))
    g = np.log(r.uniform(0.3, 1.0, T))
    _, st = gated_delta_rule_ref(q[None, :, None], K[None, :, None], v[None, :, None],
                                 np.ones((1, T, 1)), g[None, :, None])
    S = st[0, 0]
    for i in range(T):
        keep = np.exp(np.sum(g[i + 1:]))
        assert np.max(np.abs(S @ K[i] - keep * v[i])) < 1e-13


# A gate of zero empties the state before the token's write, so everything
# after it is a fresh run from that token with S0 = 0 (the "global forgetting"
# the houmin.site section attributes to alpha).
def test_zero_gate_resets_the_state():
    q, k, v, beta, g, S0 = _rand(5, T=20)
    t0 = 9
    g[:, t0] = -1.0e4  # exp underflows to exactly 0.0
    o, st = gated_delta_rule_ref(q, k, v, beta, g, S0)
    o2, st2 = gated_delta_rule_ref(q[:, t0:], k[:, t0:], v[:, t0:], beta[:, t0:],
                                   np.where(np.arange(20 - t0)[None, :, None] == 0, 0.0,
                                            g[:, t0:]))
    assert _rel(o[:, t0:], o2) < 1e-14 and _rel(st, st2) < 1e-14


# hada.io digest, "Transition d'etat structuree": with unit keys the factor
# (I - beta k k^T) has eigenvalues 1 - beta and 1, so for beta in [0, 2] and
# alpha <= 1 the free evolution (v = 0) never grows the state.
def test_free_evolution_never_grows_the_state():
    q, k, v, beta, g, S0 = _rand(6, T=40, beta_hi=2.0)
    norms = [np.linalg.norm(S0, axis=(2, 3))]
    for t in range(1, 41):
        _, st = gated_delta_rule_ref(q[:, :t], k[:, :t], 0 * v[:, :t], beta[:, :t], g[:, :t], S0)
        norms.append(np.linalg.norm(st, axis=(2, 3)))
    norms = np.stack(norms)
    assert np.all(np.diff(norms, axis=0) <= 1e-12 * norms[:-1])


# fla DeltaNet layer (initial_state / final state): a run cut in two, the
# second half started from the first half's final state, is the same run.
def test_resume_at_any_cut_is_bit_identical():
    q, k, v, beta, g, S0 = _rand(7, T=23)
    o, st = gated_delta_rule_ref(q, k, v, beta, g, S0)
    for cut in (1, 8, 16, 22):
        o1, s1 = gated_delta_rule_ref(q[:, :cut], k[:, :cut], v[:, :cut], beta[:, :cut],
                                      g[:, :cut], S0)
        o2, s2 = gated_delta_rule_ref(q[:, cut:], k[:, cut:], v[:, cut:], beta[:, cut:],
                                      g[:, cut:], s1)
        assert np.array_equal(np.concatenate([o1, o2], axis=1), o) and np.array_equal(s2, st)


# The state never depends on the queries and the outputs are linear in them.
def test_queries_only_read():
    q, k, v, beta, g, S0 = _rand(8)
    o, st = gated_delta_rule_ref(q, k, v, beta, g, S0)
    o2, st2 = gated_delta_rule_ref(2.5 * q - 0.5 * q[:, ::-1], k, v, beta, g, S0)
    o3, _ = gated_delta_rule_ref(q[:, ::-1], k, v, beta, g, S0)
    assert np.array_equal(st, st2)
    assert _rel(o2, 2.5 * o - 0.5 * o3) < 1e-13


# hada.io digest, section "Chunkwise KDA" with D_i = alpha_i I, and section
# "Pipeline Triton Chunkwise" (decay ratios from prefix sums of log alpha):
# the chunked form equals the recurrence for every chunk size, with ragged
# tails, beta up to 2 and a nonzero incoming state.
@pytest.mark.parametrize("chunk", [1, 2, 4, 16, 64, 100])
def test_gated_chunk_form_equals_recurrence(chunk):
    q, k, v, beta, g, S0 = _rand(9, B=2, T=100, H=2, Dk=8, Dv=6, beta_hi=2.0, alpha_lo=0.2)
    o, st = gated_delta_rule_ref(q, k, v, beta, g, S0)
    o2, st2 = CA.gated_chunk_forward(q, k, v, beta, g, S0, chunk)
    assert _rel(o2, o) < 1e-12 and _rel(st2, st) < 1e-12


# With alpha = 1 the gated chunk step is the ungated one (the pages' chunked
# DeltaNet with D = I).
def test_gated_chunk_step_reduces_to_ungated():
    q, k, v, beta, g, S0 = _rand(10, B=1, T=16, H=1, Dk=8, Dv=6)
    a = CA.chunk_step(S0[0, 0], q[0, :, 0], k[0, :, 0], v[0, :, 0], beta[0, :, 0])
    b = CA.gated_chunk_step(S0[0, 0], q[0, :, 0], k[0, :, 0], v[0, :, 0], beta[0, :, 0],
                            np.zeros(16))
    for x, y in zip(a, b):
        assert _rel(y, x) < 1e-14
