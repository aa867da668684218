"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test names the passage it rests on.  None of them re-types the oracle's
own loop: they check other forms of the update the pages state, closed forms,
special cases with exact answers, invariants, an exact-rational brute force
and a hand-worked example.  Together they are chosen so that a dropped term, a
wrong sign, a read before the write, an off-by-one token, a transposed state
or a lost initial state each fails at least one test.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.linalg import solve_triangular

from oracle import delta_rule_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _unit(x, axis=-1):
    return x / np.linalg.norm(x, axis=axis, keepdims=True)


def _rand(seed, B=2, T=24, H=3, Dk=5, Dv=4, beta_hi=1.0, s0=True, unit=True):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, T, H, Dk))
    k = r.standard_normal((B, T, H, Dk))
    if unit:
        q, k = _unit(q), _unit(k)
    v = r.standard_normal((B, T, H, Dv))
    beta = r.uniform(0.0, beta_hi, (B, T, H))
    S0 = r.standard_normal((B, H, Dv, Dk)) * 0.3 if s0 else None
    return q, k, v, beta, S0


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# --------------------------------------------------------------------------
# P1: the equivalent forms of one update agree.
# hada.io digest, sections "DeltaNet : ecrire l'erreur de prediction ..."
# (the three readings: memory overwrite, online gradient step, rank-1 update)
# and "Transition d'etat structuree" (the generalized Householder form);
# houmin.site "infra/delta-net", section "DeltaNet 引入 Delta Rule" (the
# erase-old / write-new form with v_old and v_new).
# --------------------------------------------------------------------------
def _run_form(step, q, k, v, beta, S0):
    """Drive a single-head per-token update `step(S, k, v, beta) -> S` and
    read o_t = S_t q_t after each write."""
    T, Dk = k.shape
    S = S0.copy()
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        S = step(S, k[t], v[t], beta[t])
        o[t] = S @ q[t]
    return o, S


def _householder(S, k, v, b):
    return S @ (np.eye(k.size) - b * np.outer(k, k)) + b * np.outer(v, k)


def _erase_write(S, k, v, b):
    v_old = S @ k
    v_new = b * v + (1.0 - b) * v_old
    return S - np.outer(v_old, k) + np.outer(v_new, k)


def _gradient_step(S, k, v, b):
    # one SGD step of size beta on the reconstruction loss 1/2 ||S k - v||^2,
    # with the gradient taken by autograd rather than written out
    St = torch.tensor(S, dtype=torch.float64, requires_grad=True)
    loss = 0.5 * torch.sum((St @ torch.tensor(k) - torch.tensor(v)) ** 2)
    (g,) = torch.autograd.grad(loss, St)
    return S - b * g.numpy()


@pytest.mark.parametrize("form", [_householder, _erase_write, _gradient_step])
def test_p1_equivalent_update_forms(form):
    q, k, v, beta, S0 = _rand(1, B=1, H=2, T=20, Dk=6, Dv=5, beta_hi=2.0)
    o_ref, st_ref = delta_rule_ref(q, k, v, beta, S0)
    for h in range(2):
        o, S = _run_form(form, q[0, :, h], k[0, :, h], v[0, :, h],
                         beta[0, :, h], S0[0, h])
        assert _rel(o, o_ref[0, :, h]) < 1e-13
        assert _rel(S, st_ref[0, h]) < 1e-13


# --------------------------------------------------------------------------
# P2: beta = 0 leaves the memory unchanged (houmin.site, "DeltaNet 引入
# Delta Rule": the beta_t = 0 case), so every read returns S0 q_t.
# --------------------------------------------------------------------------
def test_p2_beta_zero_keeps_state():
    q, k, v, beta, S0 = _rand(2)
    beta[:] = 0.0
    o, st = delta_rule_ref(q, k, v, beta, S0)
    np.testing.assert_array_equal(st, S0)
    expect = np.einsum("bhij,bthj->bthi", S0, q)
    assert _rel(o, expect) < 1e-14


# --------------------------------------------------------------------------
# P3: beta = 1 with a unit key: re-reading with the same key returns exactly
# the value just written (hada.io digest, "DeltaNet : ecrire l'erreur ...":
# the immediate re-read is (1-beta) S_{t-1} k_t + beta v_t).  Reading with
# q_t = k_t makes o_t that re-read.
# --------------------------------------------------------------------------
def test_p3_beta_one_recalls_value():
    q, k, v, beta, S0 = _rand(3, T=30, Dk=8, Dv=6)
    beta[:] = 1.0
    o, _ = delta_rule_ref(k, k, v, beta, S0)
    assert _rel(o, v) < 1e-13


def test_p3b_partial_reread_interpolates():
    # general beta: o_t (with q_t = k_t) = (1-beta_t) S_{t-1} k_t + beta_t v_t
    q, k, v, beta, S0 = _rand(31, B=1, H=1, T=12, Dk=6, Dv=4)
    o, _ = delta_rule_ref(k, k, v, beta, S0)
    for t in range(12):
        _, s_prev = delta_rule_ref(k[:, :t], k[:, :t], v[:, :t], beta[:, :t], S0)
        pred = s_prev[0, 0] @ k[0, t, 0]
        expect = (1 - beta[0, t, 0]) * pred + beta[0, t, 0] * v[0, t, 0]
        assert _rel(o[0, t, 0], expect) < 1e-12


# --------------------------------------------------------------------------
# P4: orthonormal keys with beta = 1 store every pair exactly, whatever S0
# (hada.io digest: the update only replaces the association along the
# current key and leaves orthogonal directions untouched).
# --------------------------------------------------------------------------
def test_p4_orthonormal_keys_exact_recall():
    r = np.random.default_rng(4)
    Dk, Dv, T = 8, 5, 8
    Qm, _ = np.linalg.qr(r.standard_normal((Dk, Dk)))
    k = Qm.T[:T][None, :, None, :]           # rows are orthonormal keys
    v = r.standard_normal((1, T, 1, Dv))
    q = _unit(r.standard_normal((1, T, 1, Dk)))
    beta = np.ones((1, T, 1))
    S0 = r.standard_normal((1, 1, Dv, Dk))
    _, st = delta_rule_ref(q, k, v, beta, S0)
    for i in range(T):
        np.testing.assert_allclose(st[0, 0] @ k[0, i, 0], v[0, i, 0],
                                   rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# P5: locality -- a query orthogonal to the current key sees no change from
# this token's write (hada.io digest, "DeltaNet : ecrire l'erreur ...").
# --------------------------------------------------------------------------
def test_p5_orthogonal_query_unaffected():
    q, k, v, beta, S0 = _rand(5, B=1, H=1, T=10, Dk=6, Dv=4)
    # make q_t orthogonal to k_t
    kk = k[0, :, 0]
    qq = q[0, :, 0] - np.sum(q[0, :, 0] * kk, axis=1, keepdims=True) * kk
    q[0, :, 0] = qq
    o, _ = delta_rule_ref(q, k, v, beta, S0)
    for t in range(10):
        _, s_prev = delta_rule_ref(q[:, :t], k[:, :t], v[:, :t], beta[:, :t], S0)
        np.testing.assert_allclose(o[0, t, 0], s_prev[0, 0] @ qq[t],
                                   rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# P6: with v = 0 and a unit key the transition I - beta k k^T has eigenvalue
# 1 - beta along k and 1 elsewhere (hada.io digest, "Transition d'etat
# structuree").  beta = 2 makes it a reflection (Frobenius norm kept);
# beta in (0,2) never grows the norm.  fla fla/layers/delta_net.py doubles
# beta for this negative-eigenvalue regime (allow_neg_eigval).
# --------------------------------------------------------------------------
def test_p6_reflection_preserves_norm():
    q, k, v, beta, S0 = _rand(6, T=40)
    v[:] = 0.0
    beta[:] = 2.0
    _, st = delta_rule_ref(q, k, v, beta, S0)
    n0 = np.linalg.norm(S0, axis=(2, 3))
    n1 = np.linalg.norm(st, axis=(2, 3))
    np.testing.assert_allclose(n1, n0, rtol=1e-12)


def test_p6_contraction_never_grows():
    q, k, v, beta, S0 = _rand(61, B=1, H=1, T=30, beta_hi=2.0)
    v[:] = 0.0
    prev = np.linalg.norm(S0)
    for t in range(1, 31):
        _, st = delta_rule_ref(q[:, :t], k[:, :t], v[:, :t], beta[:, :t], S0)
        cur = np.linalg.norm(st)
        assert cur <= prev * (1 + 1e-14)
        prev = cur


# --------------------------------------------------------------------------
# P7: orthonormal keys and S0 = 0: the delta rule has nothing to erase, so
# it reduces to causal linear attention on beta-scaled values,
# O = (Q K^T (.) M) diag(beta) V with M inclusive lower-triangular (hada.io
# digest, "De l'attention quadratique a un etat lineaire"; houmin.site,
# "Linear Attention").  The diagonal of M is the read-after-write.
# --------------------------------------------------------------------------
def test_p7_linear_attention_closed_form():
    r = np.random.default_rng(7)
    Dk, Dv, T = 12, 7, 12
    Qm, _ = np.linalg.qr(r.standard_normal((Dk, Dk)))
    K = Qm.T[:T]
    Q = r.standard_normal((T, Dk))
    V = r.standard_normal((T, Dv))
    beta = r.uniform(0.1, 1.9, T)
    o, st = delta_rule_ref(Q[None, :, None], K[None, :, None], V[None, :, None],
                           beta[None, :, None])
    M = np.tril(np.ones((T, T)))
    expect = ((Q @ K.T) * M) @ (beta[:, None] * V)
    assert _rel(o[0, :, 0], expect) < 1e-13
    assert _rel(st[0, 0], (beta[:, None] * V).T @ K) < 1e-13


# --------------------------------------------------------------------------
# P9: the fully parallel form in houmin.site's summary table ("总结"),
# O = (Q K^T (.) M)(I + K K^T (.) M^-)^{-1} V (beta = 1, S0 = 0, M^- strictly
# lower), evaluated with a library triangular solve.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("T", [1, 7, 64, 200])
def test_p9_fully_parallel_form(T):
    r = np.random.default_rng(9 + T)
    Dk, Dv = 16, 9
    K = _unit(r.standard_normal((T, Dk)))
    Q = _unit(r.standard_normal((T, Dk)))
    V = r.standard_normal((T, Dv))
    beta = np.ones(T)
    o, _ = delta_rule_ref(Q[None, :, None], K[None, :, None], V[None, :, None],
                          beta[None, :, None])
    M = np.tril(np.ones((T, T)))
    Mm = np.tril(np.ones((T, T)), -1)
    X = solve_triangular(np.eye(T) + (K @ K.T) * Mm, V, lower=True,
                         unit_diagonal=True)
    expect = ((Q @ K.T) * M) @ X
    assert _rel(o[0, :, 0], expect) < 1e-12


# --------------------------------------------------------------------------
# P11: resume -- the state is the whole carried context (fla
# fla/layers/delta_net.py: initial_state in, final state out through the
# layer cache).  Splitting the sequence anywhere gives the same result.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("cut", [0, 1, 13, 31, 32])
def test_p11_resume(cut):
    q, k, v, beta, S0 = _rand(11, T=32, beta_hi=2.0)
    o, st = delta_rule_ref(q, k, v, beta, S0)
    o1, s1 = delta_rule_ref(q[:, :cut], k[:, :cut], v[:, :cut], beta[:, :cut], S0)
    o2, s2 = delta_rule_ref(q[:, cut:], k[:, cut:], v[:, cut:], beta[:, cut:], s1)
    np.testing.assert_array_equal(np.concatenate([o1, o2], axis=1), o)
    np.testing.assert_array_equal(s2, st)


# --------------------------------------------------------------------------
# P12: decode is the same recurrence one token per call (hada.io digest,
# "Pipeline Triton Chunkwise": recurrent and chunked modes are two schedules
# of one recurrence).
# --------------------------------------------------------------------------
def test_p12_token_by_token_equals_sequence():
    q, k, v, beta, S0 = _rand(12, T=17)
    o, st = delta_rule_ref(q, k, v, beta, S0)
    S = S0
    for t in range(17):
        ot, S = delta_rule_ref(q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1],
                               beta[:, t:t + 1], S)
        np.testing.assert_array_equal(ot[:, 0], o[:, t])
    np.testing.assert_array_equal(S, st)


# --------------------------------------------------------------------------
# P13: structure of the map.  S_T does not depend on q; o is linear in q;
# with S0 = 0, (o, S_T) is linear in V (the state is a sum of outer products
# of value-space errors with keys).
# --------------------------------------------------------------------------
def test_p13_linearity():
    q, k, v, beta, S0 = _rand(13, T=15)
    q2 = _rand(130, T=15)[0]
    o_a, st_a = delta_rule_ref(q, k, v, beta, S0)
    o_b, st_b = delta_rule_ref(q2, k, v, beta, S0)
    np.testing.assert_array_equal(st_a, st_b)
    o_c, _ = delta_rule_ref(2.0 * q - 3.0 * q2, k, v, beta, S0)
    assert _rel(o_c, 2.0 * o_a - 3.0 * o_b) < 1e-13
    v2 = _rand(131, T=15)[2]
    oa, sa = delta_rule_ref(q, k, v, beta, None)
    ob, sb = delta_rule_ref(q, k, v2, beta, None)
    oc, sc = delta_rule_ref(q, k, 0.5 * v + 4.0 * v2, beta, None)
    assert _rel(oc, 0.5 * oa + 4.0 * ob) < 1e-13
    assert _rel(sc, 0.5 * sa + 4.0 * sb) < 1e-13


# --------------------------------------------------------------------------
# P14: exact rational brute force on tiny dyadic inputs (exact in fp64).
# The fp64 oracle must agree with exact arithmetic to rounding level.
# --------------------------------------------------------------------------
def _exact(q, k, v, beta, S0):
    T, Dk = len(k), len(k[0])
    Dv = len(v[0])
    S = [row[:] for row in S0]
    outs = []
    for t in range(T):
        err = [beta[t] * (v[t][i] - sum(S[i][j] * k[t][j] for j in range(Dk)))
               for i in range(Dv)]
        S = [[S[i][j] + err[i] * k[t][j] for j in range(Dk)] for i in range(Dv)]
        outs.append([sum(S[i][j] * q[t][j] for j in range(Dk)) for i in range(Dv)])
    return outs, S


@pytest.mark.parametrize("seed", range(6))
def test_p14_exact_rational(seed):
    r = np.random.default_rng(140 + seed)
    T, Dk, Dv = int(r.integers(1, 7)), int(r.integers(1, 5)), int(r.integers(1, 5))

    def dy(shape):  # dyadic rationals m / 8 with |m| <= 12
        return r.integers(-12, 13, shape) / 8.0

    q, k, v, S0 = dy((T, Dk)), dy((T, Dk)), dy((T, Dv)), dy((Dv, Dk))
    beta = r.integers(0, 9, T) / 4.0   # 0 .. 2 in quarters
    fr = lambda a: [[Fraction(x) for x in row] for row in a]
    o_x, s_x = _exact(fr(q), fr(k), fr(v), [Fraction(b) for b in beta], fr(S0))
    o, st = delta_rule_ref(q[None, :, None], k[None, :, None], v[None, :, None],
                           beta[None, :, None], S0[None, None])
    o_x = np.array([[float(x) for x in row] for row in o_x])
    s_x = np.array([[float(x) for x in row] for row in s_x])
    scale = max(np.max(np.abs(o_x)), np.max(np.abs(s_x)), 1.0)
    assert np.max(np.abs(o[0, :, 0] - o_x)) <= 1e-14 * scale
    assert np.max(np.abs(st[0, 0] - s_x)) <= 1e-14 * scale


# --------------------------------------------------------------------------
# Hand-worked example (tests/golden/hand_worked_d2_t3.json): every value is a
# dyadic rational, so the oracle must reproduce it bit for bit.
# --------------------------------------------------------------------------
def test_hand_worked_example():
    with open(os.path.join(GOLDEN, "hand_worked_d2_t3.json")) as f:
        g = json.load(f)
    q = np.array(g["q"], float)[None, :, None]
    k = np.array(g["k"], float)[None, :, None]
    v = np.array(g["v"], float)[None, :, None]
    beta = np.array(g["beta"], float)[None, :, None]
    o, st = delta_rule_ref(q, k, v, beta)
    np.testing.assert_array_equal(o[0, :, 0], np.array(g["o"], float))
    np.testing.assert_array_equal(st[0, 0], np.array(g["S_T"], float))


# --------------------------------------------------------------------------
# Host logic of the oracle itself: edge sizes and thread-count independence.
# --------------------------------------------------------------------------
def test_empty_sequence_returns_initial_state():
    q, k, v, beta, S0 = _rand(20, T=0)
    o, st = delta_rule_ref(q, k, v, beta, S0)
    assert o.shape == (2, 0, 3, 4)
    np.testing.assert_array_equal(st, S0)
    _, st0 = delta_rule_ref(q, k, v, beta, None)
    np.testing.assert_array_equal(st0, 0.0)


def test_thread_count_does_not_change_result(oracle_threads):
    q, k, v, beta, S0 = _rand(21, B=3, T=40, H=5)
    a = delta_rule_ref(q, k, v, beta, S0, nthreads=1)
    b = delta_rule_ref(q, k, v, beta, S0, nthreads=max(2, oracle_threads))
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_heads_and_batch_are_independent():
    q, k, v, beta, S0 = _rand(22, B=2, T=9, H=3)
    o, st = delta_rule_ref(q, k, v, beta, S0)
    for b in range(2):
        for h in range(3):
            ob, sb = delta_rule_ref(q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h:h + 1],
                                    v[b:b + 1, :, h:h + 1], beta[b:b + 1, :, h:h + 1],
                                    S0[b:b + 1, h:h + 1])
            np.testing.assert_array_equal(ob[0, :, 0], o[b, :, h])
            np.testing.assert_array_equal(sb[0, 0], st[b, h])


def test_rejects_bad_shapes():
    q, k, v, beta, S0 = _rand(23)
    with pytest.raises(ValueError):
        delta_rule_ref(q, k[:, :-1], v, beta, S0)
    with pytest.raises(ValueError):
        delta_rule_ref(q, k, v, beta, S0[:, :, :-1])


# ----------------------------------------------------------------- l2norm
# houmin.site "infra/delta-net", Gated DeltaNet code: the l2norm helper
# multiplies a row by 1/sqrt(sum of squares + 1e-6).
def test_l2norm_rows_hand_values():
    from oracle import l2norm_rows
    x = np.array([[3.0, 4.0], [0.0, 0.0], [1e-4, 0.0]])
    y = l2norm_rows(x)
    assert np.allclose(y[0], np.array([3.0, 4.0]) / np.sqrt(25.0 + 1e-6), rtol=0, atol=1e-16)
    assert np.array_equal(y[1], np.zeros(2))          # a zero row stays zero
    # eps dominates tiny rows: 1e-4 / sqrt(1e-8 + 1e-6)
    assert abs(y[2, 0] - 1e-4 / np.sqrt(1.01e-6)) < 1e-15


def test_l2norm_rows_gives_unit_rows_and_keeps_direction():
    from oracle import l2norm_rows
    r = np.random.default_rng(11)
    x = 3.0 * r.standard_normal((4, 5, 7))
    y = l2norm_rows(x)
    n2 = np.sum(x * x, axis=-1)
    assert np.allclose(np.sum(y * y, axis=-1), n2 / (n2 + 1e-6), rtol=1e-14, atol=0)
    cos = np.sum(x * y, axis=-1) / np.sqrt(n2 * np.sum(y * y, axis=-1))
    assert np.allclose(cos, 1.0, rtol=0, atol=1e-14)
