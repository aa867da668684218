"""The chunkwise rearrangement the GPU kernels rely on, checked in fp64 before
any kernel exists.

* P8: the chunked form equals the token recurrence for every chunk length,
  ragged tails, beta up to 2 and a nonzero incoming state (hada.io digest,
  "Chunkwise KDA": the chunked schedule must reproduce the token-by-token
  state and outputs exactly).
* The UT-transform packaging (paperlayer summary of arXiv:2406.06484, App.
  B.2) and the triangular-solve packaging (hada.io digest, "Restauration de
  la dependance causale") give the same per-token errors: E = U - W S^T.
* P10: the WY representation (paperlayer summary, section 3) -- the product of
  a chunk's generalized Householder transitions equals I - W^T K.
* The level split of the chunked KDA kernel (each pair's decay as a row
  factor times a column factor around the pair's level reference) gives the
  decay of the tokens between the two, D_{j+1:i} of the hada.io digest's
  "Chunkwise KDA", for strong decays, erased channels and gk = -inf.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import delta_rule_ref
from oracle.chunk_algebra import chunk_forward, chunk_step, ut_transform


def _inputs(seed, B=1, T=100, H=2, Dk=16, Dv=12, beta_hi=2.0):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, T, H, Dk))
    k = r.standard_normal((B, T, H, Dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, T, H, Dv))
    beta = r.uniform(0.0, beta_hi, (B, T, H))
    S0 = 0.5 * r.standard_normal((B, H, Dv, Dk))
    return q, k, v, beta, S0


def _rel(a, b):
    return np.max(np.abs(a - b)) / np.max(np.abs(b))


@pytest.mark.parametrize("chunk", [1, 2, 4, 16, 64, 100, 128])
def test_p8_chunk_form_equals_recurrence(chunk):
    q, k, v, beta, S0 = _inputs(80 + chunk)
    o_ref, s_ref = delta_rule_ref(q, k, v, beta, S0)
    o, s = chunk_forward(q, k, v, beta, S0, chunk=chunk)
    assert _rel(o, o_ref) < 1e-12
    assert _rel(s, s_ref) < 1e-12


def test_p8_zero_initial_state_and_unequal_dims():
    q, k, v, beta, _ = _inputs(88, T=77, Dk=32, Dv=8, beta_hi=1.0)
    o_ref, s_ref = delta_rule_ref(q, k, v, beta, None)
    o, s = chunk_forward(q, k, v, beta, None, chunk=16)
    assert _rel(o, o_ref) < 1e-12
    assert _rel(s, s_ref) < 1e-12


def test_ut_transform_gives_the_same_errors():
    q, k, v, beta, S0 = _inputs(90, T=32)
    Q, K, V, b, S = q[0, :, 0], k[0, :, 0], v[0, :, 0], beta[0, :, 0], S0[0, 0]
    _, E, _ = chunk_step(S, Q, K, V, b)
    T_, W, U = ut_transform(K, V, b)
    assert _rel(U - W @ S.T, E) < 1e-12


@pytest.mark.parametrize("L", [1, 5, 16, 64])
def test_p10_wy_representation(L):
    q, k, v, beta, _ = _inputs(100 + L, T=L, beta_hi=2.0)
    K, V, b = k[0, :, 0], v[0, :, 0], beta[0, :, 0]
    Dk = K.shape[1]
    P = np.eye(Dk)
    for i in range(L):  # S_t = S_{t-1}(I - b k k^T) + ...: right-multiply in order
        P = P @ (np.eye(Dk) - b[i] * np.outer(K[i], K[i]))
    _, W, _ = ut_transform(K, V, b)
    np.testing.assert_allclose(np.eye(Dk) - W.T @ K, P, rtol=0, atol=1e-12)


def test_chunk_state_is_affine_in_incoming_state():
    # S_{c+1} = S_c (I - W^T K) + U^T K: the per-chunk map that a split over
    # sequence segments composes (paperlayer summary, section 5: associative
    # matrix-valued recurrences).
    q, k, v, beta, S0 = _inputs(110, T=64)
    Q, K, V, b, S = q[0, :, 0], k[0, :, 0], v[0, :, 0], beta[0, :, 0], S0[0, 0]
    _, _, S_next = chunk_step(S, Q, K, V, b)
    _, W, U = ut_transform(K, V, b)
    expect = S @ (np.eye(K.shape[1]) - W.T @ K) + U.T @ K
    assert _rel(S_next, expect) < 1e-12


def _level_decays(gk, C):
    """The decay between every pair of tokens (i, j), j <= i, of a chunk as the
    chunked KDA kernel forms it: pair (i, j), i > j, belongs to the level of
    the highest bit in which i and j differ; the reference is the last token
    of the first half of that level's aligned segment; the row factor is the
    product of exp(gk) over ref+1 .. i and the column factor over j+1 .. ref.
    Returns [i, j, d] (zero above the diagonal, one on it)."""
    e = np.exp(gk)                      # per-token factors, [C, d]
    out = np.zeros((C, C, gk.shape[1]))
    for i in range(C):
        out[i, i] = 1.0
        for j in range(i):
            L = 1 << ((i ^ j).bit_length() - 1)
            ref = (i // (2 * L)) * 2 * L + L - 1
            row = np.prod(e[ref + 1:i + 1], axis=0)
            col = np.prod(e[j + 1:ref + 1], axis=0)
            out[i, j] = row * col
    return out


@pytest.mark.parametrize("case", ["amax16", "erased", "minus_inf", "weak"])
def test_kda_level_factors_give_the_pairwise_decays(case):
    # hada.io digest, "Chunkwise KDA": the chunk's couplings and reads carry
    # D_{j+1:i} = diag(exp(b_i - b_j)) with b the in-chunk prefix sums of gk.
    # The kernel's level split must give exactly those ratios for any gk <= 0,
    # including channels erased in one token ("Kimi Delta Attention").
    r = np.random.default_rng(120)
    C, d = 32, 8
    if case == "amax16":
        gk = -16.0 * r.uniform(size=(1, d)) * np.log1p(np.exp(r.standard_normal((C, d)) + 1))
    elif case == "erased":
        gk = np.zeros((C, d))
        gk[:, d // 2:] = -1e4
    elif case == "minus_inf":
        gk = -r.uniform(0, 3, (C, d))
        gk[::3, 1::2] = -np.inf
    else:
        gk = -0.02 * r.uniform(size=(C, d))
    got = _level_decays(gk, C)
    # D_{j+1:i}: the decay of tokens j+1 .. i, one product per pair
    want = np.zeros_like(got)
    for i in range(C):
        for j in range(i + 1):
            want[i, j] = np.prod(np.exp(gk[j + 1:i + 1]), axis=0)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-300)
    # where the prefix sums are finite, exp(b_i - b_j) is the same ratio
    if np.all(np.isfinite(gk)):
        b = np.cumsum(gk, axis=0)
        with np.errstate(over="ignore"):  # above the diagonal: never used
            ratio = np.exp(b[:, None, :] - b[None, :, :])
        mask = np.tril(np.ones((C, C)))[:, :, None] > 0
        np.testing.assert_allclose(np.where(mask, got, 0), np.where(mask, ratio, 0),
                                   rtol=1e-9, atol=1e-300)
    # every factor the kernel multiplies by is at most 1
    assert np.all(got <= 1.0 + 1e-15)
