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
