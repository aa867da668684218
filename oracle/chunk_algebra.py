"""Chunkwise-parallel form of the delta rule in fp64 NumPy -- TEST INFRASTRUCTURE ONLY.

Only the test suite may import this module.  It follows the chunked
rearrangement the pages give, step by step and in their order, with the
decay taken as the identity (plain DeltaNet) and no output scale:

* "Tour d'horizon des variantes d'attention lineaire de la famille DeltaNet"
  (hada.io digest), section "Chunkwise KDA : reorganiser la recurrence en
  multiplications matricielles":
    - "Atténuation cumulée et erreurs temporaires": provisional errors that
      ignore the other writes of the chunk, e_bar_i = beta_i (v_i - S_c k_i);
    - "Restauration de la dépendance causale": rho_ij = beta_i k_j^T k_i for
      j < i in a strictly lower-triangular R_c; the true errors solve the unit
      lower-triangular system (I + R_c) E = E_bar, by a triangular solve and
      not a dense inverse;
    - "Calcul de l'état de fin de chunk": S_{c+1} = S_c + E_c^T K_c
      (E_c stacked by rows here, one row per token);
    - "Calcul de toutes les sorties internes au chunk": the read matrix
      chi_ij = k_j^T q_i for j <= i (diagonal included, read after write),
      and O_c = Q_c S_c^T + A^qk E_c.
* "Parallelizing Linear Transformers with the Delta Rule over Sequence
  Length" (paperlayer summary of arXiv:2406.06484), App. B.2 "UT transform
  derivation": the same solve packaged as T = (I + A)^{-1} diag(beta) with
  A = tril(diag(beta) K K^T, -1), W = T K and U = T V (U by replacing K with
  V), so that E_c = U - W S_c^T.  Section 3 "Memory-efficient recurrence":
  the product of the chunk's generalized Householder transitions equals
  I - W^T K (the WY representation).

Every array here is per head: K, Q ``[L, Dk]``, V ``[L, Dv]``, beta ``[L]``,
S ``[Dv, Dk]``.

The gated functions take the same section with a scalar decay per token,
D_i = alpha_i I, alpha_i = exp(g_i) (section "Gated DeltaNet : oublier
d'abord l'etat entier" of the same digest for the recurrence): the cumulative
decay from the chunk boundary to token i is gamma_i = exp(b_i) with b the
in-chunk prefix sum of g (section "Pipeline Triton Chunkwise": differences of
prefix sums of the log decay stand for D_{j+1:i} = gamma_i / gamma_j), so

    e_bar_i = beta_i (v_i - gamma_i S_c k_i)
    rho_ij  = beta_i (gamma_i / gamma_j) k_j^T k_i            (j < i)
    S_{c+1} = gamma_last S_c + sum_j (gamma_last / gamma_j) e_j k_j^T
    O_i     = gamma_i S_c q_i + sum_{j <= i} (gamma_i / gamma_j) (k_j^T q_i) e_j
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def ut_transform(K, V, beta):
    """UT transform of one chunk: returns (T, W, U).

    A = tril(diag(beta) K K^T, -1); T = (I + A)^{-1} diag(beta) by a unit
    lower-triangular solve; W = T K; U = T V.
    """
    K, V, beta = _f64(K), _f64(V), _f64(beta)
    L = K.shape[0]
    A = np.tril(beta[:, None] * (K @ K.T), -1)
    T = solve_triangular(np.eye(L) + A, np.diag(beta), lower=True,
                         unit_diagonal=True)
    return T, T @ K, T @ V


def chunk_step(S, Q, K, V, beta):
    """Advance one chunk from its incoming state S.

    Returns (O_c, E_c, S_next) where E_c are the resolved per-token errors
    (one row per token; the "v_new" of the chunked kernels).
    """
    S, Q, K, V, beta = (_f64(x) for x in (S, Q, K, V, beta))
    L = K.shape[0]
    # provisional errors against the incoming state only
    E_bar = beta[:, None] * (V - K @ S.T)
    # causal coupling rho_ij = beta_i k_j.k_i (j < i), strictly lower
    R = np.tril(beta[:, None] * (K @ K.T), -1)
    E = solve_triangular(np.eye(L) + R, E_bar, lower=True, unit_diagonal=True)
    # end-of-chunk state: all rank-1 writes of the chunk in one product
    S_next = S + E.T @ K
    # outputs: incoming state read plus the chunk's own writes, diagonal included
    A_qk = np.tril(Q @ K.T)
    O = Q @ S.T + A_qk @ E
    return O, E, S_next


def chunk_forward_head(Q, K, V, beta, S0=None, chunk=64):
    """Chunkwise forward of one head: returns (O [L,Dv], S_T [Dv,Dk])."""
    Q, K, V, beta = (_f64(x) for x in (Q, K, V, beta))
    L, Dk = K.shape
    Dv = V.shape[1]
    S = np.zeros((Dv, Dk)) if S0 is None else _f64(S0).copy()
    O = np.zeros((L, Dv))
    for c0 in range(0, L, chunk):
        sl = slice(c0, min(c0 + chunk, L))
        O[sl], _, S = chunk_step(S, Q[sl], K[sl], V[sl], beta[sl])
    return O, S


def gated_chunk_step(S, Q, K, V, beta, g):
    """Advance one chunk of the gated recurrence from its incoming state S.

    Returns (O_c, E_c, S_next); g is the chunk's log decay per token."""
    S, Q, K, V, beta, g = (_f64(x) for x in (S, Q, K, V, beta, g))
    L = K.shape[0]
    b = np.cumsum(g)                       # log of the decay from the boundary
    gam = np.exp(b)
    ratio = np.exp(b[:, None] - b[None, :])  # gamma_i / gamma_j
    # provisional errors against the decayed incoming state
    E_bar = beta[:, None] * (V - gam[:, None] * (K @ S.T))
    # causal coupling with the decay between the two tokens, strictly lower
    R = np.tril(beta[:, None] * ratio * (K @ K.T), -1)
    E = solve_triangular(np.eye(L) + R, E_bar, lower=True, unit_diagonal=True)
    # end-of-chunk state: the incoming state decays through the whole chunk,
    # each write only through the tokens after it
    to_end = np.exp(b[-1] - b)
    S_next = gam[-1] * S + (to_end[:, None] * E).T @ K
    # outputs: decayed incoming state plus the decayed writes, diagonal included
    A_qk = np.tril(ratio * (Q @ K.T))
    O = gam[:, None] * (Q @ S.T) + A_qk @ E
    return O, E, S_next


def gated_chunk_forward(q, k, v, beta, g, S0=None, chunk=64):
    """Gated chunkwise forward over the op layout (g [B,T,H]).  Returns
    (o, S_T) in fp64."""
    q, k, v, beta, g = (_f64(x) for x in (q, k, v, beta, g))
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    s0 = None if S0 is None else _f64(S0)
    o = np.zeros((B, T, H, Dv))
    st = np.zeros((B, H, Dv, Dk))
    for bb in range(B):
        for h in range(H):
            S = np.zeros((Dv, Dk)) if s0 is None else s0[bb, h].copy()
            for c0 in range(0, T, chunk):
                sl = slice(c0, min(c0 + chunk, T))
                o[bb, sl, h], _, S = gated_chunk_step(S, q[bb, sl, h], k[bb, sl, h],
                                                      v[bb, sl, h], beta[bb, sl, h],
                                                      g[bb, sl, h])
            st[bb, h] = S
    return o, st


def kda_chunk_step(S, Q, K, V, beta, gk):
    """Advance one chunk of the per-channel-decay recurrence (KDA) from its
    incoming state S, as the hada.io digest's section "Chunkwise KDA" states
    it: cumulative per-channel decays from the chunk boundary, provisional
    errors against the decayed incoming state, couplings
    rho_ij = beta_i k_j^T D_{j+1:i} k_i, a unit lower-triangular solve, the
    end-of-chunk state S D_{0:L-1} + E^T K_end and the outputs with the
    diagonal included.  gk is the chunk's [L, Dk] log decay.  Returns
    (O_c, E_c, S_next)."""
    S, Q, K, V, beta, gk = (_f64(x) for x in (S, Q, K, V, beta, gk))
    L = K.shape[0]
    b = np.cumsum(gk, axis=0)                        # [L, Dk] log of D_{0:i}
    dec = np.exp(b[:, None, :] - b[None, :, :])      # [i, j, d]: D_{j+1:i}
    E_bar = beta[:, None] * (V - (K * np.exp(b)) @ S.T)
    R = np.tril(beta[:, None] * np.einsum("jd,id,ijd->ij", K, K, dec), -1)
    E = solve_triangular(np.eye(L) + R, E_bar, lower=True, unit_diagonal=True)
    K_end = K * np.exp(b[-1][None, :] - b)           # keys decayed to the chunk end
    S_next = S * np.exp(b[-1])[None, :] + E.T @ K_end
    A_qk = np.tril(np.einsum("jd,id,ijd->ij", K, Q, dec))
    O = (Q * np.exp(b)) @ S.T + A_qk @ E
    return O, E, S_next


def kda_chunk_forward(q, k, v, beta, gk, S0=None, chunk=64):
    """KDA chunkwise forward over the op layout (gk [B,T,H,Dk]).  Returns
    (o, S_T) in fp64."""
    q, k, v, beta, gk = (_f64(x) for x in (q, k, v, beta, gk))
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    s0 = None if S0 is None else _f64(S0)
    o = np.zeros((B, T, H, Dv))
    st = np.zeros((B, H, Dv, Dk))
    for bb in range(B):
        for h in range(H):
            S = np.zeros((Dv, Dk)) if s0 is None else s0[bb, h].copy()
            for c0 in range(0, T, chunk):
                sl = slice(c0, min(c0 + chunk, T))
                o[bb, sl, h], _, S = kda_chunk_step(S, q[bb, sl, h], k[bb, sl, h],
                                                    v[bb, sl, h], beta[bb, sl, h],
                                                    gk[bb, sl, h])
            st[bb, h] = S
    return o, st


def chunk_forward(q, k, v, beta, S0=None, chunk=64):
    """Chunkwise forward over the op layout: q,k [B,T,H,Dk], v [B,T,H,Dv],
    beta [B,T,H], S0 [B,H,Dv,Dk] or None.  Returns (o, S_T) in fp64."""
    q, k, v, beta = (_f64(x) for x in (q, k, v, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    s0 = None if S0 is None else _f64(S0)
    o = np.zeros((B, T, H, Dv))
    st = np.zeros((B, H, Dv, Dk))
    for b in range(B):
        for h in range(H):
            o[b, :, h], st[b, h] = chunk_forward_head(
                q[b, :, h], k[b, :, h], v[b, :, h], beta[b, :, h],
                None if s0 is None else s0[b, h], chunk)
    return o, st


__all__ = ["ut_transform", "chunk_step", "chunk_forward_head", "chunk_forward",
           "gated_chunk_step", "gated_chunk_forward"]
