"""fp64 CPU oracle of the DeltaNet delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(``deltanet_delta_rule_amd``) and imports nothing from it; the two meet only
through the seeded input generator, which holds none of the method's
arithmetic.

Contents
--------
``delta_rule_ref``
    The plain sequential recurrence in fp64 (C, ``ref_delta_rule.c``), the
    definition every GPU result is judged against.  See that file's header for
    the passages it follows.
``gated_delta_rule_ref``
    The same loop with a scalar forget gate alpha_t = exp(g_t) applied to the
    whole state before each token's prediction (the gated variant).
``kda_ref``
    The per-key-channel decay variant (Kimi Delta Attention): column j of the
    state decays by exp(gk_t[j]) before each token's prediction.
``delta_rule_bwd_ref``
    Gradients with respect to q, k, v, beta, S0 (and g for the gated rule)
    by the chain rule through the recurrence in reverse token order, in fp64
    (C, ``ref_delta_rule_bwd.c``).
``kda_bwd_ref``
    The same gradients for the per-key-channel decay, with dgk.
``l2norm_rows``
    x / sqrt(sum x^2 + eps) along the last axis in fp64: the in-kernel
    normalisation option applied to q and k before either oracle.
``chunk_algebra``
    The chunkwise-parallel rearrangement of the same recurrence in fp64 NumPy,
    step by step as the pages state it.  It is used only to pin the oracle and
    the algebra the GPU kernels rely on; GPU parity is always judged against
    ``delta_rule_ref``.

Parity status: every function here is pinned by ``tests/test_oracle.py``,
``tests/test_gated_oracle.py`` and ``tests/test_chunk_algebra.py`` (equivalent update forms, closed forms,
special cases, an exact-rational brute force and a hand-worked example).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = [os.path.join(_HERE, "ref_delta_rule.c"), os.path.join(_HERE, "ref_delta_rule_bwd.c")]
_LIB_PATH = os.path.join(_HERE, "libref_delta_rule.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile the C oracle with gcc (fp64, no FMA contraction) in place."""
    cmd = [
        "gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
        "-shared", "-fPIC", "-pthread", *_SRC, "-lm", "-o", _LIB_PATH + ".tmp",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.ref_delta_rule_f64.restype = ctypes.c_int
    lib.ref_delta_rule_f64.argtypes = [dp, dp, dp, dp, dp, dp, dp,
                                       i64, i64, i64, i64, i64, ctypes.c_int]
    lib.ref_kda_f64.restype = ctypes.c_int
    lib.ref_kda_f64.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp,
                                i64, i64, i64, i64, i64, ctypes.c_int]
    lib.ref_delta_rule_bwd_f64.restype = ctypes.c_int
    lib.ref_delta_rule_bwd_f64.argtypes = [dp] * 14 + [i64, i64, i64, i64, i64, ctypes.c_int]
    lib.ref_kda_bwd_f64.restype = ctypes.c_int
    lib.ref_kda_bwd_f64.argtypes = [dp] * 14 + [i64, i64, i64, i64, i64, ctypes.c_int]
    lib.ref_gated_delta_rule_f64.restype = ctypes.c_int
    lib.ref_gated_delta_rule_f64.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp,
                                             i64, i64, i64, i64, i64, ctypes.c_int]
    _lib = lib
    return lib


def _as_f64(x) -> np.ndarray:
    """Widen an array-like (NumPy or CPU torch tensor) to contiguous fp64."""
    if hasattr(x, "detach"):  # torch tensor: widen on the torch side first
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _check(q, k, v, beta, S0):
    q, k, v, beta = (_as_f64(x) for x in (q, k, v, beta))
    if q.ndim != 4 or k.shape != q.shape or v.ndim != 4 or beta.ndim != 3:
        raise ValueError("expected q,k [B,T,H,Dk], v [B,T,H,Dv], beta [B,T,H]")
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    if v.shape[:3] != (B, T, H) or beta.shape != (B, T, H):
        raise ValueError("inconsistent leading dimensions")
    s0 = None
    if S0 is not None:
        s0 = _as_f64(S0)
        if s0.shape != (B, H, Dv, Dk):
            raise ValueError(f"S0 must be [B,H,Dv,Dk]={B, H, Dv, Dk}, got {s0.shape}")
    return q, k, v, beta, s0, (B, T, H, Dk, Dv)


def delta_rule_ref(q, k, v, beta, S0=None, nthreads: int = 1):
    """Run the delta-rule recurrence in fp64 on the CPU.

    Arguments are array-likes with the layouts q, k ``[B,T,H,Dk]``,
    v ``[B,T,H,Dv]``, beta ``[B,T,H]`` and S0 ``[B,H,Dv,Dk]`` (or None for a
    zero initial state).  They are widened to fp64 exactly (the caller passes
    values already rounded to the dtype under test).

    Returns ``(o, S_T)`` as fp64 NumPy arrays: o ``[B,T,H,Dv]`` and
    S_T ``[B,H,Dv,Dk]``.
    """
    q, k, v, beta, s0, (B, T, H, Dk, Dv) = _check(q, k, v, beta, S0)
    o = np.zeros((B, T, H, Dv), dtype=np.float64)
    st = np.zeros((B, H, Dv, Dk), dtype=np.float64)
    rc = _load().ref_delta_rule_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                    _ptr(s0), _ptr(o), _ptr(st),
                                    B, T, H, Dk, Dv, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle failed with code {rc}")
    return o, st


def gated_delta_rule_ref(q, k, v, beta, g, S0=None, nthreads: int = 1):
    """The gated recurrence in fp64 on the CPU: before each token the whole
    state is multiplied by alpha_t = exp(g_t), then the token is predicted,
    corrected and written as in ``delta_rule_ref``.  g is ``[B,T,H]`` (the
    natural log of the forget gate); the other arguments and the return value
    are as in ``delta_rule_ref``."""
    q, k, v, beta, s0, (B, T, H, Dk, Dv) = _check(q, k, v, beta, S0)
    g = _as_f64(g)
    if g.shape != (B, T, H):
        raise ValueError(f"g must be [B,T,H]={B, T, H}, got {g.shape}")
    o = np.zeros((B, T, H, Dv), dtype=np.float64)
    st = np.zeros((B, H, Dv, Dk), dtype=np.float64)
    rc = _load().ref_gated_delta_rule_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                                          _ptr(s0), _ptr(o), _ptr(st),
                                          B, T, H, Dk, Dv, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle failed with code {rc}")
    return o, st


def kda_ref(q, k, v, beta, gk, S0=None, nthreads: int = 1):
    """The per-channel-decay recurrence (Kimi Delta Attention) in fp64 on the
    CPU: before each token, column j of the state (key channel j) is
    multiplied by exp(gk_t[j]), then the token is predicted, corrected and
    written as in ``delta_rule_ref``.  gk is ``[B,T,H,Dk]``; the rest as
    ``delta_rule_ref``."""
    q, k, v, beta, s0, (B, T, H, Dk, Dv) = _check(q, k, v, beta, S0)
    gk = _as_f64(gk)
    if gk.shape != (B, T, H, Dk):
        raise ValueError(f"gk must be [B,T,H,Dk]={B, T, H, Dk}, got {gk.shape}")
    o = np.zeros((B, T, H, Dv), dtype=np.float64)
    st = np.zeros((B, H, Dv, Dk), dtype=np.float64)
    rc = _load().ref_kda_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(gk), _ptr(s0),
                             _ptr(o), _ptr(st), B, T, H, Dk, Dv, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle failed with code {rc}")
    return o, st


def delta_rule_bwd_ref(q, k, v, beta, do, S0=None, dS_T=None, g=None, nthreads: int = 1):
    """Gradients of L = sum <do, o> + <dS_T, S_T> through the recurrence in
    fp64 on the CPU (``ref_delta_rule_bwd.c``: the chain rule through each
    token in reverse order, with the forward states kept).  g (log forget
    gate, [B,T,H]) selects the gated rule.  do is ``[B,T,H,Dv]``; dS_T is
    ``[B,H,Dv,Dk]`` or None (zero).  Returns a dict with dq, dk, dv, dbeta,
    dS0 and, for the gated rule, dg."""
    q, k, v, beta, s0, (B, T, H, Dk, Dv) = _check(q, k, v, beta, S0)
    do = _as_f64(do)
    if do.shape != (B, T, H, Dv):
        raise ValueError(f"do must be [B,T,H,Dv]={B, T, H, Dv}, got {do.shape}")
    dst = None
    if dS_T is not None:
        dst = _as_f64(dS_T)
        if dst.shape != (B, H, Dv, Dk):
            raise ValueError(f"dS_T must be [B,H,Dv,Dk]={B, H, Dv, Dk}, got {dst.shape}")
    gg = None
    if g is not None:
        gg = _as_f64(g)
        if gg.shape != (B, T, H):
            raise ValueError(f"g must be [B,T,H]={B, T, H}, got {gg.shape}")
    out = {"dq": np.zeros((B, T, H, Dk)), "dk": np.zeros((B, T, H, Dk)),
           "dv": np.zeros((B, T, H, Dv)), "dbeta": np.zeros((B, T, H)),
           "dS0": np.zeros((B, H, Dv, Dk))}
    if gg is not None:
        out["dg"] = np.zeros((B, T, H))
    rc = _load().ref_delta_rule_bwd_f64(
        _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(gg), _ptr(s0), _ptr(do), _ptr(dst),
        _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dbeta"]),
        _ptr(out.get("dg")), _ptr(out["dS0"]), B, T, H, Dk, Dv, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle failed with code {rc}")
    return out


def kda_bwd_ref(q, k, v, beta, gk, do, S0=None, dS_T=None, nthreads: int = 1):
    """Gradients of L = sum <do, o> + <dS_T, S_T> through the per-channel-decay
    recurrence of ``kda_ref`` in fp64 on the CPU (``ref_delta_rule_bwd.c``,
    ``ref_kda_bwd_f64``).  gk is ``[B,T,H,Dk]``; the rest as
    ``delta_rule_bwd_ref``.  Returns a dict with dq, dk, dv, dbeta, dgk
    ([B,T,H,Dk]) and dS0."""
    q, k, v, beta, s0, (B, T, H, Dk, Dv) = _check(q, k, v, beta, S0)
    gk = _as_f64(gk)
    if gk.shape != (B, T, H, Dk):
        raise ValueError(f"gk must be [B,T,H,Dk]={B, T, H, Dk}, got {gk.shape}")
    do = _as_f64(do)
    if do.shape != (B, T, H, Dv):
        raise ValueError(f"do must be [B,T,H,Dv]={B, T, H, Dv}, got {do.shape}")
    dst = None
    if dS_T is not None:
        dst = _as_f64(dS_T)
        if dst.shape != (B, H, Dv, Dk):
            raise ValueError(f"dS_T must be [B,H,Dv,Dk]={B, H, Dv, Dk}, got {dst.shape}")
    out = {"dq": np.zeros((B, T, H, Dk)), "dk": np.zeros((B, T, H, Dk)),
           "dv": np.zeros((B, T, H, Dv)), "dbeta": np.zeros((B, T, H)),
           "dgk": np.zeros((B, T, H, Dk)), "dS0": np.zeros((B, H, Dv, Dk))}
    rc = _load().ref_kda_bwd_f64(
        _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(gk), _ptr(s0), _ptr(do), _ptr(dst),
        _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dbeta"]),
        _ptr(out["dgk"]), _ptr(out["dS0"]), B, T, H, Dk, Dv, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle failed with code {rc}")
    return out


def l2norm_rows(x, eps: float = 1e-6):
    """Each row (last axis) of x divided by sqrt(sum of its squares + eps),
    in fp64: the l2norm helper of the gated layer on houmin.site
    ("infra/delta-net", section "Gated DeltaNet", code), which the DeltaNet
    layer applies to q and k (fla/layers/delta_net.py, the l2 norm option)."""
    x = _as_f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


__all__ = ["build", "delta_rule_ref", "gated_delta_rule_ref", "kda_ref", "delta_rule_bwd_ref",
           "kda_bwd_ref", "l2norm_rows"]
