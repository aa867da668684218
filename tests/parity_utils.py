"""Helpers shared by the GPU parity tests: run the HIP path and the fp64
oracle on the same seeded inputs and measure the error the way the tolerance
is stated -- max |gpu - ref| relative to max |ref| -- for o and the final
state separately."""
from __future__ import annotations

import os

import numpy as np
import torch

from oracle import delta_rule_ref, gated_delta_rule_ref, kda_ref

# fp32 inputs: 1e-4; bf16 inputs: 2e-2 (fp32 state), both relative to max|ref|.
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    den = np.max(np.abs(ref))
    if not np.all(np.isfinite(got)):
        return float("inf")
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def to_np(t):
    return t.detach().to("cpu").double().numpy()


def oracle_heads(x, heads):
    """Oracle on a subset of (b, h) pairs of a chunk workload's inputs (the
    gated oracle when the inputs carry log gates g, the KDA oracle when they
    carry per-channel log decays gk).

    Returns (o [T, n, Dv], S_T [n, Dv, Dk]) for the n pairs in `heads`, by
    stacking the selected heads into one batch row (heads are independent).
    """
    sel = lambda t: np.stack([to_np(t[b, :, h]) for b, h in heads], axis=1)[None]
    q, k, v = sel(x["q"]), sel(x["k"]), sel(x["v"])
    beta = sel(x["beta"])
    S0 = None
    if x["S0"] is not None:
        S0 = np.stack([x["S0"][b, h].double().numpy() for b, h in heads])[None]
    if x.get("gk") is not None:
        o, st = kda_ref(q, k, v, beta, sel(x["gk"]), S0, nthreads=threads())
    elif x.get("g") is not None:
        o, st = gated_delta_rule_ref(q, k, v, beta, sel(x["g"]), S0, nthreads=threads())
    else:
        o, st = delta_rule_ref(q, k, v, beta, S0, nthreads=threads())
    return o[0], st[0]


def oracle_all(x):
    """Oracle on every head of a chunk workload's inputs (gated when g is set,
    KDA when gk is set)."""
    if x.get("gk") is not None:
        return kda_ref(x["q"], x["k"], x["v"], x["beta"], x["gk"], x["S0"], nthreads=threads())
    if x.get("g") is not None:
        return gated_delta_rule_ref(x["q"], x["k"], x["v"], x["beta"], x["g"], x["S0"],
                                    nthreads=threads())
    return delta_rule_ref(x["q"], x["k"], x["v"], x["beta"], x["S0"], nthreads=threads())


def gather_heads(o_gpu, st_gpu, heads):
    o = np.stack([to_np(o_gpu[b, :, h]) for b, h in heads], axis=1)
    st = np.stack([to_np(st_gpu[b, h]) for b, h in heads])
    return o, st


def to_dev(x, device="cuda"):
    return {n: (None if t is None else t.to(device)) for n, t in x.items()}


def grad_errors(got: dict, ref: dict) -> dict:
    """Relative errors of the backward's gradients, each against max |ref| of
    that gradient, except dg: the gate gradient of a token is a difference of
    products of the chunk's operands (the same products whose row sums make
    dbeta), so where the gates have decayed everything it cancels to a value
    far below those products and their fp32 rounding.  Its error is measured
    against max(max |dg|, max |dbeta|)."""
    errs = {n: rel_err(to_np(got[n]), ref[n]) for n in ref}
    if "dg" in ref:
        scale = max(float(np.max(np.abs(ref["dg"]))) if ref["dg"].size else 0.0,
                    float(np.max(np.abs(ref["dbeta"]))) if ref["dbeta"].size else 0.0)
        diff = np.abs(to_np(got["dg"]) - np.asarray(ref["dg"], dtype=np.float64))
        errs["dg"] = float(np.max(diff) / scale) if diff.size and scale > 0 else errs["dg"]
    return errs

