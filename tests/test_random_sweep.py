"""Seeded random sweep of the GPU paths against the fp64 oracle.

Forty forward cases, sixteen backward cases and ten cases of the KDA
backward (with an output scale drawn half the time), drawn once from fixed seeds
over the supported space -- the rule (plain, gated with per-head A up to 16,
KDA with per-channel decay), the dtype, d_k and d_v in {16, 32, 64, 128}, the
chunk, batch, heads, sequence length (ragged tails included), beta in (0, 1)
or (0, 2), a zero or nonzero initial state, the output scale and the in-kernel
L2 norm -- each checked against the oracle with the tolerance of the other
parity tests (max |gpu - ref| <= tol * max |ref|, 1e-4 fp32 / 2e-2 bf16; the
gate gradient against max(max |dg|, max |dbeta|), see grad_errors).
The point is breadth: combinations no hand-written case names.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import deltanet_delta_rule_amd as dr
from deltanet_delta_rule_amd import workloads as W
from oracle import (delta_rule_bwd_ref, delta_rule_ref, gated_delta_rule_ref, kda_bwd_ref,
                    kda_ref, l2norm_rows)
from tests.parity_utils import TOL, grad_errors, rel_err, threads, to_dev, to_np

pytestmark = pytest.mark.gpu

DIMS = [16, 32, 64, 128]


def _draw(n, seed, backward=False):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        rule = str(rng.choice(["plain", "gated"] if backward else ["plain", "gated", "kda"]))
        c = dict(
            rule=rule,
            dtype=str(rng.choice(["bf16", "bf16", "f32"])),
            Dk=int(rng.choice(DIMS)), Dv=int(rng.choice(DIMS)),
            chunk=int(rng.choice([16, 32, 64])),
            B=int(rng.integers(1, 4)), H=int(rng.integers(1, 5)),
            T=int(rng.integers(1, 301)),
            beta_scale=float(rng.choice([1.0, 2.0])),
            s0_std=float(rng.choice([0.0, 0.02])),
            seed=20000 + 97 * i + (5000 if backward else 0))
        if not backward:
            c["scale"] = None if rng.random() < 0.6 else float(rng.uniform(0.1, 2.0))
            c["l2"] = bool(rng.random() < 0.25)
        if rule == "kda" and rng.random() < 0.5:  # the chunked KDA kernel's shapes
            c.update(dtype="bf16", Dk=128, Dv=int(rng.choice([64, 128])))
        cases.append(c)
    return cases


FWD = _draw(40, 123)
BWD = _draw(16, 456, backward=True)


def _draw_kda_bwd(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        cases.append(dict(
            rule="kda", dtype=str(rng.choice(["bf16", "bf16", "f32"])),
            Dk=int(rng.choice(DIMS)), Dv=int(rng.choice(DIMS)), chunk=32,
            B=int(rng.integers(1, 4)), H=int(rng.integers(1, 5)), T=int(rng.integers(1, 301)),
            beta_scale=float(rng.choice([1.0, 2.0])), s0_std=float(rng.choice([0.0, 0.02])),
            scale=None if rng.random() < 0.5 else float(rng.uniform(0.1, 2.0)),
            seed=40000 + 97 * i))
    return cases


KBWD = _draw_kda_bwd(10, 789)


def _id(c):
    return (f"{c['rule']}-{c['dtype']}-k{c['Dk']}v{c['Dv']}-C{c['chunk']}-B{c['B']}H{c['H']}"
            f"T{c['T']}-b{c['beta_scale']:g}-s{c['s0_std']:g}"
            + ("-sc" if c.get("scale") else "") + ("-l2" if c.get("l2") else ""))


def _workload(c):
    kw = dict(B=c["B"], H=c["H"], T=c["T"], Dk=c["Dk"], Dv=c["Dv"], chunk=c["chunk"],
              dtype=c["dtype"], beta_scale=c["beta_scale"], s0_std=c["s0_std"],
              seed=c["seed"], feature="raw" if c.get("l2") else "l2")
    if c["rule"] == "gated":
        kw.update(gate_amax=16.0)
    elif c["rule"] == "kda":
        kw.update(gate_amax=16.0, kda=True)
    return W.get("layer_1p3b", **kw)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    dr.load_library()


@pytest.mark.parametrize("c", FWD, ids=_id)
def test_forward_random_case(c):
    w = _workload(c)
    x = W.generate(w)
    d = to_dev(x)
    opts = dict(scale=c["scale"], use_qk_l2norm_in_kernel=c["l2"])
    if c["rule"] == "plain":
        o, st = dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["S0"],
                                        chunk=c["chunk"], **opts)
    elif c["rule"] == "gated":
        o, st = dr.gated_delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"],
                                              d["S0"], chunk=c["chunk"], **opts)
    else:
        o, st = dr.kda_fwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], d["S0"], **opts)
    torch.cuda.synchronize()
    q, k = x["q"], x["k"]
    if c["l2"]:
        q, k = l2norm_rows(q), l2norm_rows(k)
    if c["rule"] == "plain":
        o_ref, s_ref = delta_rule_ref(q, k, x["v"], x["beta"], x["S0"], nthreads=threads())
    elif c["rule"] == "gated":
        o_ref, s_ref = gated_delta_rule_ref(q, k, x["v"], x["beta"], x["g"], x["S0"],
                                            nthreads=threads())
    else:
        o_ref, s_ref = kda_ref(q, k, x["v"], x["beta"], x["gk"], x["S0"], nthreads=threads())
    if c["scale"] is not None:
        o_ref = o_ref * c["scale"]
    tol = TOL[w.torch_dtype]
    eo, es = rel_err(to_np(o), o_ref), rel_err(to_np(st), s_ref)
    print(f"{_id(c)}: o {eo:.2e} S_T {es:.2e}", flush=True)
    assert eo <= tol and es <= tol, (eo, es)


@pytest.mark.parametrize("c", BWD, ids=_id)
def test_backward_random_case(c):
    w = _workload(c)
    x = W.generate(w)
    d = to_dev(x)
    gen = torch.Generator().manual_seed(c["seed"] + 1)
    do = torch.randn(w.B, w.T, w.H, w.Dv, generator=gen).to(w.torch_dtype)
    dst = torch.randn(w.B, w.H, w.Dv, w.Dk, generator=gen)
    if c["rule"] == "plain":
        got = dr.delta_rule_chunk_bwd(d["q"], d["k"], d["v"], d["beta"], do.cuda(), d["S0"],
                                      dst.cuda())
    else:
        got = dr.gated_delta_rule_chunk_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"],
                                            do.cuda(), d["S0"], dst.cuda())
    torch.cuda.synchronize()
    ref = delta_rule_bwd_ref(x["q"], x["k"], x["v"], x["beta"], do, x["S0"], dst,
                             g=x.get("g"), nthreads=threads())
    tol = TOL[w.torch_dtype]
    errs = grad_errors(got, ref)
    print(f"{_id(c)}: " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
    for n, e in errs.items():
        assert e <= tol, (n, e)


@pytest.mark.parametrize("c", KBWD, ids=_id)
def test_kda_backward_random_case(c):
    w = _workload(c)
    x = W.generate(w)
    d = to_dev(x)
    gen = torch.Generator().manual_seed(c["seed"] + 1)
    do = torch.randn(w.B, w.T, w.H, w.Dv, generator=gen).to(w.torch_dtype)
    dst = torch.randn(w.B, w.H, w.Dv, w.Dk, generator=gen)
    got = dr.kda_bwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], do.cuda(), d["S0"], dst.cuda(),
                     scale=c["scale"])
    torch.cuda.synchronize()
    # <do, scale S q> = <scale do, S q>: the oracle takes the scaled upstream gradient
    do_o = do.double() * (1.0 if c["scale"] is None else c["scale"])
    ref = kda_bwd_ref(x["q"], x["k"], x["v"], x["beta"], x["gk"], do_o, x["S0"], dst,
                      nthreads=threads())
    tol = TOL[w.torch_dtype]
    errs = {n: rel_err(to_np(got[n]), ref[n]) for n in ref}
    print(f"{_id(c)}: " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
    for n, e in errs.items():
        assert e <= tol, (n, e)
