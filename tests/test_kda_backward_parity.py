"""GPU parity of the per-channel-decay backward (``kda_bwd``) against the fp64
oracle ``oracle.kda_bwd_ref``.

Seeded inputs and seeded upstream gradients (do, dS_T) go to the HIP path and
to the oracle; every gradient (dq, dk, dv, dbeta, dgk, dS0) must satisfy
max |gpu - ref| <= tol * max |ref|, tol = 1e-4 for fp32 inputs and 2e-2 for
bf16 inputs (the forward's tolerances).  Cases: every head size, lengths
that span several 16-token blocks with ragged tails, decays from near 1 to
the gated layer's draw with A up to 16 and channels erased within one token
(hada.io digest, section "Kimi Delta Attention : attenuation par canal": a
channel can be wiped while another keeps its content), an output scale,
packed sequences, an empty sequence, and the layer shape with whole heads
sampled.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import deltanet_delta_rule_amd as dr
from deltanet_delta_rule_amd import workloads as W
from oracle import kda_bwd_ref
from tests.parity_utils import TOL, rel_err, threads, to_dev, to_np

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dbeta", "dgk", "dS0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    dr.load_library()


def _kda(name="long_prefill", **kw):
    kw.setdefault("gate_amax", 1.0)
    kw["kda"] = True
    return W.get(name, **kw)


def _upstream(B, T, H, Dk, Dv, dtype, seed, with_dst=True):
    gen = torch.Generator().manual_seed(seed)
    do = torch.randn(B, T, H, Dv, generator=gen).to(dtype)
    dst = torch.randn(B, H, Dv, Dk, generator=gen) if with_dst else None
    return do, dst


def _errors(got, ref):
    return {n: rel_err(to_np(got[n]), ref[n]) for n in NAMES}


def _check(w, seed=7, with_dst=True, heads=None, x=None, scale=None):
    x = W.generate(w) if x is None else x
    do, dst = _upstream(w.B, w.T, w.H, w.Dk, w.Dv, w.torch_dtype, seed, with_dst)
    d = to_dev(x)
    g = dr.kda_bwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], do.cuda(), d["S0"],
                   None if dst is None else dst.cuda(), scale=scale)
    torch.cuda.synchronize()
    if heads is not None:
        pick = lambda t: torch.stack([t[b, :, h] for b, h in heads], dim=1)[None]
        pick_s = lambda t: torch.stack([t[b, h] for b, h in heads])[None]
        xs = {n: (None if t is None else (pick_s(t) if n == "S0" else pick(t)))
              for n, t in x.items()}
        do_r, dst_r = pick(do), (None if dst is None else pick_s(dst))
        got = {n: (pick_s(t) if n == "dS0" else pick(t)) for n, t in g.items()}
    else:
        xs, do_r, dst_r, got = x, do, dst, g
    # the oracle reads o = S q; <do, scale S q> = <scale do, S q>, so the
    # scaled upstream gradient gives every gradient of the scaled forward
    do_o = do_r.double() * (1.0 if scale is None else scale)
    ref = kda_bwd_ref(xs["q"], xs["k"], xs["v"], xs["beta"], xs["gk"], do_o, xs["S0"], dst_r,
                      nthreads=threads())
    errs = _errors(got, ref)
    tol = TOL[w.torch_dtype]
    print(f"kda bwd B{w.B} H{w.H} T{w.T} Dk{w.Dk} Dv{w.Dv} {w.dtype} "
          f"Amax{w.gate_amax:g}: " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()),
          flush=True)
    for n, e in errs.items():
        assert e <= tol, f"{n}: relative error {e:.3e} > {tol}"
    return g, ref


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Dk,Dv", [(16, 16), (32, 64), (64, 32), (64, 128), (128, 64),
                                   (128, 128)])
def test_shapes(dtype, Dk, Dv):
    _check(_kda(B=2, H=2, T=77, Dk=Dk, Dv=Dv, dtype=dtype, seed=20000 + Dk + 3 * Dv),
           seed=Dk + Dv)


@pytest.mark.parametrize("T", [1, 15, 16, 17, 33, 100])
def test_lengths(T):
    _check(_kda("layer_1p3b", B=2, H=2, T=T, seed=20100 + T), seed=T)


@pytest.mark.parametrize("amax", [0.02, 1.0, 16.0])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decay_strengths(amax, dtype):
    _check(_kda(H=3, T=90, gate_amax=amax, dtype=dtype, seed=20200 + int(100 * amax)))


@pytest.mark.parametrize("dtype,Dk,Dv,B,H", [("f32", 64, 64, 2, 130), ("bf16", 128, 128, 1, 70),
                                              ("f32", 128, 64, 1, 130), ("bf16", 128, 128, 1, 40),
                                              ("f32", 64, 128, 1, 70)])
def test_many_heads(dtype, Dk, Dv, B, H):
    # the workgroup shapes by count: more (sequence, head, row tile) than the
    # GPU has CUs at one row per lane takes two rows per lane (the first
    # three cases); 129 .. 256 one row on 512 lanes (the last two); fewer,
    # as in the other tests, one row on 256 lanes
    _check(_kda(B=B, H=H, T=40, Dk=Dk, Dv=Dv, dtype=dtype, gate_amax=16.0,
                seed=21000 + H + Dk), seed=H)


def test_erased_channels():
    # a third of the tokens erase every other channel; a quarter of the
    # channels are erased outright at one token (exp(-inf) = 0)
    w = _kda(H=2, T=70, Dk=64, Dv=64, dtype="f32", gate_amax=1.0, seed=20300)
    x = W.generate(w)
    x["gk"][:, ::3, :, ::2] = -1e4
    x["gk"][:, 40, :, 1::4] = float("-inf")
    g, _ = _check(w, x=x)
    assert torch.isfinite(g["dgk"]).all() and torch.isfinite(g["dq"]).all()


def test_without_initial_state_or_state_gradient():
    _check(_kda(B=2, H=2, T=50, Dk=64, Dv=64, dtype="f32", s0_std=0.0, seed=20400),
           with_dst=False)


def test_output_scale():
    w = _kda(B=1, H=2, T=40, Dk=64, Dv=64, dtype="f32", seed=20500)
    _check(w, scale=0.125)


def test_shared_decay_matches_the_gated_backward():
    # one log decay for every channel is the gated rule: same dq, dk, dv,
    # dbeta, dS0, and dg = sum over channels of dgk
    w = _kda(B=1, H=2, T=64, Dk=64, Dv=64, dtype="f32", seed=20600)
    x = W.generate(w)
    g1 = x["gk"][..., :1].expand_as(x["gk"]).contiguous()
    x["gk"] = g1
    d = to_dev(x)
    do, dst = _upstream(w.B, w.T, w.H, w.Dk, w.Dv, w.torch_dtype, 3)
    kb = dr.kda_bwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], do.cuda(), d["S0"], dst.cuda())
    gb = dr.gated_delta_rule_chunk_bwd(d["q"], d["k"], d["v"], d["beta"],
                                       d["gk"][..., 0].contiguous(), do.cuda(), d["S0"],
                                       dst.cuda())
    torch.cuda.synchronize()
    for n in ("dq", "dk", "dv", "dbeta", "dS0"):
        e = rel_err(to_np(kb[n]), to_np(gb[n]))
        assert e <= 2e-4, f"{n}: {e:.2e}"
    e = rel_err(to_np(kb["dgk"].sum(-1)), to_np(gb["dg"]))
    assert e <= 2e-4, f"dg: {e:.2e}"


def test_packed_sequences():
    lengths = [0, 1, 17, 33, 64, 5]
    T = sum(lengths) + 7  # seven trailing tokens in no sequence
    H, Dk, Dv = 2, 64, 64
    w = _kda(B=1, H=H, T=T, Dk=Dk, Dv=Dv, dtype="f32", seed=20700)
    x = W.generate(w)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    n = len(lengths)
    gen = torch.Generator().manual_seed(11)
    S0 = 0.1 * torch.randn(n, H, Dv, Dk, generator=gen)
    dst = torch.randn(n, H, Dv, Dk, generator=gen)
    do = torch.randn(1, T, H, Dv, generator=gen)
    d = to_dev(x)
    g = dr.kda_bwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], do.cuda(), S0.cuda(), dst.cuda(),
                   cu_seqlens=cu.cuda())
    torch.cuda.synchronize()
    for s, L in enumerate(lengths):
        a, b = int(cu[s]), int(cu[s + 1])
        if L == 0:
            assert torch.equal(g["dS0"][s].cpu(), dst[s])
            continue
        sl = lambda t: t[:, a:b]
        ref = kda_bwd_ref(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["beta"]), sl(x["gk"]),
                          sl(do), S0[s:s + 1], dst[s:s + 1])
        got = {nm: (g[nm][s:s + 1] if nm == "dS0" else g[nm][:, a:b]) for nm in NAMES}
        for nm, e in _errors(got, ref).items():
            assert e <= 1e-4, f"sequence {s} (length {L}): {nm} relative error {e:.2e}"
    # tokens in no sequence get zero gradients
    for nm in ("dq", "dk", "dv", "dbeta", "dgk"):
        assert torch.count_nonzero(g[nm][:, sum(lengths):]) == 0, nm


def test_empty_sequence():
    w = _kda(B=2, H=2, T=0, Dk=64, Dv=64, dtype="f32", seed=20800)
    x = W.generate(w)
    d = to_dev(x)
    dst = torch.randn(2, 2, 64, 64)
    do = torch.zeros(2, 0, 2, 64)
    g = dr.kda_bwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], do.cuda(), d["S0"], dst.cuda())
    torch.cuda.synchronize()
    assert torch.equal(g["dS0"].cpu(), dst)


def test_without_the_state_gradient_output():
    # dS0 not requested: nothing written for it, the other gradients the same
    w = _kda(B=1, H=2, T=40, Dk=128, Dv=128, dtype="bf16", seed=20950)
    x = W.generate(w)
    d = to_dev(x)
    do, dst = _upstream(w.B, w.T, w.H, w.Dk, w.Dv, w.torch_dtype, 9)
    a = dr.kda_bwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], do.cuda(), d["S0"], dst.cuda())
    b = dr.kda_bwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], do.cuda(), d["S0"], dst.cuda(),
                   need_dS0=False)
    torch.cuda.synchronize()
    assert b["dS0"] is None
    for n in ("dq", "dk", "dv", "dbeta", "dgk"):
        assert torch.equal(a[n], b[n]), n


def test_repeated_calls_are_bit_identical():
    w = _kda(B=2, H=3, T=45, Dk=128, Dv=128, dtype="bf16", seed=20900)
    x = W.generate(w)
    d = to_dev(x)
    do, dst = _upstream(w.B, w.T, w.H, w.Dk, w.Dv, w.torch_dtype, 5)
    a = dr.kda_bwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], do.cuda(), d["S0"], dst.cuda())
    b = dr.kda_bwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], do.cuda(), d["S0"], dst.cuda())
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(a[n], b[n]), n


def test_layer_shape_sampled_heads():
    # the layer shape (B=8, H=16, T=2048, d=128, bf16; decays with A up to 16)
    # in the launch the benchmark times, whole heads compared to the oracle
    w = W.get("layer_1p3b", gate_amax=16.0, kda=True)
    _check(w, heads=[(0, 0), (3, 7), (7, 15)])
