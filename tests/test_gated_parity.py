"""GPU parity of the gated rule (scalar forget gate alpha = exp(g)) against
the fp64 gated oracle.

The same seeded inputs go to ``gated_delta_rule_chunk_fwd`` /
``gated_delta_rule_recurrent_step`` (through the C ABI) and to the oracle,
with the tolerances of the plain rule: max |gpu - ref| <= tol * max |ref|,
tol = 1e-4 for fp32 inputs and 2e-2 for bf16 inputs, for the outputs and the
final state separately.  The gates follow the gated layer's draw (per-head
A ~ U(0, gate_amax), g = -A softplus(a + 1)); a small gate_amax keeps memory
over many chunks, the pages' 16 forgets within a few tokens on most heads.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import deltanet_delta_rule_amd as dr
from deltanet_delta_rule_amd import workloads as W
from tests.parity_utils import (TOL, gather_heads, oracle_all, oracle_heads, rel_err, to_dev,
                                to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    dr.load_library()


def _gated(name, **kw):
    kw.setdefault("gate_amax", 1.0)
    return W.get(name, **kw)


def _chunk_check(w: W.Workload, heads=None, x=None):
    x = W.generate(w) if x is None else x
    d = to_dev(x)
    o, st = dr.gated_delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["S0"],
                                          chunk=w.chunk)
    torch.cuda.synchronize()
    if heads is None:
        o_ref, s_ref = oracle_all(x)
        o_got, s_got = to_np(o), to_np(st)
    else:
        o_ref, s_ref = oracle_heads(x, heads)
        o_got, s_got = gather_heads(o, st, heads)
    tol = TOL[w.torch_dtype]
    eo, es = rel_err(o_got, o_ref), rel_err(s_got, s_ref)
    print(f"gated {w.name} B{w.B} H{w.H} T{w.T} Dk{w.Dk} Dv{w.Dv} C{w.chunk} {w.dtype} "
          f"Amax{w.gate_amax:g}: o err {eo:.3e}  S_T err {es:.3e}  (tol {tol:g})", flush=True)
    assert eo <= tol, f"o relative error {eo:.3e} > {tol}"
    assert es <= tol, f"S_T relative error {es:.3e} > {tol}"
    return x, o, st


# ---------------------------------------------------------------- chunk path
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Dk", [16, 32, 64, 128])
@pytest.mark.parametrize("Dv", [16, 64, 128])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_gated_chunk_shape_grid(dtype, Dk, Dv, chunk):
    w = _gated("long_prefill", B=2, H=2, T=3 * chunk - 5, Dk=Dk, Dv=Dv, chunk=chunk,
               dtype=dtype, seed=5000 + Dk + 7 * Dv + chunk)
    _chunk_check(w)


@pytest.mark.parametrize("amax", [0.02, 0.3, 16.0])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gated_chunk_decay_strengths(amax, dtype):
    # from memory over the whole sequence to forgetting within a token
    _chunk_check(_gated("long_prefill", H=4, T=333, dtype=dtype, gate_amax=amax,
                        seed=5100 + int(100 * amax)))


@pytest.mark.parametrize("T", [1, 5, 63, 64, 65, 129])
def test_gated_chunk_sequence_lengths(T):
    _chunk_check(_gated("layer_1p3b", B=2, H=2, T=T, seed=5200 + T))


def test_gated_chunk_many_heads_fill_grid():
    _chunk_check(_gated("gated_layer_1p3b", T=70), heads=[(0, 0), (3, 7), (7, 15)])


def test_gated_chunk_full_layer_1p3b():
    # the benchmark's gated launch, whole heads sampled across the batch
    heads = [(0, 0), (1, 5), (2, 10), (3, 15), (4, 3), (5, 8), (6, 13), (7, 15)]
    w = W.get("gated_layer_1p3b")
    _chunk_check(w, heads=heads)


def test_gated_chunk_zero_gate_resets_the_state():
    # exp(-30) ~ 1e-13: the state from before the reset no longer counts
    w = _gated("long_prefill", H=2, T=200, gate_amax=0.1)
    x = W.generate(w)
    x["g"][:, 77] = -30.0
    _chunk_check(w, x=x)


def test_gated_chunk_log_gate_zero_is_the_plain_rule():
    w = W.get("long_prefill", H=2, T=150)
    x = W.generate(w)
    d = to_dev(x)
    g0 = torch.zeros(d["beta"].shape, dtype=torch.float32, device="cuda")
    o_g, s_g = dr.gated_delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], g0, d["S0"])
    o_p, s_p = dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["S0"])
    o_ref, s_ref = oracle_all(x)
    for got in (o_g, o_p):
        assert rel_err(to_np(got), o_ref) <= 2e-2
    assert rel_err(to_np(s_g), s_ref) <= 2e-2
    # the two kernels differ only in rounding order
    assert rel_err(to_np(o_g), to_np(o_p)) <= 1e-2


def test_gated_chunk_empty_sequence_copies_state():
    w = _gated("long_prefill", H=3, T=0)
    x = to_dev(W.generate(w))
    o, st = dr.gated_delta_rule_chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["S0"])
    assert o.shape == (1, 0, 3, 128)
    torch.testing.assert_close(st, x["S0"], rtol=0, atol=0)


def test_gated_chunk_resume_matches_single_call():
    w = _gated("long_prefill", H=2, T=256)
    d = to_dev(W.generate(w))
    o, st = dr.gated_delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["S0"])
    cut = 128
    sl = lambda t, a, b: t[:, a:b].contiguous()
    part = lambda a, b, s: dr.gated_delta_rule_chunk_fwd(
        sl(d["q"], a, b), sl(d["k"], a, b), sl(d["v"], a, b), sl(d["beta"], a, b),
        sl(d["g"], a, b), s)
    o1, s1 = part(0, cut, d["S0"])
    o2, s2 = part(cut, 256, s1)
    torch.testing.assert_close(torch.cat([o1, o2], 1), o, rtol=0, atol=0)
    torch.testing.assert_close(s2, st, rtol=0, atol=0)


def test_gated_chunk_writes_every_output_and_nothing_else():
    w = _gated("long_prefill", B=2, H=2, T=97)
    d = to_dev(W.generate(w))
    G = 64
    n_o, n_s = 2 * 97 * 2 * 128, 2 * 2 * 128 * 128
    obuf = torch.full((n_o + 2 * G,), float("nan"), dtype=torch.bfloat16, device="cuda")
    sbuf = torch.full((n_s + 2 * G,), float("nan"), dtype=torch.float32, device="cuda")
    o = obuf[G:G + n_o].view(2, 97, 2, 128)
    st = sbuf[G:G + n_s].view(2, 2, 128, 128)
    dr.gated_delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["S0"], o=o,
                                  S_T=st)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any() and not torch.isnan(st).any()
    assert torch.isnan(obuf[:G]).all() and torch.isnan(obuf[-G:]).all()
    assert torch.isnan(sbuf[:G]).all() and torch.isnan(sbuf[-G:]).all()


# --------------------------------------------------------------- decode path
def _decode_check(w: W.Workload, heads=None):
    x = W.generate(w)
    d = to_dev(x)
    S = d["S0"].clone()
    outs = [dr.gated_delta_rule_recurrent_step(d["q"][t], d["k"][t], d["v"][t], d["beta"][t],
                                               d["g"][t], S) for t in range(w.T)]
    torch.cuda.synchronize()
    o = torch.stack(outs)
    # step-major [steps, B, H, .] inputs read as [B, steps, H, .] sequences
    seq = {n: (None if t is None else (t.transpose(0, 1).contiguous() if n != "S0" else t))
           for n, t in x.items()}
    o_seq = o.transpose(0, 1)
    if heads is None:
        o_ref, s_ref = oracle_all(seq)
        o_got, s_got = to_np(o_seq), to_np(S)
    else:
        o_ref, s_ref = oracle_heads(seq, heads)
        o_got, s_got = gather_heads(o_seq, S, heads)
    tol = TOL[w.torch_dtype]
    eo, es = rel_err(o_got, o_ref), rel_err(s_got, s_ref)
    print(f"gated decode B{w.B} H{w.H} Dk{w.Dk} Dv{w.Dv} steps{w.T} {w.dtype}: o err {eo:.3e} "
          f"S err {es:.3e}", flush=True)
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Dk", [16, 64, 128])
@pytest.mark.parametrize("Dv", [16, 128])
def test_gated_decode_small(dtype, Dk, Dv):
    _decode_check(_gated("decode", B=3, H=2, T=12, Dk=Dk, Dv=Dv, dtype=dtype,
                         seed=5300 + Dk + Dv))


def test_gated_decode_full_size_sampled_heads():
    heads = [(b, h) for b in (0, 64, 127) for h in (0, 7, 15)]
    _decode_check(W.get("gated_decode", T=64), heads=heads)


def test_gated_decode_matches_chunk_path():
    w = _gated("long_prefill", B=2, H=3, T=40, gate_amax=0.5)
    d = to_dev(W.generate(w))
    o_c, s_c = dr.gated_delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"],
                                             d["S0"])
    S = d["S0"].clone()
    col = lambda t, i: t[:, i].contiguous()
    o_d = torch.stack([dr.gated_delta_rule_recurrent_step(col(d["q"], t), col(d["k"], t),
                                                          col(d["v"], t), col(d["beta"], t),
                                                          col(d["g"], t), S)
                       for t in range(40)], dim=1)
    assert rel_err(to_np(o_d), to_np(o_c)) <= 2e-2
    assert rel_err(to_np(S), to_np(s_c)) <= 2e-2
