"""GPU parity of the KDA decode step (per-key-channel decay, ``kda_recurrent_step``)
against the fp64 KDA oracle.

hada.io digest, section "Kimi Delta Attention : attenuation par canal": before
each token, column j of the state is multiplied by exp(gk[j]).  Seeded
step-major inputs go to the HIP path one token at a time and, read as
sequences, to ``oracle.kda_ref``; outputs and the final state must satisfy
max |gpu - ref| <= tol * max |ref|, tol = 1e-4 for fp32 inputs and 2e-2 for
bf16 inputs.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import deltanet_delta_rule_amd as dr
from deltanet_delta_rule_amd import workloads as W
from tests.parity_utils import TOL, gather_heads, oracle_all, oracle_heads, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    dr.load_library()


def _kda(name="decode", **kw):
    kw.setdefault("gate_amax", 1.0)
    kw.setdefault("kda", True)
    return W.get(name, **kw)


def _decode(d, T, S, **kw):
    outs = [dr.kda_recurrent_step(d["q"][t], d["k"][t], d["v"][t], d["beta"][t], d["gk"][t], S,
                                  **kw) for t in range(T)]
    torch.cuda.synchronize()
    return torch.stack(outs)


def _decode_check(w: W.Workload, heads=None, x=None, **kw):
    x = W.generate(w) if x is None else x
    d = to_dev(x)
    S = d["S0"].clone() if d["S0"] is not None else torch.zeros(
        w.B, w.H, w.Dv, w.Dk, device="cuda")
    o = _decode(d, w.T, S, **kw)
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
    print(f"kda decode B{w.B} H{w.H} Dk{w.Dk} Dv{w.Dv} steps{w.T} {w.dtype} "
          f"Amax{w.gate_amax:g}: o err {eo:.3e} S err {es:.3e}", flush=True)
    assert eo <= tol and es <= tol
    return x, o, S


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Dk", [16, 32, 64, 128])
@pytest.mark.parametrize("Dv", [16, 128])
def test_kda_decode_small(dtype, Dk, Dv):
    _decode_check(_kda(B=3, H=2, T=12, Dk=Dk, Dv=Dv, dtype=dtype, seed=8000 + Dk + Dv))


@pytest.mark.parametrize("amax", [0.05, 16.0])
def test_kda_decode_decay_strengths(amax):
    _decode_check(_kda(B=2, H=4, T=40, gate_amax=amax, seed=8100 + int(amax)))


def test_kda_decode_full_size_sampled_heads():
    heads = [(b, h) for b in (0, 64, 127) for h in (0, 7, 15)]
    _decode_check(W.get("kda_decode", T=64), heads=heads)


def test_kda_decode_with_scale():
    w = _kda(B=2, H=3, T=10, seed=8200)
    x = W.generate(w)
    d = to_dev(x)
    S = d["S0"].clone()
    o = _decode(d, w.T, S, scale=0.125)
    seq = {n: (None if t is None else (t.transpose(0, 1).contiguous() if n != "S0" else t))
           for n, t in x.items()}
    o_ref, s_ref = oracle_all(seq)
    assert rel_err(to_np(o.transpose(0, 1)), 0.125 * o_ref) <= 2e-2
    assert rel_err(to_np(S), s_ref) <= 2e-2


def test_kda_decode_equal_channels_is_the_gated_step():
    # one decay on every channel is the gated rule's scalar gate
    w = W.get("decode", B=4, H=2, T=6, gate_amax=1.0, seed=8300)
    d = to_dev(W.generate(w))
    S_g, S_k = d["S0"].clone(), d["S0"].clone()
    for t in range(w.T):
        gk = d["g"][t][..., None].expand(-1, -1, w.Dk).contiguous()
        o_g = dr.gated_delta_rule_recurrent_step(d["q"][t], d["k"][t], d["v"][t], d["beta"][t],
                                                 d["g"][t], S_g)
        o_k = dr.kda_recurrent_step(d["q"][t], d["k"][t], d["v"][t], d["beta"][t], gk, S_k)
        torch.testing.assert_close(o_k, o_g, rtol=0, atol=0)
    torch.testing.assert_close(S_k, S_g, rtol=0, atol=0)


def test_kda_decode_rejects_both_decays():
    w = _kda(B=1, H=1, T=1)
    d = to_dev(W.generate(w))
    with pytest.raises((ValueError, RuntimeError)):
        dr._step_call(True, d["q"][0], d["k"][0], d["v"][0], d["beta"][0],
                      torch.zeros(1, 1, device="cuda"), d["S0"].clone(), None, None,
                      gk=d["gk"][0])
