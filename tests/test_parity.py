"""GPU parity of the HIP path against the fp64 oracle.

Every case feeds the same seeded, dtype-rounded inputs to
``delta_rule_chunk_fwd`` / ``delta_rule_recurrent_step`` (through the C ABI)
and to the oracle, then checks max |gpu - ref| <= tol * max |ref| for the
outputs and, separately, the final state: tol = 1e-4 for fp32 inputs and
2e-2 for bf16 inputs (fp32 state in both).  Small cases span several chunks
and a ragged tail; full-size cases run the exact launch the benchmark times
and compare whole heads chosen across the batch.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import deltanet_delta_rule_amd as dr
from deltanet_delta_rule_amd import workloads as W
from oracle import delta_rule_ref
from tests.parity_utils import (TOL, gather_heads, oracle_heads, rel_err, threads,
                                to_dev, to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    dr.load_library()


def _chunk_check(w: W.Workload, heads=None, **kw):
    x = W.generate(w)
    d = to_dev(x)
    o, st = dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["S0"],
                                    chunk=w.chunk, **kw)
    torch.cuda.synchronize()
    if heads is None:
        o_ref, s_ref = delta_rule_ref(x["q"], x["k"], x["v"], x["beta"], x["S0"],
                                      nthreads=threads())
        o_got, s_got = to_np(o), to_np(st)
    else:
        o_ref, s_ref = oracle_heads(x, heads)
        o_got, s_got = gather_heads(o, st, heads)
    tol = TOL[w.torch_dtype]
    eo, es = rel_err(o_got, o_ref), rel_err(s_got, s_ref)
    print(f"{w.name} B{w.B} H{w.H} T{w.T} Dk{w.Dk} Dv{w.Dv} C{w.chunk} {w.dtype}: "
          f"o err {eo:.3e}  S_T err {es:.3e}  (tol {tol:g})", flush=True)
    assert eo <= tol, f"o relative error {eo:.3e} > {tol}"
    assert es <= tol, f"S_T relative error {es:.3e} > {tol}"
    return x, o, st


# ---------------------------------------------------------------- chunk path
SMALL = [
    W.get("tiny_fp32"),
    W.get("small_model", B=2, H=3, T=200),
    W.get("layer_1p3b", B=1, H=4, T=200),
    W.get("long_prefill", H=2, T=333),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_chunk_workload_small(w):
    _chunk_check(w)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Dk", [16, 32, 64, 128])
@pytest.mark.parametrize("Dv", [16, 32, 64, 128])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_chunk_shape_grid(dtype, Dk, Dv, chunk):
    w = W.get("long_prefill", B=2, H=2, T=3 * chunk - 5, Dk=Dk, Dv=Dv, chunk=chunk,
              dtype=dtype, seed=1000 + Dk + 7 * Dv + chunk)
    _chunk_check(w)


@pytest.mark.parametrize("T", [1, 5, 16, 63, 64, 65, 129])
def test_chunk_sequence_lengths(T):
    _chunk_check(W.get("layer_1p3b", B=2, H=2, T=T, seed=2000 + T))


def test_chunk_many_heads_fill_grid():
    # B*H*Dv/64 >= 256: the 4-wave launch used by the benchmark shape
    _chunk_check(W.get("layer_1p3b", B=8, H=16, T=70), heads=[(0, 0), (3, 7), (7, 15)])


@pytest.mark.parametrize("Dv, waves", [(32, 2), (16, 1)])
def test_chunk_two_and_one_wave_launches(Dv, waves):
    # the launch takes 4 state waves (64 value rows) when Dv allows it, else
    # 2 (Dv = 32) or 1 (Dv = 16): the narrower launches at d_k = 128 with
    # many heads
    _chunk_check(W.get("layer_1p3b", B=4, H=16, T=90, Dv=Dv, seed=2100 + waves),
                 heads=[(0, 1), (2, 9), (3, 15)])


# full sizes, exactly the launches the benchmark times (sampled heads)
def test_chunk_full_small_model():
    w = W.get("small_model")
    _chunk_check(w, heads=[(b, h) for b in range(w.B) for h in range(w.H)])


def test_chunk_full_layer_1p3b():
    heads = [(0, 0), (1, 5), (2, 10), (3, 15), (4, 3), (5, 8), (6, 13), (7, 15)]
    _chunk_check(W.get("layer_1p3b"), heads=heads)


def test_chunk_full_long_prefill():
    _chunk_check(W.get("long_prefill"), heads=[(0, 0), (0, 11)])


# ------------------------------------------------------------- edge cases
def test_chunk_empty_sequence_copies_state():
    w = W.get("long_prefill", H=3, T=0)
    x = to_dev(W.generate(w))
    o, st = dr.delta_rule_chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["S0"])
    assert o.shape == (1, 0, 3, 128)
    torch.testing.assert_close(st, x["S0"], rtol=0, atol=0)
    _, st0 = dr.delta_rule_chunk_fwd(x["q"], x["k"], x["v"], x["beta"], None)
    assert torch.count_nonzero(st0) == 0


def test_chunk_beta_zero_keeps_state_exactly():
    w = W.get("long_prefill", H=2, T=150)
    x = W.generate(w)
    x["beta"].zero_()
    d = to_dev(x)
    o, st = dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["S0"])
    torch.testing.assert_close(st, d["S0"], rtol=0, atol=0)
    o_ref, _ = delta_rule_ref(x["q"], x["k"], x["v"], x["beta"], x["S0"])
    assert rel_err(to_np(o), o_ref) <= 2e-2


def test_chunk_state_in_place_and_no_final_state():
    w = W.get("long_prefill", H=2, T=140)
    x = W.generate(w)
    d = to_dev(x)
    o_a, st_a = dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["S0"])
    S = d["S0"].clone()
    o_b, st_b = dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], S, S_T=S)
    assert st_b.data_ptr() == S.data_ptr()
    torch.testing.assert_close(o_b, o_a, rtol=0, atol=0)
    torch.testing.assert_close(S, st_a, rtol=0, atol=0)
    o_c, st_c = dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["S0"],
                                        output_final_state=False)
    assert st_c is None
    torch.testing.assert_close(o_c, o_a, rtol=0, atol=0)


def test_chunk_deterministic():
    w = W.get("layer_1p3b", B=2, H=16, T=300)
    d = to_dev(W.generate(w))
    a = dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["S0"])
    b = dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["S0"])
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_chunk_writes_every_output_and_nothing_else():
    w = W.get("long_prefill", B=2, H=2, T=97)
    x = W.generate(w)
    d = to_dev(x)
    G = 64  # guard elements each side (keeps 16-byte alignment)
    n_o = 2 * 97 * 2 * 128
    n_s = 2 * 2 * 128 * 128
    obuf = torch.full((n_o + 2 * G,), float("nan"), dtype=torch.bfloat16, device="cuda")
    sbuf = torch.full((n_s + 2 * G,), float("nan"), dtype=torch.float32, device="cuda")
    o = obuf[G:G + n_o].view(2, 97, 2, 128)
    st = sbuf[G:G + n_s].view(2, 2, 128, 128)
    dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["S0"], o=o, S_T=st)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any() and not torch.isnan(st).any()
    assert torch.isnan(obuf[:G]).all() and torch.isnan(obuf[-G:]).all()
    assert torch.isnan(sbuf[:G]).all() and torch.isnan(sbuf[-G:]).all()


def test_chunk_resume_matches_single_call():
    # splitting a sequence at a chunk boundary and carrying S_T as S0
    w = W.get("long_prefill", H=2, T=256)
    x = W.generate(w)
    d = to_dev(x)
    o, st = dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["S0"])
    cut = 128
    sl = lambda t, a, b: t[:, a:b].contiguous()
    o1, s1 = dr.delta_rule_chunk_fwd(sl(d["q"], 0, cut), sl(d["k"], 0, cut),
                                     sl(d["v"], 0, cut), sl(d["beta"], 0, cut), d["S0"])
    o2, s2 = dr.delta_rule_chunk_fwd(sl(d["q"], cut, 256), sl(d["k"], cut, 256),
                                     sl(d["v"], cut, 256), sl(d["beta"], cut, 256), s1)
    torch.testing.assert_close(torch.cat([o1, o2], 1), o, rtol=0, atol=0)
    torch.testing.assert_close(s2, st, rtol=0, atol=0)


# --------------------------------------------------------------- decode path
def _decode_run(w: W.Workload, x, steps=None):
    d = to_dev(x)
    S = d["S0"].clone()
    outs = []
    for t in range(steps or w.T):
        outs.append(dr.delta_rule_recurrent_step(d["q"][t], d["k"][t], d["v"][t],
                                                 d["beta"][t], S))
    torch.cuda.synchronize()
    return torch.stack(outs), S


def _decode_check(w: W.Workload, heads=None):
    x = W.generate(w)
    o, S = _decode_run(w, x)
    # the decode inputs are step-major [steps, B, H, .]: as a sequence, B<->steps
    seq = {n: (None if t is None else (t.transpose(0, 1).contiguous() if n != "S0" else t))
           for n, t in x.items()}
    o_seq = o.transpose(0, 1)
    if heads is None:
        o_ref, s_ref = delta_rule_ref(seq["q"], seq["k"], seq["v"], seq["beta"], seq["S0"],
                                      nthreads=threads())
        o_got, s_got = to_np(o_seq), to_np(S)
    else:
        o_ref, s_ref = oracle_heads(seq, heads)
        o_got, s_got = gather_heads(o_seq, S, heads)
    tol = TOL[w.torch_dtype]
    # every step's output, then the final state
    for t in range(w.T):
        e = rel_err(o_got[t] if heads else o_got[:, t], o_ref[t] if heads else o_ref[:, t])
        assert e <= tol, f"step {t}: o relative error {e:.3e} > {tol}"
    eo, es = rel_err(o_got, o_ref), rel_err(s_got, s_ref)
    print(f"decode B{w.B} H{w.H} Dk{w.Dk} Dv{w.Dv} steps{w.T} {w.dtype}: o err {eo:.3e} "
          f"S err {es:.3e}", flush=True)
    assert es <= tol


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Dk", [16, 32, 64, 128])
@pytest.mark.parametrize("Dv", [16, 64, 128])
def test_decode_small(dtype, Dk, Dv):
    _decode_check(W.get("decode", B=3, H=2, T=12, Dk=Dk, Dv=Dv, dtype=dtype,
                        seed=3000 + Dk + Dv))


def test_decode_full_size_sampled_heads():
    w = W.get("decode")
    heads = [(b, h) for b in (0, 17, 64, 127) for h in (0, 5, 10, 15)]
    _decode_check(w, heads=heads)


def test_decode_matches_chunk_path():
    # the same recurrence in its two schedules (token-serial vs chunked)
    w = W.get("long_prefill", B=2, H=3, T=40)
    x = W.generate(w)
    d = to_dev(x)
    o_c, s_c = dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["S0"])
    S = d["S0"].clone()
    o_d = torch.stack([dr.delta_rule_recurrent_step(d["q"][:, t].contiguous(),
                                                    d["k"][:, t].contiguous(),
                                                    d["v"][:, t].contiguous(),
                                                    d["beta"][:, t].contiguous(), S)
                       for t in range(40)], dim=1)
    assert rel_err(to_np(o_d), to_np(o_c)) <= 2e-2
    assert rel_err(to_np(S), to_np(s_c)) <= 2e-2
