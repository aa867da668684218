"""GPU parity of the chunked forward's options (``delta_rule_chunk_fwd_ex``):
packed variable-length sequences (``cu_seqlens``) and the output scale, for
the plain and the gated rule.

Packed sequences must give, bit for bit, what separate calls on each sequence
give (the same kernel runs the same chunks from each sequence's first token),
and match the fp64 oracle per sequence within the tolerances of the plain
calls (1e-4 fp32, 2e-2 bf16, relative to max |ref|).  Offsets that do not
cover the row, or that decrease, must leave the uncovered outputs untouched
and give empty sequences, never an access outside the buffers.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import deltanet_delta_rule_amd as dr
from deltanet_delta_rule_amd import workloads as W
from tests.parity_utils import TOL, oracle_all, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    dr.load_library()


def _packed(lengths, gated, dtype="bf16", Dk=128, Dv=128, chunk=64, H=2, seed=6000):
    """One batch row holding len(lengths) sequences; per-sequence S0."""
    T = int(sum(lengths))
    w = W.get("long_prefill", B=1, H=H, T=T, Dk=Dk, Dv=Dv, chunk=chunk, dtype=dtype,
              gate_amax=0.5 if gated else 0.0, seed=seed)
    x = W.generate(w)
    n = len(lengths)
    S0 = 0.02 * torch.randn(n, H, Dv, Dk, generator=torch.Generator().manual_seed(seed + 1))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    return w, x, S0, cu


def _call(d, gated, S0, **kw):
    if gated:
        return dr.gated_delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], S0, **kw)
    return dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], S0, **kw)


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("dtype,Dk,Dv,chunk", [("bf16", 128, 128, 64), ("f32", 32, 64, 32),
                                               ("bf16", 64, 16, 16)])
def test_packed_sequences_equal_separate_calls(gated, dtype, Dk, Dv, chunk):
    lengths = [0, 1, 63, 64, 65, 200, 17]
    w, x, S0, cu = _packed(lengths, gated, dtype, Dk, Dv, chunk)
    d = to_dev(x)
    S0d, cud = S0.cuda(), cu.cuda()
    o, st = _call(d, gated, S0d, chunk=chunk, cu_seqlens=cud)
    torch.cuda.synchronize()
    tol = TOL[w.torch_dtype]
    for s, L in enumerate(lengths):
        a, b = int(cu[s]), int(cu[s + 1])
        sl = {n: (None if t is None else t[:, a:b].contiguous()) for n, t in d.items()}
        o1, st1 = _call(sl, gated, S0d[s:s + 1].contiguous(), chunk=chunk)
        torch.cuda.synchronize()
        assert torch.equal(o[:, a:b], o1), f"sequence {s} (length {L}): o differs"
        assert torch.equal(st[s:s + 1], st1), f"sequence {s} (length {L}): S_T differs"
        if L:
            xs = {n: (None if t is None else t[:, a:b].contiguous()) for n, t in x.items()}
            xs["S0"] = S0[s:s + 1]
            o_ref, s_ref = oracle_all(xs)
            assert rel_err(to_np(o[:, a:b]), o_ref) <= tol
            assert rel_err(to_np(st[s:s + 1]), s_ref) <= tol
        else:
            assert torch.equal(st[s], S0d[s])
    print(f"packed {lengths} gated={gated} {dtype} Dk{Dk} Dv{Dv} C{chunk}: equal", flush=True)


def test_packed_offsets_are_clamped_and_gaps_untouched():
    # offsets [0, 50, 30, 140, 999]: sequence 1 is inverted (empty), the last
    # one runs past the row (clamped to T = 160), and tokens 30..49 belong to
    # sequence 0 only up to 50; every token past a sequence stays NaN
    w, x, S0, _ = _packed([40, 40, 80], False)
    d = to_dev(x)
    cu = torch.tensor([0, 50, 30, 140, 999], dtype=torch.int32, device="cuda")
    S0d = 0.02 * torch.randn(4, 2, 128, 128, device="cuda")
    o = torch.full_like(d["v"], float("nan"))
    o, st = dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], S0d, cu_seqlens=cu, o=o)
    torch.cuda.synchronize()
    assert not torch.isnan(o[:, :50]).any() and not torch.isnan(o[:, 50:160]).any()
    assert torch.equal(st[1], S0d[1])   # inverted range: empty sequence
    # sequence 2 is tokens 30..139 after clamping; sequence 3 is 140..159
    for s, (a, b) in [(0, (0, 50)), (3, (140, 160))]:
        sl = {n: (None if t is None else t[:, a:b].contiguous()) for n, t in d.items()}
        o1, st1 = dr.delta_rule_chunk_fwd(sl["q"], sl["k"], sl["v"], sl["beta"],
                                          S0d[s:s + 1].contiguous())
        assert torch.equal(st[s:s + 1], st1)
        if s == 3:
            assert torch.equal(o[:, a:b], o1)


def test_packed_gap_outputs_stay_untouched():
    w, x, S0, _ = _packed([30, 30, 40], False)
    d = to_dev(x)
    cu = torch.tensor([0, 30, 30, 70], dtype=torch.int32, device="cuda")  # tokens 70..99 in no sequence
    o = torch.full_like(d["v"], float("nan"))
    dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], None, cu_seqlens=cu, o=o,
                            output_final_state=False)
    torch.cuda.synchronize()
    assert not torch.isnan(o[:, :70]).any()
    assert torch.isnan(o[:, 70:]).all()


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_output_scale(gated, dtype):
    w = W.get("long_prefill", B=2, H=2, T=150, dtype=dtype, gate_amax=0.5 if gated else 0.0)
    x = W.generate(w)
    d = to_dev(x)
    scale = 128 ** -0.5
    o_s, st_s = _call(d, gated, d["S0"], scale=scale)
    o_1, st_1 = _call(d, gated, d["S0"])
    torch.cuda.synchronize()
    assert torch.equal(st_s, st_1)  # the state never sees the scale
    o_ref, _ = oracle_all(x)
    tol = TOL[w.torch_dtype]
    assert rel_err(to_np(o_s), scale * o_ref) <= tol
    # the scale is applied in fp32 before the output is rounded
    assert rel_err(to_np(o_s), scale * to_np(o_1)) <= (1e-6 if dtype == "f32" else 8e-3)


# ------------------------------------------------ in-kernel q/k L2 norm
def _l2_inputs(x):
    from oracle import l2norm_rows
    xs = dict(x)
    xs["q"] = torch.from_numpy(l2norm_rows(x["q"]))
    xs["k"] = torch.from_numpy(l2norm_rows(x["k"]))
    return xs


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("dtype,Dk,Dv,chunk", [("bf16", 128, 128, 64), ("f32", 128, 64, 64),
                                               ("f32", 16, 32, 16), ("bf16", 32, 128, 32),
                                               ("bf16", 64, 64, 64)])
def test_l2norm_in_kernel_matches_oracle(gated, dtype, Dk, Dv, chunk):
    w = W.get("long_prefill", B=2, H=2, T=3 * chunk - 7, Dk=Dk, Dv=Dv, chunk=chunk, dtype=dtype,
              feature="raw", gate_amax=0.5 if gated else 0.0, seed=6100 + Dk + Dv + chunk)
    x = W.generate(w)
    d = to_dev(x)
    o, st = _call(d, gated, d["S0"], chunk=chunk, use_qk_l2norm_in_kernel=True)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_all(_l2_inputs(x))
    tol = TOL[w.torch_dtype]
    eo, es = rel_err(to_np(o), o_ref), rel_err(to_np(st), s_ref)
    print(f"l2norm gated={gated} {dtype} Dk{Dk} Dv{Dv} C{chunk}: o {eo:.2e} S_T {es:.2e}",
          flush=True)
    assert eo <= tol and es <= tol


def test_l2norm_full_layer_sampled_heads():
    from tests.parity_utils import gather_heads, oracle_heads
    w = W.get("layer_1p3b", feature="raw")
    x = W.generate(w)
    d = to_dev(x)
    o, st = dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], None,
                                    use_qk_l2norm_in_kernel=True)
    torch.cuda.synchronize()
    heads = [(0, 0), (3, 9), (7, 15)]
    o_ref, s_ref = oracle_heads(_l2_inputs(x), heads)
    o_got, s_got = gather_heads(o, st, heads)
    assert rel_err(o_got, o_ref) <= 2e-2 and rel_err(s_got, s_ref) <= 2e-2


def test_l2norm_zero_rows_and_packed_sequences():
    # zero q / k rows normalise to zero (nothing written, nothing read), and
    # packed sequences still equal separate calls bit for bit
    lengths = [70, 0, 129, 5]
    w, x, S0, cu = _packed(lengths, True, "bf16")
    x = dict(x)
    x["q"] = 3.0 * x["q"].float()
    x["k"] = 3.0 * x["k"].float()
    x["k"][:, 10] = 0
    x["q"][:, 11] = 0
    x["q"], x["k"] = x["q"].to(torch.bfloat16), x["k"].to(torch.bfloat16)
    d = to_dev(x)
    S0d, cud = S0.cuda(), cu.cuda()
    o, st = _call(d, True, S0d, cu_seqlens=cud, use_qk_l2norm_in_kernel=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o[:, 11]) == 0
    for s in range(len(lengths)):
        a, b = int(cu[s]), int(cu[s + 1])
        sl = {n: (None if t is None else t[:, a:b].contiguous()) for n, t in d.items()}
        o1, st1 = _call(sl, True, S0d[s:s + 1].contiguous(), use_qk_l2norm_in_kernel=True)
        assert torch.equal(o[:, a:b], o1) and torch.equal(st[s:s + 1], st1)
        if b > a:
            xs = _l2_inputs({n: (None if t is None else t[:, a:b].contiguous())
                             for n, t in x.items()})
            xs["S0"] = S0[s:s + 1]
            o_ref, s_ref = oracle_all(xs)
            assert rel_err(to_np(o[:, a:b]), o_ref) <= 2e-2
            assert rel_err(to_np(st[s:s + 1]), s_ref) <= 2e-2


# ------------------------------------------------------ decode-step options
def _decode_opts_check(w, gated, **kw):
    x = W.generate(w)
    d = to_dev(x)
    S = d["S0"].clone()
    outs = []
    for t in range(w.T):
        if gated:
            outs.append(dr.gated_delta_rule_recurrent_step(d["q"][t], d["k"][t], d["v"][t],
                                                           d["beta"][t], d["g"][t], S, **kw))
        else:
            outs.append(dr.delta_rule_recurrent_step(d["q"][t], d["k"][t], d["v"][t],
                                                     d["beta"][t], S, **kw))
    torch.cuda.synchronize()
    seq = {n: (None if t is None else (t.transpose(0, 1).contiguous() if n != "S0" else t))
           for n, t in x.items()}
    if kw.get("use_qk_l2norm_in_kernel"):
        seq = _l2_inputs(seq)
    o_ref, s_ref = oracle_all(seq)
    o_ref = o_ref * (kw.get("scale") or 1.0)
    tol = TOL[w.torch_dtype]
    o_seq = torch.stack(outs).transpose(0, 1)
    eo, es = rel_err(to_np(o_seq), o_ref), rel_err(to_np(S), s_ref)
    print(f"decode opts {kw} gated={gated} Dk{w.Dk} {w.dtype}: o {eo:.2e} S {es:.2e}", flush=True)
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Dk,Dv", [(16, 16), (64, 128), (128, 128)])
def test_decode_l2norm_and_scale(gated, dtype, Dk, Dv):
    w = W.get("decode", B=3, H=2, T=10, Dk=Dk, Dv=Dv, dtype=dtype, feature="raw",
              gate_amax=0.5 if gated else 0.0, seed=6300 + Dk + Dv)
    _decode_opts_check(w, gated, use_qk_l2norm_in_kernel=True, scale=Dk ** -0.5)


@pytest.mark.parametrize("gated", [False, True])
def test_decode_scale_only(gated):
    w = W.get("decode", B=4, H=2, T=8, gate_amax=0.5 if gated else 0.0, seed=6400)
    _decode_opts_check(w, gated, scale=0.25)


def test_decode_l2norm_matches_chunk_l2norm():
    w = W.get("long_prefill", B=2, H=3, T=40, feature="raw", gate_amax=0.5)
    d = to_dev(W.generate(w))
    o_c, s_c = dr.gated_delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["S0"],
                                             use_qk_l2norm_in_kernel=True)
    S = d["S0"].clone()
    col = lambda t, i: t[:, i].contiguous()
    o_d = torch.stack([dr.gated_delta_rule_recurrent_step(
        col(d["q"], t), col(d["k"], t), col(d["v"], t), col(d["beta"], t), col(d["g"], t), S,
        use_qk_l2norm_in_kernel=True) for t in range(40)], dim=1)
    assert rel_err(to_np(o_d), to_np(o_c)) <= 2e-2
    assert rel_err(to_np(S), to_np(s_c)) <= 2e-2
