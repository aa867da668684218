"""GPU parity of the token-serial schedule (``DR_FUSED_RECURRENT``:
``fused_recurrent=True`` on the chunked entry points and on ``kda_fwd``)
against the fp64 oracles.

hada.io digest, section "Kernel Triton recurrent fusionne pour le decodage":
each program owns a slab of one head's state and walks the tokens in order.
Seeded inputs go to the HIP path and to the oracle of the rule (plain, gated,
per-key-channel decay); o and S_T must satisfy max |gpu - ref| <= tol * max
|ref|, tol = 1e-4 for fp32 inputs and 2e-2 for bf16 inputs.  Lengths span
several 16-token staging blocks with ragged tails; packed sequences must equal
separate calls bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import deltanet_delta_rule_amd as dr
from deltanet_delta_rule_amd import workloads as W
from oracle import l2norm_rows
from tests.parity_utils import TOL, gather_heads, oracle_all, oracle_heads, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

RULES = ["plain", "gated", "kda"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    dr.load_library()


def _work(rule, **kw):
    if rule == "gated":
        kw.setdefault("gate_amax", 1.0)
    elif rule == "kda":
        kw.setdefault("gate_amax", 1.0)
        kw["kda"] = True
    return W.get(kw.pop("name", "long_prefill"), **kw)


def _run(d, rule, S0, **kw):
    if rule == "kda":
        return dr.kda_fwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], S0, fused_recurrent=True,
                          **kw)
    if rule == "gated":
        return dr.gated_delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], S0,
                                             fused_recurrent=True, **kw)
    return dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], S0, fused_recurrent=True,
                                   **kw)


def _check(w, rule, heads=None, x=None, **kw):
    x = W.generate(w) if x is None else x
    d = to_dev(x)
    o, st = _run(d, rule, d["S0"], **kw)
    torch.cuda.synchronize()
    if heads is None:
        o_ref, s_ref = oracle_all(x)
        o_got, s_got = to_np(o), to_np(st)
    else:
        o_ref, s_ref = oracle_heads(x, heads)
        o_got, s_got = gather_heads(o, st, heads)
    tol = TOL[w.torch_dtype]
    eo, es = rel_err(o_got, o_ref), rel_err(s_got, s_ref)
    print(f"fused recurrent {rule} B{w.B} H{w.H} T{w.T} Dk{w.Dk} Dv{w.Dv} {w.dtype}: "
          f"o err {eo:.3e} S_T err {es:.3e}", flush=True)
    assert eo <= tol, f"o relative error {eo:.3e} > {tol}"
    assert es <= tol, f"S_T relative error {es:.3e} > {tol}"
    return d, o, st


@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Dk,Dv", [(16, 16), (32, 128), (64, 64), (128, 16), (128, 128)])
def test_shapes(rule, dtype, Dk, Dv):
    _check(_work(rule, B=2, H=2, T=37, Dk=Dk, Dv=Dv, dtype=dtype,
                 seed=9000 + Dk + 3 * Dv + 7 * RULES.index(rule)), rule)


@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("T", [1, 15, 16, 17, 100])
def test_lengths(rule, T):
    _check(_work(rule, name="layer_1p3b", B=2, H=2, T=T, seed=9100 + T), rule)


@pytest.mark.parametrize("rule", RULES)
def test_without_initial_state_and_final_state(rule):
    w = _work(rule, name="layer_1p3b", B=2, H=3, T=40, seed=9200)
    x = W.generate(w)
    d = to_dev(x)
    o, st = _run(d, rule, None, output_final_state=False)
    torch.cuda.synchronize()
    assert st is None
    o_ref, _ = oracle_all(x)
    assert rel_err(to_np(o), o_ref) <= 2e-2


@pytest.mark.parametrize("rule", RULES)
def test_l2norm_and_scale(rule):
    w = _work(rule, B=2, H=2, T=50, feature="raw", seed=9300)
    x = W.generate(w)
    d = to_dev(x)
    o, st = _run(d, rule, d["S0"], scale=0.125, use_qk_l2norm_in_kernel=True)
    torch.cuda.synchronize()
    xn = dict(x)
    for n in ("q", "k"):
        xn[n] = torch.from_numpy(l2norm_rows(x[n].double().numpy()))
    o_ref, s_ref = oracle_all(xn)
    assert rel_err(to_np(o), 0.125 * o_ref) <= 2e-2
    assert rel_err(to_np(st), s_ref) <= 2e-2


@pytest.mark.parametrize("rule", ["plain", "gated"])
def test_matches_chunked_schedule(rule):
    w = _work(rule, B=2, H=2, T=130, seed=9400)
    d = to_dev(W.generate(w))
    o_r, s_r = _run(d, rule, d["S0"])
    if rule == "gated":
        o_c, s_c = dr.gated_delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"],
                                                 d["S0"])
    else:
        o_c, s_c = dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["S0"])
    assert rel_err(to_np(o_r), to_np(o_c)) <= 2e-2
    assert rel_err(to_np(s_r), to_np(s_c)) <= 2e-2


def test_kda_matches_decode_steps():
    w = _work("kda", B=2, H=3, T=20, seed=9500)
    d = to_dev(W.generate(w))
    o_f, s_f = _run(d, "kda", d["S0"])
    S = d["S0"].clone()
    col = lambda t, i: t[:, i].contiguous()
    o_d = torch.stack([dr.kda_recurrent_step(col(d["q"], t), col(d["k"], t), col(d["v"], t),
                                             col(d["beta"], t), col(d["gk"], t), S)
                       for t in range(w.T)], dim=1)
    # the same per-token arithmetic in both kernels
    assert rel_err(to_np(o_f), to_np(o_d)) <= 1e-2
    assert rel_err(to_np(s_f), to_np(S)) <= 1e-5


@pytest.mark.parametrize("amax", [0.05, 16.0])
def test_kda_decay_strengths(amax):
    _check(_work("kda", H=4, T=70, gate_amax=amax, seed=9600 + int(amax)), "kda")


def test_kda_layer_shape_sampled_heads():
    heads = [(0, 0), (3, 7), (7, 15)]
    w = _work("kda", name="layer_1p3b", T=512, seed=9700)
    _check(w, "kda", heads=heads)


def test_kda_equal_channels_is_the_gated_rule():
    w = _work("gated", B=2, H=2, T=45, seed=9800)
    x = W.generate(w)
    d = to_dev(x)
    gk = d["g"][..., None].expand(-1, -1, -1, w.Dk).contiguous()
    o_k, s_k = dr.kda_fwd(d["q"], d["k"], d["v"], d["beta"], gk, d["S0"], fused_recurrent=True)
    o_g, s_g = _run(d, "gated", d["S0"])
    torch.testing.assert_close(o_k, o_g, rtol=0, atol=0)
    torch.testing.assert_close(s_k, s_g, rtol=0, atol=0)


@pytest.mark.parametrize("rule", ["plain", "kda"])
def test_packed_sequences_equal_separate_calls(rule):
    lengths = [0, 1, 16, 33, 70, 5]
    T = sum(lengths)
    w = _work(rule, B=1, H=2, T=T, seed=9900)
    x = W.generate(w)
    d = to_dev(x)
    n = len(lengths)
    S0 = 0.02 * torch.randn(n, 2, 128, 128, generator=torch.Generator().manual_seed(9901))
    S0d = S0.cuda()
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    o, st = _run(d, rule, S0d, cu_seqlens=cu.cuda())
    torch.cuda.synchronize()
    for s, L in enumerate(lengths):
        a, b = int(cu[s]), int(cu[s + 1])
        sl = {k: (None if t is None else t[:, a:b].contiguous()) for k, t in d.items()}
        o1, st1 = _run(sl, rule, S0d[s:s + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(o[:, a:b], o1), f"sequence {s}: o differs"
        assert torch.equal(st[s:s + 1], st1), f"sequence {s}: S_T differs"
        if L:
            xs = {k: (None if t is None else t[:, a:b].contiguous()) for k, t in x.items()}
            xs["S0"] = S0[s:s + 1]
            o_ref, s_ref = oracle_all(xs)
            assert rel_err(to_np(o[:, a:b]), o_ref) <= 2e-2
            assert rel_err(to_np(st[s:s + 1]), s_ref) <= 2e-2


def test_packed_gaps_untouched_and_in_place_state():
    w = _work("kda", B=1, H=2, T=90, seed=9950)
    d = to_dev(W.generate(w))
    cu = torch.tensor([0, 30, 20, 60], dtype=torch.int32, device="cuda")  # seq 1 inverted
    S = 0.02 * torch.randn(3, 2, 128, 128, device="cuda")
    S_in = S.clone()
    o = torch.full_like(d["v"], float("nan"))
    dr.kda_fwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], S, cu_seqlens=cu, o=o, S_T=S,
               fused_recurrent=True)
    torch.cuda.synchronize()
    assert not torch.isnan(o[:, :60]).any()
    assert torch.isnan(o[:, 60:]).all()
    assert torch.equal(S[1], S_in[1])        # the inverted range is an empty sequence
    sl = {k: (None if t is None else t[:, 20:60].contiguous()) for k, t in d.items()}
    o2, s2 = dr.kda_fwd(sl["q"], sl["k"], sl["v"], sl["beta"], sl["gk"], S_in[2:3].contiguous(),
                        fused_recurrent=True)
    assert torch.equal(S[2:3], s2)


def test_writes_every_output_and_nothing_else():
    w = _work("kda", B=2, H=2, T=53, seed=9960)
    d = to_dev(W.generate(w))
    G = 64
    n_o, n_s = 2 * 53 * 2 * 128, 2 * 2 * 128 * 128
    obuf = torch.full((n_o + 2 * G,), float("nan"), dtype=torch.bfloat16, device="cuda")
    sbuf = torch.full((n_s + 2 * G,), float("nan"), dtype=torch.float32, device="cuda")
    o = obuf[G:G + n_o].view(2, 53, 2, 128)
    st = sbuf[G:G + n_s].view(2, 2, 128, 128)
    dr.kda_fwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], d["S0"], o=o, S_T=st,
               fused_recurrent=True)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any() and not torch.isnan(st).any()
    assert torch.isnan(obuf[:G]).all() and torch.isnan(obuf[-G:]).all()
    assert torch.isnan(sbuf[:G]).all() and torch.isnan(sbuf[-G:]).all()


def test_empty_sequence_copies_state():
    w = _work("kda", H=3, T=0)
    d = to_dev(W.generate(w))
    o, st = dr.kda_fwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], d["S0"], fused_recurrent=True)
    assert o.shape == (1, 0, 3, 128)
    torch.testing.assert_close(st, d["S0"], rtol=0, atol=0)
