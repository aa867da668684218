"""GPU parity of the chunked KDA forward (``kda_fwd`` on bf16 inputs with
d_k = 128 and d_v a multiple of 64) against the fp64 KDA oracle.

hada.io digest, section "Chunkwise KDA": per-channel cumulative decays
inside each 32-token chunk, decayed couplings and read weights, the unit
lower-triangular solve, and the end-of-chunk state as one product.  Seeded
inputs go to the HIP path and to ``oracle.kda_ref``; o and S_T must satisfy
max |gpu - ref| <= 2e-2 * max |ref| (bf16 inputs).  Lengths span one to
several chunks with ragged tails; decays go from near 1 to erasing a channel
within one token (the digest's section "Kimi Delta Attention : attenuation
par canal": per-channel decay lets one channel be wiped while another keeps
its content): the gated layer's draw with A up to 16, constant gk down to
-1e4 on every token and channel, half the channels erased while the other
half keep everything, and channels at gk = -inf.
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


def _kda(name="long_prefill", **kw):
    kw.setdefault("gate_amax", 1.0)
    kw["kda"] = True
    return W.get(name, **kw)


def _check(w, heads=None, x=None, **kw):
    x = W.generate(w) if x is None else x
    d = to_dev(x)
    o, st = dr.kda_fwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], d["S0"], **kw)
    torch.cuda.synchronize()
    if heads is None:
        o_ref, s_ref = oracle_all(x)
        o_got, s_got = to_np(o), to_np(st)
    else:
        o_ref, s_ref = oracle_heads(x, heads)
        o_got, s_got = gather_heads(o, st, heads)
    tol = TOL[w.torch_dtype]
    eo, es = rel_err(o_got, o_ref), rel_err(s_got, s_ref)
    print(f"kda chunk B{w.B} H{w.H} T{w.T} Dv{w.Dv} Amax{w.gate_amax:g}: o err {eo:.3e} "
          f"S_T err {es:.3e}", flush=True)
    assert eo <= tol, f"o relative error {eo:.3e} > {tol}"
    assert es <= tol, f"S_T relative error {es:.3e} > {tol}"
    return d, o, st


@pytest.mark.parametrize("Dv", [64, 128])
def test_value_widths(Dv):
    _check(_kda(B=2, H=2, T=150, Dv=Dv, seed=10000 + Dv))


@pytest.mark.parametrize("T", [1, 15, 16, 17, 63, 64, 65, 130, 257])
def test_lengths(T):
    _check(_kda("layer_1p3b", B=2, H=2, T=T, seed=10100 + T))


@pytest.mark.parametrize("amax", [0.02, 0.3, 1.0, 16.0])
def test_decay_strengths(amax):
    _check(_kda(H=4, T=200, gate_amax=amax, seed=10200 + int(100 * amax)))


@pytest.mark.parametrize("gval", [-5.0, -12.0, -80.0, -1e4])
def test_constant_strong_decay(gval):
    # the same gk on every token and channel: a token's write survives the
    # next token by exp(gval) (from e^-5 down to nothing at all)
    w = _kda(B=1, H=2, T=140, seed=10300)
    x = W.generate(w)
    x["gk"] = torch.full_like(x["gk"], gval)
    _check(w, x=x)


def test_half_the_channels_erased():
    # channels 64..127 forget everything at every token (gk = -1e4), channels
    # 0..63 keep everything (gk = 0)
    w = _kda(B=2, H=2, T=100, seed=10350)
    x = W.generate(w)
    gk = torch.zeros_like(x["gk"])
    gk[..., 64:] = -1e4
    x["gk"] = gk
    _check(w, x=x)


def test_erasure_mixed_into_the_gate_draw():
    # the A ~ U(0, 16) draw, with every third token erasing every other
    # channel and a block of tokens and channels that keeps everything
    w = _kda(B=2, H=2, T=161, gate_amax=16.0, seed=10360)
    x = W.generate(w)
    gk = x["gk"].clone()
    gk[:, ::3, :, ::2] = -1e4
    gk[:, 40:75, :, 10:30] = 0.0
    x["gk"] = gk
    _check(w, x=x)


def test_channels_at_minus_infinity():
    # exp(-inf) = 0 exactly: a quarter of the channels erased outright
    w = _kda(B=1, H=2, T=90, gate_amax=16.0, seed=10370)
    x = W.generate(w)
    gk = x["gk"].clone()
    gk[..., 96:] = float("-inf")
    x["gk"] = gk
    _check(w, x=x)


def test_zero_decay_is_the_plain_rule():
    w = W.get("long_prefill", B=2, H=2, T=150, seed=10400)
    x = W.generate(w)
    d = to_dev(x)
    gk = torch.zeros(2, 150, 2, 128, device="cuda")
    o_k, s_k = dr.kda_fwd(d["q"], d["k"], d["v"], d["beta"], gk, d["S0"])
    o_ref, s_ref = oracle_all(x)
    assert rel_err(to_np(o_k), o_ref) <= 2e-2
    assert rel_err(to_np(s_k), s_ref) <= 2e-2


def test_equal_channels_matches_the_gated_chunk_kernel():
    w = W.get("long_prefill", B=2, H=2, T=130, gate_amax=1.0, seed=10500)
    d = to_dev(W.generate(w))
    gk = d["g"][..., None].expand(-1, -1, -1, 128).contiguous()
    o_k, s_k = dr.kda_fwd(d["q"], d["k"], d["v"], d["beta"], gk, d["S0"])
    o_g, s_g = dr.gated_delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["S0"])
    assert rel_err(to_np(o_k), to_np(o_g)) <= 2e-2
    assert rel_err(to_np(s_k), to_np(s_g)) <= 2e-2


@pytest.mark.parametrize("amax", [1.0, 16.0])
def test_matches_token_serial_schedule(amax):
    w = _kda(B=2, H=2, T=333, gate_amax=amax, seed=10600)
    d = to_dev(W.generate(w))
    o_c, s_c = dr.kda_fwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], d["S0"])
    o_r, s_r = dr.kda_fwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], d["S0"],
                          fused_recurrent=True)
    assert rel_err(to_np(o_c), to_np(o_r)) <= 2e-2
    assert rel_err(to_np(s_c), to_np(s_r)) <= 2e-2


def test_in_kernel_l2norm():
    # raw q, k normalised inside the kernel, against the oracle on the
    # normalised rows and against the token-serial kernel's own L2 option
    from oracle import l2norm_rows
    w = _kda("layer_1p3b", B=2, H=2, T=100, feature="raw", seed=10750)
    x = W.generate(w)
    d = to_dev(x)
    o, st = dr.kda_fwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], None,
                       use_qk_l2norm_in_kernel=True)
    xn = dict(x)
    for n in ("q", "k"):
        xn[n] = torch.from_numpy(l2norm_rows(x[n].double().numpy()))
    o_ref, s_ref = oracle_all(xn)
    assert rel_err(to_np(o), o_ref) <= 2e-2
    assert rel_err(to_np(st), s_ref) <= 2e-2
    o_r, s_r = dr.kda_fwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], None,
                          use_qk_l2norm_in_kernel=True, fused_recurrent=True)
    assert rel_err(to_np(o), to_np(o_r)) <= 2e-2
    assert rel_err(to_np(st), to_np(s_r)) <= 2e-2


def test_output_scale_and_no_initial_state():
    w = _kda("layer_1p3b", B=2, H=2, T=90, seed=10700)
    x = W.generate(w)
    d = to_dev(x)
    o, st = dr.kda_fwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], None, scale=0.125)
    o_ref, s_ref = oracle_all(x)
    assert rel_err(to_np(o), 0.125 * o_ref) <= 2e-2
    assert rel_err(to_np(st), s_ref) <= 2e-2


@pytest.mark.parametrize("amax", [1.0, 16.0])
def test_layer_shape_sampled_heads(amax):
    # the benchmark's launch: B8 H16 T2048 d128, whole heads sampled
    heads = [(0, 0), (3, 7), (7, 15)]
    _check(_kda("layer_1p3b", gate_amax=amax, seed=10800), heads=heads)


def test_packed_sequences_equal_separate_calls():
    lengths = [0, 1, 64, 65, 130, 17]
    T = sum(lengths)
    w = _kda(B=1, H=2, T=T, seed=10900)
    x = W.generate(w)
    d = to_dev(x)
    n = len(lengths)
    S0 = 0.02 * torch.randn(n, 2, 128, 128, generator=torch.Generator().manual_seed(10901))
    S0d = S0.cuda()
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    o, st = dr.kda_fwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], S0d, cu_seqlens=cu.cuda())
    torch.cuda.synchronize()
    for s, L in enumerate(lengths):
        a, b = int(cu[s]), int(cu[s + 1])
        sl = {k: (None if t is None else t[:, a:b].contiguous()) for k, t in d.items()}
        o1, st1 = dr.kda_fwd(sl["q"], sl["k"], sl["v"], sl["beta"], sl["gk"],
                             S0d[s:s + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(o[:, a:b], o1), f"sequence {s}: o differs"
        assert torch.equal(st[s:s + 1], st1), f"sequence {s}: S_T differs"
        if L:
            xs = {k: (None if t is None else t[:, a:b].contiguous()) for k, t in x.items()}
            xs["S0"] = S0[s:s + 1]
            o_ref, s_ref = oracle_all(xs)
            assert rel_err(to_np(o[:, a:b]), o_ref) <= 2e-2
            assert rel_err(to_np(st[s:s + 1]), s_ref) <= 2e-2


def test_resume_matches_single_call():
    w = _kda(B=1, H=2, T=256, seed=11000)
    d = to_dev(W.generate(w))
    o, st = dr.kda_fwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], d["S0"])
    sl = lambda t, a, b: t[:, a:b].contiguous()
    part = lambda a, b, s: dr.kda_fwd(sl(d["q"], a, b), sl(d["k"], a, b), sl(d["v"], a, b),
                                      sl(d["beta"], a, b), sl(d["gk"], a, b), s)
    o1, s1 = part(0, 128, d["S0"])
    o2, s2 = part(128, 256, s1)
    torch.testing.assert_close(torch.cat([o1, o2], 1), o, rtol=0, atol=0)
    torch.testing.assert_close(s2, st, rtol=0, atol=0)


def test_in_place_state_and_canaries():
    w = _kda(B=2, H=2, T=77, seed=11100)
    d = to_dev(W.generate(w))
    G = 64
    n_o = 2 * 77 * 2 * 128
    obuf = torch.full((n_o + 2 * G,), float("nan"), dtype=torch.bfloat16, device="cuda")
    o = obuf[G:G + n_o].view(2, 77, 2, 128)
    S = d["S0"].clone()
    o_ref, s_ref = dr.kda_fwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], d["S0"])
    dr.kda_fwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], S, o=o, S_T=S)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S, s_ref)
    assert torch.isnan(obuf[:G]).all() and torch.isnan(obuf[-G:]).all()


def test_is_deterministic():
    w = _kda(B=2, H=4, T=200, seed=11200)
    d = to_dev(W.generate(w))
    a = dr.kda_fwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], d["S0"])
    b = dr.kda_fwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], d["S0"])
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_empty_sequence_copies_state():
    w = _kda(H=3, T=0)
    d = to_dev(W.generate(w))
    o, st = dr.kda_fwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], d["S0"])
    assert o.shape == (1, 0, 3, 128)
    torch.testing.assert_close(st, d["S0"], rtol=0, atol=0)
