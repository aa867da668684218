"""GPU parity of the segment-parallel schedule of the chunked forward
(``dr_chunk_opts.workspace``) against the fp64 oracles and the plain schedule.

The affine state map of a segment (S_out = S_in M + H, from the update as a
product of transitions plus rank-one writes: hada.io digest, sections
"Chunkwise KDA" and "Transition diagonale-bas rang") lets the library run the
segments of one sequence in parallel.  Seeded inputs go through both
schedules; o and S_T must satisfy max |gpu - ref| <= tol * max |ref| against
the oracle (tol 1e-4 fp32, 2e-2 bf16), and the workspace must have been used
(it starts as NaN).  Shapes give ragged last segments and last chunks.
"""
from __future__ import annotations

import pytest
import torch

import deltanet_delta_rule_amd as dr
from deltanet_delta_rule_amd import workloads as W
from oracle import l2norm_rows
from tests.parity_utils import TOL, oracle_all, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    dr.load_library()


def _run(d, gated, ws, **kw):
    if gated:
        return dr.gated_delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"],
                                             d["S0"], workspace=ws, **kw)
    return dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["S0"], workspace=ws,
                                   **kw)


def _check(w, gated=False, x=None, segmented=True, **kw):
    x = W.generate(w) if x is None else x
    d = to_dev(x)
    need = dr.chunk_fwd_workspace_bytes(w.B, w.T, w.H, w.Dk, w.Dv, w.chunk, w.torch_dtype)
    assert need > 0, "the shape should have a segment plan"
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
    o, st = _run(d, gated, ws, chunk=w.chunk, **kw)
    torch.cuda.synchronize()
    if segmented:
        assert not torch.isnan(ws[:16]).any(), "workspace untouched: segment schedule not used"
    else:
        assert torch.isnan(ws).all(), "the plain schedule should have run"
    o_p, st_p = _run(d, gated, False, chunk=w.chunk, **kw)
    ref_x = x
    if kw.get("use_qk_l2norm_in_kernel"):
        ref_x = dict(x)
        for n in ("q", "k"):
            ref_x[n] = torch.from_numpy(l2norm_rows(x[n].double().numpy()))
    o_ref, s_ref = oracle_all(ref_x)
    o_ref = o_ref * kw.get("scale", 1.0)
    tol = TOL[w.torch_dtype]
    eo, es = rel_err(to_np(o), o_ref), rel_err(to_np(st), s_ref)
    print(f"segments {'gated' if gated else 'plain'} B{w.B} H{w.H} T{w.T} Dk{w.Dk} Dv{w.Dv} "
          f"C{w.chunk} {w.dtype}: o err {eo:.3e} S_T err {es:.3e}", flush=True)
    assert eo <= tol and es <= tol
    assert rel_err(to_np(o), to_np(o_p)) <= tol and rel_err(to_np(st), to_np(st_p)) <= tol


@pytest.mark.parametrize("gated", [False, True])
def test_one_long_sequence(gated):
    _check(W.get("long_prefill", H=2, T=7000, gate_amax=0.5 if gated else 0.0, seed=12000),
           gated)


@pytest.mark.parametrize("gated", [False, True])
def test_batch_of_two_flattened(gated):
    # d = 64: 21 segments of 5 chunks (the combined state-and-map pass, plain
    # and gated rule)
    _check(W.get("small_model", B=2, H=2, T=6500, gate_amax=0.5 if gated else 0.0,
                 seed=12100), gated)


def test_small_model_config_segments():
    # the small-model config (B4 H8 T2048 d64): 8 segments of 4 chunks
    _check(W.get("small_model", seed=12150))


def test_gated_long_prefill_full_size_sampled_heads():
    # the long-prefill shape with the gated layer's gate draw (A up to 16),
    # through the combined pass of the gated rule; whole heads sampled
    from tests.parity_utils import gather_heads, oracle_heads
    w = W.get("long_prefill", gate_amax=16.0, seed=12160)
    x = W.generate(w)
    d = to_dev(x)
    assert dr.chunk_fwd_workspace_bytes(w.B, w.T, w.H, w.Dk, w.Dv, w.chunk) > 0
    o, st = dr.gated_delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["S0"])
    torch.cuda.synchronize()
    heads = [(0, 3), (0, 12)]
    o_ref, s_ref = oracle_heads(x, heads)
    o_got, s_got = gather_heads(o, st, heads)
    eo, es = rel_err(o_got, o_ref), rel_err(s_got, s_ref)
    print(f"segments gated long_prefill full size: o err {eo:.3e} S_T err {es:.3e}", flush=True)
    assert eo <= 2e-2 and es <= 2e-2


def test_fp32_inputs():
    _check(W.get("long_prefill", H=2, T=3300, Dk=64, Dv=64, chunk=32, dtype="f32",
                 seed=12200))


def test_value_width_differs_from_key_width():
    _check(W.get("long_prefill", H=2, T=6200, Dk=128, Dv=64, seed=12300))
    _check(W.get("long_prefill", H=2, T=6200, Dk=32, Dv=128, seed=12301))


def test_l2norm_scale_and_zero_state():
    _check(W.get("layer_1p3b", B=1, H=2, T=6300, feature="raw", seed=12400),
           use_qk_l2norm_in_kernel=True, scale=0.125)


def test_no_final_state():
    w = W.get("long_prefill", H=2, T=6150, seed=12500)
    x = W.generate(w)
    d = to_dev(x)
    need = dr.chunk_fwd_workspace_bytes(w.B, w.T, w.H, w.Dk, w.Dv, w.chunk)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o, st = dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["S0"], workspace=ws,
                                    output_final_state=False)
    assert st is None
    o_ref, _ = oracle_all(x)
    assert rel_err(to_np(o), o_ref) <= 2e-2


def test_long_prefill_full_size_sampled_heads():
    # the long-prefill config itself (B1 H16 T32768), whole heads sampled
    from tests.parity_utils import gather_heads, oracle_heads
    w = W.get("long_prefill")
    x = W.generate(w)
    d = to_dev(x)
    assert dr.chunk_fwd_workspace_bytes(w.B, w.T, w.H, w.Dk, w.Dv, w.chunk) > 0
    o, st = dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["S0"])
    torch.cuda.synchronize()
    heads = [(0, 0), (0, 9)]
    o_ref, s_ref = oracle_heads(x, heads)
    o_got, s_got = gather_heads(o, st, heads)
    eo, es = rel_err(o_got, o_ref), rel_err(s_got, s_ref)
    print(f"segments long_prefill full size: o err {eo:.3e} S_T err {es:.3e}", flush=True)
    assert eo <= 2e-2 and es <= 2e-2


@pytest.mark.parametrize("case", ["amax1", "amax16_erased"])
def test_kda_long_sequence(case):
    # per-key-channel decay: the chunked KDA kernel on the segments, with the
    # gated layer's draw (A up to 1, or up to 16 with every fifth token
    # erasing half the channels)
    amax = 1.0 if case == "amax1" else 16.0
    w = W.get("long_prefill", H=2, T=6700, gate_amax=amax, kda=True, seed=12700)
    x = W.generate(w)
    if case != "amax1":
        x["gk"][:, ::5, :, 64:] = -1e4
    d = to_dev(x)
    need = dr.chunk_fwd_workspace_bytes(w.B, w.T, w.H, w.Dk, w.Dv, 64)
    assert need > 0
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
    o, st = dr.kda_fwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], d["S0"], workspace=ws)
    torch.cuda.synchronize()
    assert not torch.isnan(ws[:16]).any()
    o_p, st_p = dr.kda_fwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], d["S0"], workspace=False)
    o_ref, s_ref = oracle_all(x)
    eo, es = rel_err(to_np(o), o_ref), rel_err(to_np(st), s_ref)
    print(f"segments kda T{w.T}: o err {eo:.3e} S_T err {es:.3e}", flush=True)
    assert eo <= 2e-2 and es <= 2e-2
    assert rel_err(to_np(o), to_np(o_p)) <= 2e-2 and rel_err(to_np(st), to_np(st_p)) <= 2e-2


def test_small_workspace_falls_back_to_the_plain_schedule():
    w = W.get("long_prefill", H=2, T=6600, seed=12600)
    d = to_dev(W.generate(w))
    ws = torch.full((64,), float("nan"), dtype=torch.float32, device="cuda")
    o, st = dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["S0"], workspace=ws)
    o_p, st_p = dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["S0"],
                                        workspace=False)
    torch.cuda.synchronize()
    assert torch.isnan(ws).all()
    assert torch.equal(o, o_p) and torch.equal(st, st_p)
