"""GPU parity of the backward (``delta_rule_chunk_bwd`` and
``gated_delta_rule_chunk_bwd``) against the fp64 backward oracle.

Seeded inputs and seeded upstream gradients (do, dS_T) go to the HIP path and
to ``oracle.delta_rule_bwd_ref``; every gradient (dq, dk, dv, dbeta, dS0 and,
for the gated rule, dg) must satisfy max |gpu - ref| <= tol * max |ref|,
tol = 1e-4 for fp32 inputs and 2e-2 for bf16 inputs, the forward's
tolerances (dg against max(max |dg|, max |dbeta|): where the gates have
decayed everything its value is a cancellation far below the products it is
made of, see tests.parity_utils.grad_errors).  Cases span several chunks of the backward (32 tokens for bf16,
16 for fp32) with ragged tails, every head size, beta up to 2, a nonzero
incoming state, gates from weak to strong (per-head A up to 16, so that a
chunk's decay underflows), and the layer shape with whole heads sampled.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import deltanet_delta_rule_amd as dr
from deltanet_delta_rule_amd import workloads as W
from oracle import delta_rule_bwd_ref
from tests.parity_utils import TOL, grad_errors, rel_err, threads, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    dr.load_library()


def _upstream(w, seed, with_dst=True):
    gen = torch.Generator().manual_seed(seed)
    do = torch.randn(w.B, w.T, w.H, w.Dv, generator=gen).to(w.torch_dtype)
    dst = torch.randn(w.B, w.H, w.Dv, w.Dk, generator=gen) if with_dst else None
    return do, dst


def _check(w, seed=7, with_dst=True, heads=None):
    x = W.generate(w)
    do, dst = _upstream(w, seed, with_dst)
    d = to_dev(x)
    dstd = None if dst is None else dst.cuda()
    if x.get("g") is None:
        g = dr.delta_rule_chunk_bwd(d["q"], d["k"], d["v"], d["beta"], do.cuda(), d["S0"], dstd)
    else:
        g = dr.gated_delta_rule_chunk_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], do.cuda(),
                                          d["S0"], dstd)
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
    ref = delta_rule_bwd_ref(xs["q"], xs["k"], xs["v"], xs["beta"], do_r, xs["S0"], dst_r,
                             g=xs.get("g"), nthreads=threads())
    tol = TOL[w.torch_dtype]
    names = ("dq", "dk", "dv", "dbeta", "dS0") + (("dg",) if "dg" in ref else ())
    errs = {n: e for n, e in grad_errors(got, ref).items() if n in names}
    print(f"bwd {w.name} B{w.B} H{w.H} T{w.T} Dk{w.Dk} Dv{w.Dv} {w.dtype}: " +
          " ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
    for n, e in errs.items():
        assert e <= tol, f"{n}: relative error {e:.3e} > {tol}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Dk,Dv", [(16, 16), (32, 64), (64, 32), (64, 128), (128, 64),
                                   (128, 128)])
def test_backward_shapes(dtype, Dk, Dv):
    w = W.get("long_prefill", B=2, H=2, T=77, Dk=Dk, Dv=Dv, dtype=dtype,
              seed=7000 + Dk + 3 * Dv)
    _check(w, seed=Dk + Dv)


@pytest.mark.parametrize("T", [1, 16, 31, 32, 33, 100])
def test_backward_sequence_lengths(T):
    _check(W.get("layer_1p3b", B=1, H=2, T=T, seed=7100 + T), seed=T)


def test_backward_without_state_gradient_or_initial_state():
    w = W.get("layer_1p3b", B=2, H=2, T=70, seed=7200)
    _check(w, with_dst=False)


def test_backward_small_model_workload():
    _check(W.get("small_model", B=2, H=3, T=200))


def test_backward_layer_shape_sampled_heads():
    _check(W.get("layer_1p3b", T=512), heads=[(0, 0), (3, 7), (7, 15)])


@pytest.mark.parametrize("gated", [False, True])
def test_backward_single_pass_schedule(gated):
    # more (b, h) than half the compute units: one reverse pass per (b, h)
    w = W.get("layer_1p3b", B=9, H=16, T=80, Dk=64, Dv=64, gate_amax=4.0 if gated else 0.0,
              seed=7400)
    _check(w, heads=[(0, 0), (4, 9), (8, 15)])


@pytest.mark.parametrize("gated", [False, True])
def test_backward_chunk_runs_with_empty_workgroups(gated):
    # 40 (b, h): the recursion pass, then six workgroups per (b, h) over 8
    # chunks in runs of two, the last two workgroups without chunks
    w = W.get("layer_1p3b", B=5, H=8, T=250, Dk=64, Dv=64, gate_amax=4.0 if gated else 0.0,
              seed=7500)
    _check(w, heads=[(0, 0), (2, 5), (4, 7)])


@pytest.mark.parametrize("gated", [False, True])
def test_backward_split_reverse_walk(gated):
    # 80 (b, h) and 10 chunks with a ragged tail: the reverse walk in two
    # pieces on two streams (the single pass over chunks 3..9 from dS_T; the
    # recursion alone over the same chunks for dS at chunk 3, then the single
    # pass over chunks 0..2 from it)
    w = W.get("layer_1p3b", B=5, H=16, T=300, Dk=64, Dv=64, gate_amax=4.0 if gated else 0.0,
              seed=7450)
    _check(w, heads=[(0, 0), (2, 7), (4, 15)])


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("dtype,Dk,Dv", [("bf16", 64, 128), ("bf16", 128, 64), ("bf16", 32, 32),
                                         ("f32", 64, 64)])
def test_backward_segmented_recursion(gated, dtype, Dk, Dv):
    # 4 (b, h), 1000 tokens: the state-gradient recursion in segments (bf16:
    # 32 chunks in 8 segments of 4, the last chunk 8 tokens long), each
    # segment's map and response to dO formed at once, then chained
    w = W.get("layer_1p3b", B=1, H=4, T=1000, Dk=Dk, Dv=Dv, dtype=dtype,
              gate_amax=4.0 if gated else 0.0, beta_scale=2.0, s0_std=0.02, seed=7470)
    _check(w, seed=9)


def test_backward_one_sequence_full_size_sampled_heads():
    # the benchmark's one-sequence backward: B1 H16 T2048 d128, 64 chunks in
    # 8 segments (every head computed, three checked)
    _check(W.get("layer_1p3b", B=1), heads=[(0, 0), (0, 9), (0, 15)])
    _check(W.get("gated_layer_1p3b", B=1), heads=[(0, 3), (0, 12)])


@pytest.mark.parametrize("name,B,T", [("layer_1p3b", 8, 512), ("gated_layer_1p3b", 8, 300),
                                      ("layer_1p3b", 1, 1000), ("gated_layer_1p3b", 2, 130)])
def test_backward_reuses_forward_checkpoints(name, B, T):
    # the checkpointing forward (outputs and every chunk's incoming state in
    # the backward's workspace), then the backward on those checkpoints:
    # equal, bit for bit, to the forward at the backward's chunk and to the
    # backward that forms the checkpoints itself (split walk at 128 (b, h),
    # segmented recursion at 4, two-pass at 32)
    w = W.get(name, B=B, T=T, seed=7480)
    d = to_dev(W.generate(w))
    do, dst = _upstream(w, 13)
    do, dst = do.cuda(), dst.cuda()
    g = d.get("g")
    o, st, ws = dr.delta_rule_chunk_fwd_checkpointed(d["q"], d["k"], d["v"], d["beta"], d["S0"],
                                                     g=g)
    if g is None:
        o2, st2 = dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["S0"], chunk=32,
                                          workspace=False)
        ref = dr.delta_rule_chunk_bwd(d["q"], d["k"], d["v"], d["beta"], do, d["S0"], dst)
        got = dr.delta_rule_chunk_bwd(d["q"], d["k"], d["v"], d["beta"], do, d["S0"], dst,
                                      workspace=ws, checkpoints_ready=True)
    else:
        o2, st2 = dr.gated_delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], g, d["S0"],
                                                chunk=32, workspace=False)
        ref = dr.gated_delta_rule_chunk_bwd(d["q"], d["k"], d["v"], d["beta"], g, do, d["S0"],
                                            dst)
        got = dr.gated_delta_rule_chunk_bwd(d["q"], d["k"], d["v"], d["beta"], g, do, d["S0"],
                                            dst, workspace=ws, checkpoints_ready=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(st, st2)
    for n in ref:
        assert torch.equal(ref[n], got[n]), n


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("B,H,T", [
    (8, 16, 256),    # split walk, 128 (b, h), its fewest chunks: 8 (pieces 2 + 6)
    (5, 13, 257),    # split walk, 65 (b, h), 9 chunks, a one-token tail
    (2, 16, 512),    # segmented recursion, 32 (b, h): 4 segments of 4 chunks
    (1, 1, 4096),    # segmented recursion, one (b, h): 16 segments of 8 chunks
    (2, 8, 480),     # 16 (b, h), 15 chunks: too few for 4 segments, two-pass
])
def test_backward_schedule_boundaries(gated, B, H, T):
    w = W.get("layer_1p3b", B=B, H=H, T=T, Dk=64, Dv=64, gate_amax=4.0 if gated else 0.0,
              beta_scale=2.0, s0_std=0.02, seed=7490 + T)
    heads = None if B * H <= 2 else [(0, 0), (B // 2, H // 2), (B - 1, H - 1)]
    _check(w, seed=17, heads=heads)


@pytest.mark.parametrize("dtype,T,gated", [("f32", 77, False), ("f32", 40, True),
                                          ("bf16", 33, True), ("bf16", 1, False)])
def test_checkpointed_forward_edge_cases(dtype, T, gated):
    # fp32 (16-token chunks) and bf16, ragged and one-token sequences, S_T
    # carried in place over S0: outputs equal the chunked forward at the
    # backward's chunk, and the backward on the kept checkpoints equals the
    # one that forms them (and the oracle)
    w = W.get("layer_1p3b", B=2, H=3, T=T, Dk=32, Dv=64, dtype=dtype,
              gate_amax=4.0 if gated else 0.0, s0_std=0.02, seed=7510 + T)
    d = to_dev(W.generate(w))
    do, dst = _upstream(w, 21)
    do, dst = do.cuda(), dst.cuda()
    g = d.get("g")
    c = 16 if dtype == "f32" else 32
    S0 = d["S0"].clone()
    carry = d["S0"].clone()
    o, st, ws = dr.delta_rule_chunk_fwd_checkpointed(d["q"], d["k"], d["v"], d["beta"], carry,
                                                     g=g, S_T=carry)
    assert st.data_ptr() == carry.data_ptr()
    fwd = dr.delta_rule_chunk_fwd if g is None else \
        (lambda *a, **kw: dr.gated_delta_rule_chunk_fwd(*a[:4], g, *a[4:], **kw))
    o2, st2 = fwd(d["q"], d["k"], d["v"], d["beta"], S0, chunk=c, workspace=False)
    bwd = dr.delta_rule_chunk_bwd if g is None else \
        (lambda *a, **kw: dr.gated_delta_rule_chunk_bwd(*a[:4], g, *a[4:], **kw))
    ref = bwd(d["q"], d["k"], d["v"], d["beta"], do, S0, dst)
    got = bwd(d["q"], d["k"], d["v"], d["beta"], do, S0, dst, workspace=ws,
              checkpoints_ready=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(st, st2)
    for n in ref:
        assert torch.equal(ref[n], got[n]), n


def test_checkpointed_forward_without_final_state_and_empty():
    w = W.get("layer_1p3b", B=1, H=2, T=64, Dk=64, Dv=64, seed=7520)
    d = to_dev(W.generate(w))
    o, st, ws = dr.delta_rule_chunk_fwd_checkpointed(d["q"], d["k"], d["v"], d["beta"],
                                                     output_final_state=False)
    o2, _ = dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], chunk=32,
                                    workspace=False)
    assert st is None and torch.equal(o, o2)
    e = W.get("layer_1p3b", B=1, H=2, T=0, Dk=64, Dv=64, seed=7521)
    de = to_dev(W.generate(e))
    S0 = torch.randn(1, 2, 64, 64, device="cuda")
    o, st, ws = dr.delta_rule_chunk_fwd_checkpointed(de["q"], de["k"], de["v"], de["beta"], S0)
    assert o.shape == (1, 0, 2, 64) and torch.equal(st, S0)


def test_backward_full_size_sampled_heads():
    # the benchmark's configuration and launch: B8 H16 T2048 d128, 64 chunks,
    # the split reverse walk (every head computed, two checked)
    _check(W.get("layer_1p3b"), heads=[(0, 1), (7, 14)])
    _check(W.get("gated_layer_1p3b"), heads=[(3, 2), (6, 11)])


def test_backward_split_walk_is_deterministic():
    w = W.get("gated_layer_1p3b", B=5, H=16, T=300, Dk=64, Dv=64, seed=7460)
    d = to_dev(W.generate(w))
    do, dst = _upstream(w, 5)
    run = lambda: dr.gated_delta_rule_chunk_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"],
                                                do.cuda(), d["S0"], dst.cuda())
    a, b = run(), run()
    for n in a:
        assert torch.equal(a[n], b[n]), n


def test_backward_empty_sequence_passes_the_state_gradient():
    w = W.get("long_prefill", H=2, T=0)
    d = to_dev(W.generate(w))
    dst = torch.randn(1, 2, 128, 128, device="cuda")
    do = torch.zeros(1, 0, 2, 128, dtype=torch.bfloat16, device="cuda")
    g = dr.delta_rule_chunk_bwd(d["q"], d["k"], d["v"], d["beta"], do, d["S0"], dst)
    torch.testing.assert_close(g["dS0"], dst, rtol=0, atol=0)


def test_backward_is_deterministic():
    w = W.get("layer_1p3b", B=2, H=4, T=96, seed=7300)
    d = to_dev(W.generate(w))
    do, dst = _upstream(w, 3)
    a = dr.delta_rule_chunk_bwd(d["q"], d["k"], d["v"], d["beta"], do.cuda(), None, dst.cuda())
    b = dr.delta_rule_chunk_bwd(d["q"], d["k"], d["v"], d["beta"], do.cuda(), None, dst.cuda())
    for n in a:
        assert torch.equal(a[n], b[n]), n


# ----------------------------------------------------------------- gated rule

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Dk,Dv", [(16, 16), (32, 64), (64, 32), (64, 128), (128, 64),
                                   (128, 128)])
def test_gated_backward_shapes(dtype, Dk, Dv):
    w = W.get("gated_layer_1p3b", B=2, H=2, T=77, Dk=Dk, Dv=Dv, dtype=dtype,
              seed=7400 + Dk + 3 * Dv)
    _check(w, seed=Dk + Dv + 1)


@pytest.mark.parametrize("T", [1, 16, 31, 32, 33, 100])
def test_gated_backward_sequence_lengths(T):
    _check(W.get("gated_layer_1p3b", B=1, H=2, T=T, seed=7500 + T), seed=T + 50)


@pytest.mark.parametrize("amax", [0.05, 1.0, 16.0])
def test_gated_backward_gate_strengths(amax):
    # weak gates (the decays' derivatives dominate nothing), moderate, and
    # strong enough that exp(b) underflows within a chunk
    w = W.get("gated_layer_1p3b", B=2, H=3, T=130, gate_amax=amax, seed=7600)
    _check(w, seed=11)


def test_gated_backward_without_state_gradient_or_initial_state():
    w = W.get("gated_layer_1p3b", B=2, H=2, T=70, seed=7700)
    _check(w, with_dst=False)


def test_gated_backward_layer_shape_sampled_heads():
    _check(W.get("gated_layer_1p3b", T=512), heads=[(0, 0), (5, 9), (7, 15)])


def test_backward_full_length_sampled_heads():
    # the layer workload at its full length, both rules, three heads checked
    _check(W.get("layer_1p3b", B=2, H=16), heads=[(0, 3), (1, 12)])
    _check(W.get("gated_layer_1p3b", B=2, H=16), heads=[(0, 5), (1, 14)])


def test_gated_backward_with_zero_gate_matches_plain():
    w = W.get("layer_1p3b", B=2, H=2, T=90, seed=7800)
    d = to_dev(W.generate(w))
    do, dst = _upstream(w, 5)
    a = dr.delta_rule_chunk_bwd(d["q"], d["k"], d["v"], d["beta"], do.cuda(), d["S0"],
                                dst.cuda())
    zero = torch.zeros(w.B, w.T, w.H, device="cuda")
    b = dr.gated_delta_rule_chunk_bwd(d["q"], d["k"], d["v"], d["beta"], zero, do.cuda(),
                                      d["S0"], dst.cuda())
    for n in a:
        e = rel_err(to_np(b[n]), to_np(a[n]).astype(np.float64))
        assert e <= TOL[w.torch_dtype], (n, e)


def test_gated_backward_empty_sequence_passes_the_state_gradient():
    w = W.get("gated_layer_1p3b", B=1, H=2, T=0)
    d = to_dev(W.generate(w))
    dst = torch.randn(1, 2, 128, 128, device="cuda")
    do = torch.zeros(1, 0, 2, 128, dtype=torch.bfloat16, device="cuda")
    g = torch.zeros(1, 0, 2, device="cuda")
    out = dr.gated_delta_rule_chunk_bwd(d["q"], d["k"], d["v"], d["beta"], g, do, d["S0"], dst)
    torch.testing.assert_close(out["dS0"], dst, rtol=0, atol=0)
    assert out["dg"].numel() == 0


def test_gated_backward_is_deterministic():
    w = W.get("gated_layer_1p3b", B=2, H=4, T=96, seed=7900)
    d = to_dev(W.generate(w))
    do, dst = _upstream(w, 3)
    a = dr.gated_delta_rule_chunk_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], do.cuda(),
                                      None, dst.cuda())
    b = dr.gated_delta_rule_chunk_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], do.cuda(),
                                      None, dst.cuda())
    for n in a:
        assert torch.equal(a[n], b[n]), n


@pytest.mark.parametrize("name", ["layer_1p3b", "gated_layer_1p3b"])
def test_checkpoints_are_the_prefix_states(name):
    # The backward's first pass runs the forward kernel without outputs (the
    # specialisation that skips Q K^T, S Q^T and the output products) and
    # leaves each 32-token chunk's incoming state in the workspace, in bf16.
    # Checkpoint c must be the final state of a forward over the first 32 c
    # tokens with outputs (the same state path), rounded to bf16.
    w = W.get(name, B=2, H=2, T=150, seed=8100)
    d = to_dev(W.generate(w))
    do, dst = _upstream(w, 9)
    lib = dr.load_library()
    nbytes = int(lib.delta_rule_chunk_bwd_workspace_bytes(w.B, w.T, w.H, w.Dk, w.Dv, dr.DR_BF16))
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    if d.get("g") is None:
        dr.delta_rule_chunk_bwd(d["q"], d["k"], d["v"], d["beta"], do.cuda(), d["S0"],
                                dst.cuda(), workspace=ws)
    else:
        dr.gated_delta_rule_chunk_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], do.cuda(),
                                      d["S0"], dst.cuda(), workspace=ws)
    torch.cuda.synchronize()
    n = (w.T + 31) // 32
    ck = ws[: w.B * w.H * n * w.Dv * w.Dk * 2].view(torch.bfloat16).view(w.B, w.H, n, w.Dv, w.Dk)
    for c in range(n):
        tp = 32 * c
        if c == 0:
            ref = torch.zeros(w.B, w.H, w.Dv, w.Dk, device="cuda") if d["S0"] is None else d["S0"]
        else:
            sl = lambda t: t[:, :tp].contiguous()
            if d.get("g") is None:
                _, ref = dr.delta_rule_chunk_fwd(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["beta"]),
                                                 d["S0"], chunk=32, workspace=False)
            else:
                _, ref = dr.gated_delta_rule_chunk_fwd(sl(d["q"]), sl(d["k"]), sl(d["v"]),
                                                       sl(d["beta"]), sl(d["g"]), d["S0"],
                                                       chunk=32, workspace=False)
        torch.cuda.synchronize()
        assert torch.equal(ck[:, :, c], ref.to(torch.bfloat16)), f"checkpoint {c}"
