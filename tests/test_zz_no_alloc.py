"""GPU test of delta_rule_chunk_fwd_noalloc (the chunked forward whose
segment-parallel schedule takes its scratch from the library's static
per-GPU array) against delta_rule_chunk_fwd_ex with a caller workspace, both
called through the C ABI.

The two share every kernel, so their outputs must be equal bit for bit; they
are also checked against the fp64 oracle (max |gpu - ref| <= 2e-2 max |ref|
for bf16 inputs).  Two calls in a row, the second on a smaller shape, show
that nothing depends on what an earlier call left in the shared array.
"""
from __future__ import annotations

import ctypes

import pytest
import torch

import deltanet_delta_rule_amd as dr
from deltanet_delta_rule_amd import workloads as W
from tests.parity_utils import oracle_all, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return dr.load_library()


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _opts(d, workspace=None):
    o = dr.dr_chunk_opts(g=None, cu_seqlens=None, num_seqs=0, scale=1.0, flags=0, gk=None,
                         workspace=None, workspace_bytes=0)
    if d.get("g") is not None:
        o.g = d["g"].data_ptr()
    if d.get("gk") is not None:
        o.gk = d["gk"].data_ptr()
    if workspace is not None:
        o.workspace = workspace.data_ptr()
        o.workspace_bytes = workspace.numel()
    return o


def _run(lib, w, d, noalloc, chunk):
    """One call through the C ABI; returns (status, o, S_T)."""
    code = dr.DR_BF16 if w.dtype == "bf16" else dr.DR_F32
    o = torch.full((w.B, w.T, w.H, w.Dv), float("nan"), dtype=w.torch_dtype, device="cuda")
    st = torch.full((w.B, w.H, w.Dv, w.Dk), float("nan"), dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = (_p(d["q"]), _p(d["k"]), _p(d["v"]), _p(d["beta"]), _p(d["S0"]), _p(o), _p(st),
            w.B, w.T, w.H, w.Dk, w.Dv, chunk)
    if noalloc:
        opts = _opts(d)
        status = lib.delta_rule_chunk_fwd_noalloc(*args, ctypes.byref(opts), code, stream)
    else:
        need = int(lib.delta_rule_chunk_fwd_workspace_bytes(w.B, w.T, w.H, w.Dk, w.Dv, chunk,
                                                            code))
        ws = torch.full((max(need, 16),), 0xFF, dtype=torch.uint8, device="cuda")
        opts = _opts(d, ws if need > 0 else None)
        status = lib.delta_rule_chunk_fwd_ex(*args, ctypes.byref(opts), code, stream)
    torch.cuda.synchronize()
    return status, o, st


def _same_as_workspace_path(lib, w, x, chunk=64, oracle=True):
    d = to_dev(x)
    need = int(lib.delta_rule_chunk_fwd_workspace_bytes(w.B, w.T, w.H, w.Dk, w.Dv, chunk,
                                                        dr.DR_BF16))
    print(f"noalloc B{w.B} H{w.H} T{w.T} Dk{w.Dk} Dv{w.Dv} chunk {chunk}: segment scratch "
          f"{need} bytes", flush=True)
    s1, o1, st1 = _run(lib, w, d, True, chunk)
    s2, o2, st2 = _run(lib, w, d, False, chunk)
    assert s1 == dr.DR_OK and s2 == dr.DR_OK, (s1, s2)
    assert torch.equal(o1, o2), "o differs from the workspace entry point"
    assert torch.equal(st1, st2), "S_T differs from the workspace entry point"
    if oracle:
        o_ref, s_ref = oracle_all(x)
        assert rel_err(to_np(o1), o_ref) <= 2e-2
        assert rel_err(to_np(st1), s_ref) <= 2e-2
    return need


def test_two_calls_in_a_row_second_smaller(lib):
    # one long sequence per head (segment-parallel schedule), then a smaller
    # one with a different plan: the second must not see the first's scratch
    w1 = W.get("long_prefill", H=2, T=7000, seed=13000)
    n1 = _same_as_workspace_path(lib, w1, W.generate(w1))
    w2 = W.get("long_prefill", H=1, T=6200, Dv=64, seed=13001)
    n2 = _same_as_workspace_path(lib, w2, W.generate(w2))
    assert 0 < n2 < n1


def test_gated_and_kda_rules(lib):
    w = W.get("long_prefill", H=2, T=6600, gate_amax=1.0, seed=13100)
    _same_as_workspace_path(lib, w, W.generate(w))
    w = W.get("long_prefill", H=2, T=6500, gate_amax=16.0, kda=True, seed=13101)
    _same_as_workspace_path(lib, w, W.generate(w))


def test_shape_that_fills_the_gpu_uses_no_scratch(lib):
    # the plain schedule: equal to delta_rule_chunk_fwd
    w = W.get("layer_1p3b", B=4, T=256, seed=13200)
    assert lib.delta_rule_chunk_fwd_workspace_bytes(w.B, w.T, w.H, w.Dk, w.Dv, 64,
                                                    dr.DR_BF16) == 0
    x = W.generate(w)
    d = to_dev(x)
    s1, o1, st1 = _run(lib, w, d, True, 64)
    assert s1 == dr.DR_OK
    o2, st2 = dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["S0"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(st1, st2)


def test_plan_beyond_the_static_scratch_enqueues_nothing(lib):
    w = W.get("long_prefill", H=4, T=65536, Dv=64, s0_std=0.0, seed=13300)
    need = int(lib.delta_rule_chunk_fwd_workspace_bytes(w.B, w.T, w.H, w.Dk, w.Dv, 64,
                                                        dr.DR_BF16))
    assert need > dr.DR_STATIC_SCRATCH_BYTES
    z = lambda *s: torch.zeros(*s, dtype=torch.bfloat16, device="cuda")
    d = {"q": z(1, w.T, w.H, w.Dk), "k": z(1, w.T, w.H, w.Dk), "v": z(1, w.T, w.H, w.Dv),
         "beta": z(1, w.T, w.H), "S0": None}
    status, o, st = _run(lib, w, d, True, 64)
    assert status == dr.DR_ERR_SCRATCH
    assert torch.isnan(o).all() and torch.isnan(st).all()
    with pytest.raises(dr.DeltaRuleScratchError):
        dr.delta_rule_chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["beta"])
