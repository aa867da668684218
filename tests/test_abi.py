"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function ``include/deltarule.h``
declares, and reject bad arguments on the host before any HIP call.  Only
rejected calls are made here: a call that passes validation would enqueue GPU
work, which this suite never does.
"""
from __future__ import annotations

import ctypes
import glob
import os
import re

import pytest

import deltanet_delta_rule_amd as dr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Fake device addresses: valid-looking and 16-byte aligned, far apart, never
# dereferenced because every call below fails validation first.
P = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(8)]
MISALIGNED = ctypes.c_void_p(0x100000 * 9 + 4)   # element-aligned, not 16-byte
ODD = ctypes.c_void_p(0x100000 * 9 + 1)          # not even element-aligned


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dr.LIB_PATH):
        from deltanet_delta_rule_amd import build
        build.build()
    return dr.load_library()


def _declared_functions():
    names = set()
    for path in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b([A-Za-z_]\w*)\s*\(", text):
            name = m.group(1)
            if name.startswith(("delta_rule_", "gated_delta_rule_")):
                names.add(name)
    return sorted(names)


def test_header_declares_entry_points():
    names = _declared_functions()
    assert "delta_rule_chunk_fwd" in names
    assert "delta_rule_recurrent_step" in names
    assert "gated_delta_rule_chunk_fwd" in names
    assert "gated_delta_rule_recurrent_step" in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), f"libdeltarule.so does not export {name}"


def test_status_strings_and_version(lib):
    for code in range(5):
        s = dr.delta_rule_status_string(code)
        assert s.startswith("DR_")
    assert "unknown" in dr.delta_rule_status_string(99)
    assert dr.delta_rule_version() >= 100
    assert lib.delta_rule_last_hip_error() == 0


def _chunk(lib, q=P[0], k=P[1], v=P[2], beta=P[3], S0=None, o=P[4], S_T=P[5],
           B=2, T=64, H=2, Dk=64, Dv=64, chunk=64, dtype=dr.DR_BF16):
    return lib.delta_rule_chunk_fwd(q, k, v, beta, S0, o, S_T, B, T, H, Dk, Dv,
                                    chunk, dtype, None)


def _step(lib, q=P[0], k=P[1], v=P[2], beta=P[3], S=P[4], o=P[5], B=2, H=2,
          Dk=64, Dv=64, dtype=dr.DR_BF16):
    return lib.delta_rule_recurrent_step(q, k, v, beta, S, o, B, H, Dk, Dv,
                                         dtype, None)


@pytest.mark.parametrize("kw", [
    dict(B=-1), dict(T=-1), dict(H=-1), dict(chunk=-16), dict(dtype=7),
    dict(q=None), dict(k=None), dict(v=None), dict(beta=None), dict(o=None),
    dict(q=MISALIGNED), dict(k=MISALIGNED), dict(S0=MISALIGNED),
    dict(S_T=MISALIGNED), dict(v=ODD), dict(beta=ODD), dict(o=ODD),
    dict(o=MISALIGNED),              # the chunked kernels store o in 8/16-byte vectors
    dict(o=P[0]),                    # output overlaps q
    dict(S_T=P[1]),                  # final state overlaps k
    dict(S0=P[6], S_T=P[4]),         # final state overlaps o
])
def test_chunk_rejects_invalid(lib, kw):
    assert _chunk(lib, **kw) == dr.DR_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [
    dict(Dk=48), dict(Dv=8), dict(Dk=256), dict(chunk=8), dict(chunk=128),
    dict(chunk=48), dict(T=2 ** 31),
    dict(B=1, H=2 ** 21, Dk=128, Dv=128),   # one chunk of all heads exceeds 2^30 bytes
])
def test_chunk_rejects_unsupported(lib, kw):
    assert _chunk(lib, **kw) == dr.DR_ERR_UNSUPPORTED


def test_chunk_empty_batch_is_a_no_op(lib):
    # B or H zero: nothing to do, no HIP call
    assert _chunk(lib, B=0) == dr.DR_OK
    assert _chunk(lib, H=0, q=None, k=None) == dr.DR_OK


@pytest.mark.parametrize("kw", [
    dict(B=-3), dict(dtype=2), dict(q=None), dict(S=None), dict(o=None),
    dict(q=MISALIGNED), dict(S=MISALIGNED), dict(beta=ODD), dict(v=ODD),
    dict(o=P[4]),                          # o overlaps S
    dict(S=P[2]),                          # state overlaps v
])
def test_step_rejects_invalid(lib, kw):
    assert _step(lib, **kw) == dr.DR_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(Dk=24), dict(Dv=512), dict(Dk=8)])
def test_step_rejects_unsupported(lib, kw):
    assert _step(lib, **kw) == dr.DR_ERR_UNSUPPORTED


def test_step_empty_batch_is_a_no_op(lib):
    assert _step(lib, B=0) == dr.DR_OK


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 4, 1, 16)
    with pytest.raises(ValueError):
        dr.delta_rule_chunk_fwd(x, x, x, x[..., 0])
    with pytest.raises(ValueError):
        dr.delta_rule_recurrent_step(x[:, 0], x[:, 0], x[:, 0], x[:, 0, :, 0],
                                     torch.zeros(1, 1, 16, 16))


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(dr, "_lib", None)
    monkeypatch.setattr(dr, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        dr.load_library()


# ------------------------------------------------------------- gated rule
GP = ctypes.c_void_p(0x100000 * 7)   # the log gates, apart from every other buffer


def _gchunk(lib, g=GP, q=P[0], k=P[1], v=P[2], beta=P[3], S0=None, o=P[4], S_T=P[5],
            B=2, T=64, H=2, Dk=64, Dv=64, chunk=64, dtype=dr.DR_BF16):
    return lib.gated_delta_rule_chunk_fwd(q, k, v, beta, g, S0, o, S_T, B, T, H, Dk, Dv,
                                          chunk, dtype, None)


def _gstep(lib, g=GP, q=P[0], k=P[1], v=P[2], beta=P[3], S=P[4], o=P[5], B=2, H=2,
           Dk=64, Dv=64, dtype=dr.DR_BF16):
    return lib.gated_delta_rule_recurrent_step(q, k, v, beta, g, S, o, B, H, Dk, Dv,
                                               dtype, None)


@pytest.mark.parametrize("kw", [
    dict(g=None),                    # the gate is required when T > 0
    dict(g=ODD),                     # not 4-byte aligned
    dict(g=P[4]),                    # gates overlap the output
    dict(S_T=GP),                    # final state overlaps the gates
    dict(B=-1), dict(q=None), dict(o=P[0]),
])
def test_gated_chunk_rejects_invalid(lib, kw):
    assert _gchunk(lib, **kw) == dr.DR_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(Dk=48), dict(chunk=128), dict(Dv=8)])
def test_gated_chunk_rejects_unsupported(lib, kw):
    assert _gchunk(lib, **kw) == dr.DR_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [
    dict(g=None), dict(g=ODD),
    dict(g=P[4]),                    # gates overlap the state
    dict(o=GP),                      # output overlaps the gates
    dict(S=None), dict(q=MISALIGNED),
])
def test_gated_step_rejects_invalid(lib, kw):
    assert _gstep(lib, **kw) == dr.DR_ERR_INVALID_ARG


def test_gated_empty_batch_is_a_no_op(lib):
    assert _gchunk(lib, B=0) == dr.DR_OK
    assert _gstep(lib, H=0) == dr.DR_OK


def test_gated_binding_checks_the_gate():
    import torch
    x = torch.zeros(1, 4, 1, 16)
    with pytest.raises(ValueError):
        dr.gated_delta_rule_chunk_fwd(x, x, x, x[..., 0], x[..., 0])
    with pytest.raises(ValueError):
        dr.gated_delta_rule_recurrent_step(x[:, 0], x[:, 0], x[:, 0], x[:, 0, :, 0],
                                           x[:, 0, :, 0], torch.zeros(1, 1, 16, 16))


# ------------------------------------------------- extended chunked forward
CU = ctypes.c_void_p(0x100000 * 8)   # sequence offsets, apart from every other buffer


def _ex(lib, opts=None, q=P[0], k=P[1], v=P[2], beta=P[3], S0=None, o=P[4], S_T=P[5],
        B=1, T=64, H=2, Dk=64, Dv=64, chunk=64, dtype=dr.DR_BF16):
    return lib.delta_rule_chunk_fwd_ex(q, k, v, beta, S0, o, S_T, B, T, H, Dk, Dv, chunk,
                                       None if opts is None else ctypes.byref(opts), dtype, None)


def _opts(**kw):
    o = dr.dr_chunk_opts(g=None, cu_seqlens=None, num_seqs=0, scale=1.0, flags=0, gk=None,
                         workspace=None, workspace_bytes=0)
    for name, val in kw.items():
        setattr(o, name, val)
    return o


def test_chunk_options_struct_layout():
    # pointer, pointer, int64, float, uint32, pointer, pointer, int64: 56 bytes
    assert ctypes.sizeof(dr.dr_chunk_opts) == 56
    assert dr.dr_chunk_opts.scale.offset == 24 and dr.dr_chunk_opts.flags.offset == 28
    assert dr.dr_chunk_opts.gk.offset == 32
    assert dr.dr_chunk_opts.workspace.offset == 40
    assert dr.dr_chunk_opts.workspace_bytes.offset == 48


@pytest.mark.parametrize("kw, call", [
    (dict(cu_seqlens=CU.value, num_seqs=3), dict(B=2)),          # packed needs B == 1
    (dict(cu_seqlens=CU.value, num_seqs=-1), {}),                # negative count
    (dict(cu_seqlens=ODD.value, num_seqs=2), {}),                # misaligned offsets
    (dict(cu_seqlens=P[4].value, num_seqs=2), {}),               # offsets overlap o
    (dict(cu_seqlens=CU.value, num_seqs=2), dict(S_T=CU)),       # S_T overlaps offsets
    (dict(scale=float("nan")), {}),
    (dict(scale=float("inf")), {}),
    (dict(flags=4), {}),                                         # unknown flag bit
    (dict(flags=0x80000001), {}),
    (dict(g=ODD.value), {}),                                     # gate misaligned
    (dict(g=P[4].value), {}),                                    # gate overlaps o
    (dict(gk=MISALIGNED.value), {}),                             # channel decay misaligned
    (dict(gk=P[4].value), {}),                                   # channel decay overlaps o
    (dict(gk=P[7].value, g=P[6].value), {}),                     # both decay kinds
    (dict(gk=P[7].value, flags=3), dict(S_T=P[7])),              # S_T overlaps gk
    (dict(workspace=MISALIGNED.value, workspace_bytes=1 << 20), {}),   # workspace misaligned
    (dict(workspace=P[4].value, workspace_bytes=1 << 20), {}),         # workspace overlaps o
    (dict(workspace=P[1].value, workspace_bytes=1 << 20), {}),         # workspace overlaps k
    (dict(workspace=P[6].value, workspace_bytes=1 << 20, gk=P[6].value + 4096), {}),  # and gk
    (dict(workspace=P[7].value, workspace_bytes=-1), {}),              # negative size
])
def test_chunk_ex_rejects_invalid(lib, kw, call):
    assert _ex(lib, _opts(**kw), **call) == dr.DR_ERR_INVALID_ARG


def test_chunk_ex_rejects_unsupported(lib):
    assert _ex(lib, _opts(scale=0.5), Dk=48) == dr.DR_ERR_UNSUPPORTED
    assert _ex(lib, None, chunk=128) == dr.DR_ERR_UNSUPPORTED


def test_chunk_ex_no_sequences_is_a_no_op(lib):
    assert _ex(lib, _opts(cu_seqlens=CU.value, num_seqs=0)) == dr.DR_OK
    assert _ex(lib, _opts(scale=2.0), H=0) == dr.DR_OK


# ------------------------------------------------- extended decode step
def _sx(lib, opts=None, q=P[0], k=P[1], v=P[2], beta=P[3], S=P[4], o=P[5], B=2, H=2,
        Dk=64, Dv=64, dtype=dr.DR_BF16):
    return lib.delta_rule_recurrent_step_ex(q, k, v, beta, S, o, B, H, Dk, Dv,
                                            None if opts is None else ctypes.byref(opts),
                                            dtype, None)


def test_step_options_struct_layout():
    assert ctypes.sizeof(dr.dr_step_opts) == 24
    assert dr.dr_step_opts.scale.offset == 8 and dr.dr_step_opts.flags.offset == 12
    assert dr.dr_step_opts.gk.offset == 16


@pytest.mark.parametrize("kw, call", [
    (dict(scale=float("nan")), {}), (dict(scale=float("-inf")), {}),
    (dict(flags=4), {}), (dict(g=ODD.value), {}), (dict(g=P[4].value), {}),
    (dict(scale=2.0), dict(S=None)), (dict(flags=1), dict(q=MISALIGNED)),
    (dict(gk=MISALIGNED.value), {}),                       # per-channel decay misaligned
    (dict(gk=P[4].value), {}),                             # overlaps S
    (dict(gk=P[7].value, g=P[6].value), {}),               # both decay kinds
])
def test_step_ex_rejects_invalid(lib, kw, call):
    o = dr.dr_step_opts(g=None, scale=1.0, flags=0, gk=None)
    for n, val in kw.items():
        setattr(o, n, val)
    assert _sx(lib, o, **call) == dr.DR_ERR_INVALID_ARG


def test_step_ex_unsupported_and_empty(lib):
    o = dr.dr_step_opts(g=None, scale=1.0, flags=1, gk=None)
    assert _sx(lib, o, Dk=24) == dr.DR_ERR_UNSUPPORTED
    assert _sx(lib, o, B=0) == dr.DR_OK


# ---------------------------------------------------------------- backward
def test_backward_workspace_size(lib):
    f = lib.delta_rule_chunk_bwd_workspace_bytes
    # bf16: 32-token chunks, bf16 states; fp32: 16-token chunks, fp32 states;
    # one state per chunk and head (the forward checkpoints), as much again
    # for the gradients of the chunk states, and one [B,T,H,Dv] tensor of the
    # input dtype (the solve's Z), each part rounded up to 256 bytes
    al = lambda x: (x + 255) // 256 * 256
    assert f(2, 100, 3, 64, 32, dr.DR_BF16) == 2 * al(2 * 3 * 4 * 32 * 64 * 2) + al(2 * 100 * 3 * 32 * 2)
    assert f(2, 100, 3, 64, 32, dr.DR_F32) == 2 * al(2 * 3 * 7 * 32 * 64 * 4) + al(2 * 100 * 3 * 32 * 4)
    assert f(1, 3, 1, 16, 16, dr.DR_BF16) == 2 * al(16 * 16 * 2) + al(3 * 16 * 2)
    assert f(1, 0, 1, 16, 16, dr.DR_BF16) == 0
    # few (b, h) and enough chunks: the segments' maps of the state-gradient
    # recursion follow, P segments of fp32 [Dv,Dk] responses and [Dk,Dk] maps
    # per (b, h): 128 / (B H) segments, at most 16 and of at least 4 chunks,
    # used from 4 segments and up to 32 (b, h)
    base = lambda B, T, H, Dk, Dv: (2 * al(B * H * (T // 32) * Dv * Dk * 2) +
                                    al(B * T * H * Dv * 2))
    assert f(1, 2048, 16, 128, 128, dr.DR_BF16) == base(1, 2048, 16, 128, 128) + \
        2 * al(8 * 16 * 128 * 128 * 4)                          # 8 segments of 8 chunks
    assert f(1, 512, 16, 128, 64, dr.DR_BF16) == base(1, 512, 16, 128, 64) + \
        al(4 * 16 * 64 * 128 * 4) + al(4 * 16 * 128 * 128 * 4)  # 4 segments of 4 chunks
    assert f(2, 2048, 16, 64, 64, dr.DR_BF16) == base(2, 2048, 16, 64, 64) + \
        2 * al(2 * 4 * 16 * 64 * 64 * 4)                        # 32 (b, h): 4 segments
    assert f(4, 2048, 16, 64, 64, dr.DR_BF16) == base(4, 2048, 16, 64, 64)   # 64 (b, h): none
    assert f(1, 448, 16, 64, 64, dr.DR_BF16) == base(1, 448, 16, 64, 64)     # 14 chunks: 3 segments
    assert f(1, 10, 1, 24, 16, dr.DR_BF16) == 0   # unsupported size
    assert f(-1, 10, 1, 16, 16, dr.DR_BF16) == 0


def _bwd(lib, ws=P[7], wsb=1 << 40, q=P[0], k=P[1], v=P[2], beta=P[3], dout=P[4], dq=P[5],
         dk=P[6], dv=ctypes.c_void_p(0x100000 * 10), dbeta=ctypes.c_void_p(0x100000 * 11),
         dS0=None, S0=None, dST=None, B=1, T=64, H=2, Dk=64, Dv=64, dtype=dr.DR_BF16):
    return lib.delta_rule_chunk_bwd(q, k, v, beta, S0, dout, dST, dq, dk, dv, dbeta, dS0, ws,
                                    wsb, B, T, H, Dk, Dv, dtype, None)


@pytest.mark.parametrize("kw", [
    dict(ws=None), dict(wsb=16), dict(ws=MISALIGNED), dict(dout=None), dict(dq=None),
    dict(dq=P[0]),                   # output overlaps q
    dict(dk=P[5]),                   # two outputs overlap
    dict(ws=P[4]),                   # workspace overlaps do
    dict(dbeta=ODD), dict(B=-1), dict(dtype=5),
])
def test_backward_rejects_invalid(lib, kw):
    assert _bwd(lib, **kw) == dr.DR_ERR_INVALID_ARG


def _fwdck(lib, ws=P[7], wsb=1 << 40, q=P[0], k=P[1], v=P[2], beta=P[3], g=None, S0=None,
           o=P[5], ST=None, B=1, T=64, H=2, Dk=64, Dv=64, dtype=dr.DR_BF16):
    return lib.delta_rule_chunk_fwd_checkpointed(q, k, v, beta, g, S0, o, ST, ws, wsb, B, T, H,
                                                 Dk, Dv, dtype, None)


@pytest.mark.parametrize("kw", [
    dict(ws=None), dict(wsb=16), dict(ws=MISALIGNED), dict(o=None), dict(q=None),
    dict(o=P[0]),                    # output overlaps q
    dict(ws=P[1]),                   # checkpoints over k
    dict(ws=P[5]),                   # checkpoints over o
    dict(ST=P[7]),                   # final state over the checkpoints
    dict(B=-1), dict(dtype=5),
])
def test_checkpointed_forward_rejects_invalid(lib, kw):
    assert _fwdck(lib, **kw) == dr.DR_ERR_INVALID_ARG


def test_checkpointed_forward_rejects_unsupported_and_empty(lib):
    assert _fwdck(lib, Dk=48) == dr.DR_ERR_UNSUPPORTED
    assert _fwdck(lib, B=0) == dr.DR_OK
    assert _fwdck(lib, H=0) == dr.DR_OK


def _bwdx(lib, flags=1, g=None, dg=None, ws=P[7], wsb=1 << 40, q=P[0], k=P[1], v=P[2],
          beta=P[3], dout=P[4], dq=P[5], dk=P[6], dv=ctypes.c_void_p(0x100000 * 10),
          dbeta=ctypes.c_void_p(0x100000 * 11), dS0=None, S0=None, dST=None, B=1, T=64, H=2,
          Dk=64, Dv=64, dtype=dr.DR_BF16):
    return lib.delta_rule_chunk_bwd_ex(q, k, v, beta, g, S0, dout, dST, dq, dk, dv, dbeta, dg,
                                       dS0, ws, wsb, B, T, H, Dk, Dv, flags, dtype, None)


@pytest.mark.parametrize("kw", [
    dict(flags=2), dict(flags=0xffffffff),          # unknown flag bits
    dict(ws=None), dict(wsb=16), dict(dq=P[0]),
    dict(g=ctypes.c_void_p(0x100000 * 12)),          # gated without dg
    dict(dtype=5),
])
def test_backward_ex_rejects_invalid(lib, kw):
    assert _bwdx(lib, **kw) == dr.DR_ERR_INVALID_ARG


def test_backward_rejects_unsupported_and_empty(lib):
    assert _bwd(lib, Dk=48) == dr.DR_ERR_UNSUPPORTED
    assert _bwd(lib, B=0) == dr.DR_OK


def _gbwd(lib, g=ctypes.c_void_p(0x100000 * 12), dg=ctypes.c_void_p(0x100000 * 13), ws=P[7],
          wsb=1 << 40, q=P[0], k=P[1], v=P[2], beta=P[3], dout=P[4], dq=P[5], dk=P[6],
          dv=ctypes.c_void_p(0x100000 * 10), dbeta=ctypes.c_void_p(0x100000 * 11), dS0=None,
          S0=None, dST=None, B=1, T=64, H=2, Dk=64, Dv=64, dtype=dr.DR_BF16):
    return lib.gated_delta_rule_chunk_bwd(q, k, v, beta, g, S0, dout, dST, dq, dk, dv, dbeta,
                                          dg, dS0, ws, wsb, B, T, H, Dk, Dv, dtype, None)


@pytest.mark.parametrize("kw", [
    dict(g=None), dict(dg=None),     # both required when T > 0
    dict(g=ODD), dict(dg=ctypes.c_void_p(0x100000 * 13 + 2)),   # not 4-byte aligned
    dict(dg=P[3]),                   # dg overlaps beta
    dict(dg=P[5]),                   # dg overlaps dq
    dict(dg=P[7]),                   # dg overlaps the workspace
    dict(dq=ctypes.c_void_p(0x100000 * 12)),   # an output overlaps g
    dict(ws=None), dict(dout=None), dict(dtype=7),
])
def test_gated_backward_rejects_invalid(lib, kw):
    assert _gbwd(lib, **kw) == dr.DR_ERR_INVALID_ARG


def test_gated_backward_rejects_unsupported_and_empty(lib):
    assert _gbwd(lib, Dv=40) == dr.DR_ERR_UNSUPPORTED
    assert _gbwd(lib, H=0) == dr.DR_OK


# ------------------------------------------ per-channel-decay backward
def test_kda_backward_workspace_size(lib):
    f = lib.kda_bwd_workspace_bytes
    f.restype = ctypes.c_int64
    f.argtypes = [ctypes.c_int64] * 6
    # the state of every row tile at every 16-token block start of every
    # sequence (B*T/16 + sequences blocks), then fp32 partials of dq, dk, dgk
    # ([tiles, B*T*H, Dk] each) and of dbeta; rows per tile = lanes (at most
    # 512, 128 rows' worth) / (Dk / 8) lanes per row (Dk 128: 32, 64: 64, 32
    # and 16: 128); from Dk = 64, twice that (two rows per lane) when one
    # would need more than 256 workgroups, half (half the lanes) when it
    # would need at most 128; each part rounded up to 256 bytes
    al = lambda x: (x + 255) // 256 * 256

    def want(B, T, H, Dk, Dv, n):
        rl = {128: 32, 64: 64, 32: 128, 16: 128}[Dk]
        wg = n * H * -(-Dv // rl)
        rw = rl if Dk < 64 else 2 * rl if wg > 256 else rl // 2 if 2 * wg <= 256 else rl
        R = -(-Dv // rw)
        ck = (B * T // 16 + n) * H * R * rw * Dk * 4
        return al(ck) + al(3 * R * B * T * H * Dk * 4) + al(R * B * T * H * 4)

    assert f(8, 2048, 16, 128, 128, 8) == want(8, 2048, 16, 128, 128, 8)
    assert f(2, 77, 3, 64, 32, 2) == want(2, 77, 3, 64, 32, 2)
    assert f(1, 300, 2, 16, 64, 5) == want(1, 300, 2, 16, 64, 5)
    assert f(2, 40, 130, 64, 64, 2) == want(2, 40, 130, 64, 64, 2)    # two rows per lane
    assert f(1, 40, 70, 128, 128, 1) == want(1, 40, 70, 128, 128, 1)  # two rows per lane
    assert f(1, 40, 64, 128, 128, 1) == want(1, 40, 64, 128, 128, 1)  # one: 256 workgroups
    assert f(1, 40, 40, 128, 128, 1) == want(1, 40, 40, 128, 128, 1)  # 160: full width
    assert f(1, 2048, 16, 128, 128, 1) == want(1, 2048, 16, 128, 128, 1)  # 64: half width
    assert f(1, 0, 2, 32, 32, 1) == want(1, 0, 2, 32, 32, 1)
    assert f(1, 10, 1, 24, 16, 1) == -1      # unsupported size
    assert f(-1, 10, 1, 16, 16, 1) == -1


def _kbwd(lib, gk=ctypes.c_void_p(0x100000 * 12), dgk=ctypes.c_void_p(0x100000 * 13), ws=P[7],
          wsb=1 << 40, q=P[0], k=P[1], v=P[2], beta=P[3], dout=P[4], dq=P[5], dk=P[6],
          dv=ctypes.c_void_p(0x100000 * 10), dbeta=ctypes.c_void_p(0x100000 * 11), dS0=None,
          S0=None, dST=None, cu=None, nseq=0, scale=1.0, B=1, T=64, H=2, Dk=64, Dv=64,
          dtype=dr.DR_BF16):
    return lib.kda_bwd(q, k, v, beta, gk, S0, dout, dST, dq, dk, dv, dbeta, dgk, dS0, cu, nseq,
                       scale, ws, wsb, B, T, H, Dk, Dv, dtype, None)


@pytest.mark.parametrize("kw", [
    dict(gk=None), dict(dgk=None),   # both required when T > 0
    dict(gk=MISALIGNED), dict(dgk=ctypes.c_void_p(0x100000 * 13 + 4)),  # 16-byte vectors
    dict(dgk=P[1]),                  # dgk overlaps k
    dict(dgk=P[7]),                  # dgk overlaps the workspace
    dict(dq=ctypes.c_void_p(0x100000 * 12)),   # an output overlaps gk
    dict(ws=None), dict(wsb=16), dict(dout=None), dict(dv=None),
    dict(scale=float("nan")), dict(scale=float("inf")),
    dict(cu=P[7], nseq=2, B=2),      # packed sequences need B = 1
    dict(cu=ctypes.c_void_p(0x100000 * 14 + 2), nseq=2),   # misaligned offsets
    dict(cu=P[5], nseq=2),           # offsets overlap an output
    dict(B=-1), dict(dtype=3),
])
def test_kda_backward_rejects_invalid(lib, kw):
    assert _kbwd(lib, **kw) == dr.DR_ERR_INVALID_ARG


def test_kda_backward_rejects_unsupported_and_empty(lib):
    assert _kbwd(lib, Dk=48) == dr.DR_ERR_UNSUPPORTED
    assert _kbwd(lib, Dv=24) == dr.DR_ERR_UNSUPPORTED
    assert _kbwd(lib, B=0) == dr.DR_OK
    assert _kbwd(lib, H=0) == dr.DR_OK
    assert _kbwd(lib, cu=ctypes.c_void_p(0x100000 * 14), nseq=0) == dr.DR_OK


# ------------------------------------------- segment-parallel workspace size
def test_chunk_fwd_workspace_bytes(lib):
    f = lib.delta_rule_chunk_fwd_workspace_bytes
    f.restype = ctypes.c_int64
    f.argtypes = [ctypes.c_int64] * 6 + [ctypes.c_int]
    # one long prefill (B1 H16 T32768 d128): 8 segments of 4096 tokens;
    # H_p / S_in and M_p in fp32 plus the offsets
    seg = 8 * 16 * 128 * 128 * 4
    assert f(1, 32768, 16, 128, 128, 64, dr.DR_BF16) == 2 * seg + 256
    # the 1.3B layer shape fills the GPU with the plain schedule
    assert f(8, 2048, 16, 128, 128, 64, dr.DR_BF16) == 0
    # too short to cut into six segments of sixteen chunks
    assert f(1, 6000, 2, 128, 128, 64, dr.DR_BF16) == 0
    # the small-model shape (B4 H8 T2048 d64): with d_k <= 64 segments may be
    # as short as 4 chunks, so 8 segments of 256 tokens
    seg64 = 4 * 8 * 8 * 64 * 64 * 4
    assert f(4, 2048, 8, 64, 64, 64, dr.DR_BF16) == 2 * seg64 + 256
    # ... but not shorter: 2 chunks per segment would be needed here
    assert f(4, 1024, 8, 64, 64, 64, dr.DR_BF16) == 0
    assert f(1, 0, 16, 128, 128, 64, dr.DR_BF16) == 0
    # invalid arguments
    assert f(1, 32768, 16, 48, 128, 64, dr.DR_BF16) == -1
    assert f(1, 32768, 16, 128, 128, 100, dr.DR_BF16) == -1
    assert f(1, 32768, 16, 128, 128, 64, 7) == -1


# ------------------------------------------------ chunked forward, no allocation
def _na(lib, opts=None, q=P[0], k=P[1], v=P[2], beta=P[3], S0=None, o=P[4], S_T=P[5],
        B=1, T=64, H=2, Dk=64, Dv=64, chunk=64, dtype=dr.DR_BF16):
    return lib.delta_rule_chunk_fwd_noalloc(q, k, v, beta, S0, o, S_T, B, T, H, Dk, Dv, chunk,
                                            None if opts is None else ctypes.byref(opts),
                                            dtype, None)


@pytest.mark.parametrize("kw, call", [
    (dict(workspace=P[7].value, workspace_bytes=1 << 20), {}),   # the scratch is the library's
    (dict(workspace_bytes=1 << 20), {}),
    (dict(flags=4), {}), (dict(scale=float("nan")), {}),
    ({}, dict(o=P[0])), ({}, dict(q=MISALIGNED)), ({}, dict(B=-1)),
])
def test_noalloc_rejects_invalid(lib, kw, call):
    assert _na(lib, _opts(**kw), **call) == dr.DR_ERR_INVALID_ARG


def test_noalloc_rejects_a_plan_beyond_the_static_scratch(lib):
    # B1 H4 T65536, d_k 128, d_v 64: 64 segments, H_p 8 MiB + M_p 16 MiB, more
    # than DR_STATIC_SCRATCH_BYTES; refused before any HIP call (fake
    # pointers 4 GiB apart)
    f = lib.delta_rule_chunk_fwd_workspace_bytes
    need = f(1, 65536, 4, 128, 64, 64, dr.DR_BF16)
    assert need > dr.DR_STATIC_SCRATCH_BYTES
    far = [ctypes.c_void_p((1 << 32) * (i + 1)) for i in range(6)]
    st = _na(lib, None, q=far[0], k=far[1], v=far[2], beta=far[3], o=far[4], S_T=far[5],
             T=65536, H=4, Dk=128, Dv=64)
    assert st == dr.DR_ERR_SCRATCH
    assert "DR_ERR_SCRATCH" in dr.delta_rule_status_string(st)
    assert lib.delta_rule_last_hip_error() == 0


def test_static_scratch_holds_every_plan_with_128_value_rows(lib):
    # the segment count is capped by the GPU's 256 CUs, so with d_v = 128 the
    # largest plan (d_k = 128) needs 16 MiB + a few hundred bytes
    f = lib.delta_rule_chunk_fwd_workspace_bytes
    worst = max(f(B, T, H, 128, 128, c, dr.DR_BF16)
                for B in (1, 2, 4) for H in (1, 2, 4, 8, 16)
                for T in (8192, 32768, 262144) for c in (16, 32, 64))
    assert 0 < worst <= dr.DR_STATIC_SCRATCH_BYTES
