"""MI355X-native DeltaNet delta-rule operator.

A thin ctypes binding over ``libdeltarule.so`` (HIP kernels for gfx950 behind
the C ABI of ``include/deltarule.h``).  The functions below carry the C entry
points' names and only marshal arguments: they check devices, dtypes, shapes
and contiguity, allocate missing outputs with torch, and pass raw device
pointers plus torch's current HIP stream.  Every step of the operator runs in
the library's kernels; there is no CPU or PyTorch fallback.  If the library
is not built, the first call raises.

    o, S_T = delta_rule_chunk_fwd(q, k, v, beta, S0=None, chunk=64)
    o      = delta_rule_recurrent_step(q, k, v, beta, S)   # S updated in place

and the gated rule (g = log of the per-token, per-head forget gate, fp32):

    o, S_T = gated_delta_rule_chunk_fwd(q, k, v, beta, g, S0=None, chunk=64)
    o      = gated_delta_rule_recurrent_step(q, k, v, beta, g, S)

Both chunked calls also take ``scale=`` (output scale), ``cu_seqlens=``
(packed variable-length sequences in one batch row) and
``use_qk_l2norm_in_kernel=``, which route them to ``delta_rule_chunk_fwd_ex``.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "delta_rule_chunk_fwd",
    "delta_rule_recurrent_step",
    "gated_delta_rule_chunk_fwd",
    "gated_delta_rule_recurrent_step",
    "delta_rule_chunk_bwd",
    "gated_delta_rule_chunk_bwd",
    "delta_rule_chunk_fwd_checkpointed",
    "delta_rule_chunk_fwd_noalloc",
    "DeltaRuleScratchError",
    "kda_recurrent_step",
    "kda_fwd",
    "kda_bwd",
    "kda_bwd_workspace_bytes",
    "DR_FUSED_RECURRENT",
    "chunk_fwd_workspace_bytes",
    "delta_rule_status_string",
    "delta_rule_version",
    "DeltaRuleError",
    "LIB_PATH",
    "load_library",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdeltarule.so")

DR_OK, DR_ERR_INVALID_ARG, DR_ERR_UNSUPPORTED, DR_ERR_HIP, DR_ERR_SCRATCH = 0, 1, 2, 3, 4
# DR_STATIC_SCRATCH_BYTES of include/deltarule.h
DR_STATIC_SCRATCH_BYTES = 16 * 1024 * 1024 + 64 * 1024
DR_F32, DR_BF16 = 0, 1
DR_BWD_CHECKPOINTS_READY = 1

_lib = None


class dr_chunk_opts(ctypes.Structure):
    """``dr_chunk_opts`` of include/deltarule.h."""
    _fields_ = [("g", ctypes.c_void_p), ("cu_seqlens", ctypes.c_void_p),
                ("num_seqs", ctypes.c_int64), ("scale", ctypes.c_float),
                ("flags", ctypes.c_uint32), ("gk", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64)]


class dr_step_opts(ctypes.Structure):
    """``dr_step_opts`` of include/deltarule.h."""
    _fields_ = [("g", ctypes.c_void_p), ("scale", ctypes.c_float), ("flags", ctypes.c_uint32),
                ("gk", ctypes.c_void_p)]


class DeltaRuleError(RuntimeError):
    """A HIP runtime failure reported by libdeltarule."""


class DeltaRuleScratchError(RuntimeError):
    """delta_rule_chunk_fwd_noalloc: the shape needs more scratch than the
    library's static buffer holds (DR_ERR_SCRATCH)."""


def load_library():
    """Load libdeltarule.so (built in place by ``deltanet_delta_rule_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"libdeltarule.so is not built ({LIB_PATH}); run "
            "`python -m deltanet_delta_rule_amd.build` first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.delta_rule_chunk_fwd.restype = i32
    lib.delta_rule_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp,
                                         i64, i64, i64, i64, i64, i64, i32, vp]
    lib.delta_rule_recurrent_step.restype = i32
    lib.delta_rule_recurrent_step.argtypes = [vp, vp, vp, vp, vp, vp,
                                              i64, i64, i64, i64, i32, vp]
    lib.delta_rule_chunk_fwd_ex.restype = i32
    lib.delta_rule_chunk_fwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp,
                                            i64, i64, i64, i64, i64, i64,
                                            ctypes.POINTER(dr_chunk_opts), i32, vp]
    lib.delta_rule_chunk_fwd_noalloc.restype = i32
    lib.delta_rule_chunk_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp,
                                                 i64, i64, i64, i64, i64, i64,
                                                 ctypes.POINTER(dr_chunk_opts), i32, vp]
    lib.gated_delta_rule_chunk_fwd.restype = i32
    lib.gated_delta_rule_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp,
                                               i64, i64, i64, i64, i64, i64, i32, vp]
    lib.delta_rule_recurrent_step_ex.restype = i32
    lib.delta_rule_recurrent_step_ex.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                                 ctypes.POINTER(dr_step_opts), i32, vp]
    lib.gated_delta_rule_recurrent_step.restype = i32
    lib.gated_delta_rule_recurrent_step.argtypes = [vp, vp, vp, vp, vp, vp, vp,
                                                    i64, i64, i64, i64, i32, vp]
    lib.delta_rule_chunk_fwd_workspace_bytes.restype = i64
    lib.delta_rule_chunk_fwd_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, i32]
    lib.delta_rule_chunk_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.delta_rule_chunk_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i32]
    lib.delta_rule_chunk_bwd.restype = i32
    lib.delta_rule_chunk_bwd.argtypes = [vp] * 13 + [ctypes.c_size_t, i64, i64, i64, i64, i64,
                                                     i32, vp]
    lib.gated_delta_rule_chunk_bwd.restype = i32
    lib.gated_delta_rule_chunk_bwd.argtypes = [vp] * 15 + [ctypes.c_size_t, i64, i64, i64, i64,
                                                           i64, i32, vp]
    lib.delta_rule_chunk_fwd_checkpointed.restype = i32
    lib.delta_rule_chunk_fwd_checkpointed.argtypes = [vp] * 9 + [ctypes.c_size_t, i64, i64, i64,
                                                                 i64, i64, i32, vp]
    lib.delta_rule_chunk_bwd_ex.restype = i32
    lib.delta_rule_chunk_bwd_ex.argtypes = [vp] * 15 + [ctypes.c_size_t, i64, i64, i64, i64, i64,
                                                        ctypes.c_uint32, i32, vp]
    lib.kda_bwd_workspace_bytes.restype = i64
    lib.kda_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64]
    lib.kda_bwd.restype = i32
    lib.kda_bwd.argtypes = [vp] * 15 + [i64, ctypes.c_float, vp, ctypes.c_size_t,
                                        i64, i64, i64, i64, i64, i32, vp]
    lib.delta_rule_status_string.restype = ctypes.c_char_p
    lib.delta_rule_status_string.argtypes = [i32]
    lib.delta_rule_last_hip_error.restype = i32
    lib.delta_rule_last_hip_error.argtypes = []
    lib.delta_rule_version.restype = i32
    lib.delta_rule_version.argtypes = []
    _lib = lib
    return lib


def delta_rule_status_string(status: int) -> str:
    return load_library().delta_rule_status_string(int(status)).decode()


def delta_rule_version() -> int:
    return int(load_library().delta_rule_version())


def _check(status: int) -> None:
    if status == DR_OK:
        return
    msg = delta_rule_status_string(status)
    if status == DR_ERR_HIP:
        raise DeltaRuleError(f"{msg} (hipError {load_library().delta_rule_last_hip_error()})")
    if status == DR_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    if status == DR_ERR_SCRATCH:
        raise DeltaRuleScratchError(msg)
    raise ValueError(msg)


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return DR_F32
    if t.dtype == torch.bfloat16:
        return DR_BF16
    raise ValueError(f"q/k/v/beta must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, shape, dtype, device):
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


DR_QK_L2NORM = 1
DR_FUSED_RECURRENT = 2


def chunk_fwd_workspace_bytes(B, T, H, Dk, Dv, chunk=64, dtype=None):
    """Bytes of device workspace the segment-parallel schedule of the chunked
    forward needs for this shape, or 0 when the plain schedule already fills
    the GPU (``delta_rule_chunk_fwd_workspace_bytes``)."""
    torch = _torch()
    code = DR_F32 if dtype == torch.float32 else DR_BF16
    return int(load_library().delta_rule_chunk_fwd_workspace_bytes(B, T, H, Dk, Dv, chunk, code))


def _chunk_call(gated, q, k, v, beta, g, S0, chunk, output_final_state, o, S_T, stream,
                scale=None, cu_seqlens=None, l2norm=False, gk=None, recurrent=False,
                workspace=None):
    torch = _torch()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("the chunked forward needs GPU tensors")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    _dtype_code(q)
    _need(q, "q", (B, T, H, Dk), dt, dev)
    _need(k, "k", (B, T, H, Dk), dt, dev)
    _need(v, "v", (B, T, H, Dv), dt, dev)
    _need(beta, "beta", (B, T, H), dt, dev)
    if gated:
        _need(g, "g", (B, T, H), torch.float32, dev)
    if gk is not None:
        _need(gk, "gk", (B, T, H, Dk), torch.float32, dev)
    nseq = B
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError("packed sequences (cu_seqlens) need a batch of 1")
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
            raise ValueError("cu_seqlens must be a 1-D tensor of num_seqs + 1 offsets")
        if cu_seqlens.dtype != torch.int32:
            cu_seqlens = cu_seqlens.to(torch.int32)
        nseq = cu_seqlens.numel() - 1
        _need(cu_seqlens, "cu_seqlens", (nseq + 1,), torch.int32, dev)
    if S0 is not None:
        _need(S0, "S0", (nseq, H, Dv, Dk), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=dt, device=dev)
    else:
        _need(o, "o", (B, T, H, Dv), dt, dev)
    if output_final_state:
        if S_T is None:
            S_T = torch.empty((nseq, H, Dv, Dk), dtype=torch.float32, device=dev)
        else:
            _need(S_T, "S_T", (nseq, H, Dv, Dk), torch.float32, dev)
    else:
        S_T = None
    lib = load_library()
    common = (_ptr(q), _ptr(k), _ptr(v), _ptr(beta))
    tail = (B, T, H, Dk, Dv, int(chunk))
    # segment-parallel schedule for sequences too few to fill the GPU:
    # workspace=None allocates it when the library asks for one, False never,
    # "static" takes the library's static scratch (delta_rule_chunk_fwd_noalloc)
    ws_ptr, ws_bytes = None, 0
    noalloc = isinstance(workspace, str)
    if noalloc and workspace != "static":
        raise ValueError(f"workspace must be a tensor, None, False or 'static', not {workspace!r}")
    if (not noalloc and workspace is not False and cu_seqlens is None and not recurrent
            and T > 0):
        if workspace is None:
            need = lib.delta_rule_chunk_fwd_workspace_bytes(B, T, H, Dk, Dv, int(chunk),
                                                            _dtype_code(q))
            if need > 0:
                workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        if workspace is not None and workspace is not False:
            if workspace.device != dev or not workspace.is_contiguous():
                raise ValueError("workspace must be a contiguous tensor on the inputs' GPU")
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if (scale is None and cu_seqlens is None and not l2norm and gk is None and not recurrent
            and ws_ptr is None and not noalloc):
        if gated:
            st = lib.gated_delta_rule_chunk_fwd(*common, _ptr(g), _ptr(S0), _ptr(o), _ptr(S_T),
                                                *tail, _dtype_code(q), _stream(dev, stream))
        else:
            st = lib.delta_rule_chunk_fwd(*common, _ptr(S0), _ptr(o), _ptr(S_T), *tail,
                                          _dtype_code(q), _stream(dev, stream))
    else:
        opts = dr_chunk_opts(g=g.data_ptr() if gated else None,
                             cu_seqlens=None if cu_seqlens is None else cu_seqlens.data_ptr(),
                             num_seqs=nseq if cu_seqlens is not None else 0,
                             scale=1.0 if scale is None else float(scale),
                             flags=(DR_QK_L2NORM if l2norm else 0)
                             | (DR_FUSED_RECURRENT if recurrent else 0),
                             gk=None if gk is None else gk.data_ptr(),
                             workspace=ws_ptr, workspace_bytes=ws_bytes)
        entry = lib.delta_rule_chunk_fwd_noalloc if noalloc else lib.delta_rule_chunk_fwd_ex
        st = entry(*common, _ptr(S0), _ptr(o), _ptr(S_T), *tail, ctypes.byref(opts),
                   _dtype_code(q), _stream(dev, stream))
    _check(st)
    return o, S_T


def delta_rule_chunk_fwd(q, k, v, beta, S0=None, *, chunk: int = 64,
                         output_final_state: bool = True, o=None, S_T=None,
                         scale=None, cu_seqlens=None, use_qk_l2norm_in_kernel=False,
                         fused_recurrent=False, workspace=None, stream=None):
    """Chunkwise forward.  q, k ``[B,T,H,Dk]``; v ``[B,T,H,Dv]``; beta
    ``[B,T,H]`` (float32 or bfloat16, all the same dtype, on one GPU);
    S0 ``[B,H,Dv,Dk]`` float32 or None.  Returns ``(o, S_T)``; S_T is None
    when ``output_final_state`` is False.  ``o`` / ``S_T`` may be passed in
    (S_T may be S0 itself to carry the state in place).  ``scale`` multiplies
    the outputs; ``cu_seqlens`` (int32 ``[N+1]`` on the GPU, B = 1) packs N
    sequences, whose states S0 / S_T are then ``[N,H,Dv,Dk]``.
    ``use_qk_l2norm_in_kernel`` normalises the rows of q and k inside the
    kernel (x / sqrt(sum x^2 + 1e-6)).  ``fused_recurrent`` runs the
    token-serial schedule instead of the chunked one (same results up to
    rounding; for short sequences).  When the sequences are too few to fill
    the GPU, a device ``workspace`` (allocated here when None; pass False to
    disable) lets the library run the segment-parallel schedule."""
    return _chunk_call(False, q, k, v, beta, None, S0, chunk, output_final_state, o, S_T,
                       stream, scale, cu_seqlens, use_qk_l2norm_in_kernel,
                       recurrent=fused_recurrent, workspace=workspace)


def delta_rule_chunk_fwd_noalloc(q, k, v, beta, S0=None, *, g=None, gk=None, chunk: int = 64,
                                 output_final_state: bool = True, o=None, S_T=None,
                                 scale=None, cu_seqlens=None, use_qk_l2norm_in_kernel=False,
                                 fused_recurrent=False, stream=None):
    """The chunked forward of any rule (plain; gated with ``g``; KDA with
    ``gk``) with the segment-parallel schedule's scratch taken from the
    library's static per-GPU buffer instead of a workspace
    (``delta_rule_chunk_fwd_noalloc``): the library allocates nothing.  Pass
    ``o`` (and ``S_T``) to allocate nothing here either.  Raises
    ``DeltaRuleScratchError`` when the shape's schedule needs more than
    ``DR_STATIC_SCRATCH_BYTES``.  Calls that overlap in time on one GPU race on
    that buffer."""
    if g is not None and gk is not None:
        raise ValueError("g and gk are exclusive")
    return _chunk_call(g is not None, q, k, v, beta, g, S0, 64 if gk is not None else chunk,
                       output_final_state, o, S_T, stream, scale, cu_seqlens,
                       use_qk_l2norm_in_kernel, gk=gk, recurrent=fused_recurrent,
                       workspace="static")


def gated_delta_rule_chunk_fwd(q, k, v, beta, g, S0=None, *, chunk: int = 64,
                               output_final_state: bool = True, o=None, S_T=None,
                               scale=None, cu_seqlens=None, use_qk_l2norm_in_kernel=False,
                               fused_recurrent=False, workspace=None, stream=None):
    """Chunkwise forward of the gated rule: as ``delta_rule_chunk_fwd`` plus
    g ``[B,T,H]`` float32, the log of each token's forget gate (<= 0)."""
    return _chunk_call(True, q, k, v, beta, g, S0, chunk, output_final_state, o, S_T, stream,
                       scale, cu_seqlens, use_qk_l2norm_in_kernel, recurrent=fused_recurrent,
                       workspace=workspace)


def kda_fwd(q, k, v, beta, gk, S0=None, *, output_final_state: bool = True, o=None, S_T=None,
            scale=None, cu_seqlens=None, use_qk_l2norm_in_kernel=False, fused_recurrent=False,
            workspace=None, stream=None):
    """Forward of Kimi Delta Attention over whole sequences: as
    ``delta_rule_chunk_fwd`` plus gk ``[B,T,H,Dk]`` float32, the log decay
    (<= 0) of each key channel at each token (column j of the state is
    multiplied by exp(gk_t[j]) before token t).  bf16 inputs with Dk = 128 and
    Dv a multiple of 64 run the chunked kernel (32-token chunks; exact up to
    rounding for any gk <= 0, down to -inf); everything else, or
    ``fused_recurrent=True``, runs the token-serial schedule.  Long sequences that do
    not fill the GPU run the chunked kernel segment-parallel (``workspace``
    as in ``delta_rule_chunk_fwd``)."""
    return _chunk_call(False, q, k, v, beta, None, S0, 64, output_final_state, o, S_T, stream,
                       scale, cu_seqlens, use_qk_l2norm_in_kernel, gk=gk,
                       recurrent=fused_recurrent, workspace=workspace)


def _step_call(gated, q, k, v, beta, g, S, o, stream, scale=None, l2norm=False, gk=None):
    torch = _torch()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("the decode step needs GPU tensors")
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    _dtype_code(q)
    _need(q, "q", (B, H, Dk), dt, dev)
    _need(k, "k", (B, H, Dk), dt, dev)
    _need(v, "v", (B, H, Dv), dt, dev)
    _need(beta, "beta", (B, H), dt, dev)
    if gated:
        _need(g, "g", (B, H), torch.float32, dev)
    if gk is not None:
        _need(gk, "gk", (B, H, Dk), torch.float32, dev)
    _need(S, "S", (B, H, Dv, Dk), torch.float32, dev)
    if o is None:
        o = torch.empty((B, H, Dv), dtype=dt, device=dev)
    else:
        _need(o, "o", (B, H, Dv), dt, dev)
    lib = load_library()
    common = (_ptr(q), _ptr(k), _ptr(v), _ptr(beta))
    if scale is None and not l2norm and gk is None:
        if gated:
            st = lib.gated_delta_rule_recurrent_step(*common, _ptr(g), _ptr(S), _ptr(o), B, H,
                                                     Dk, Dv, _dtype_code(q), _stream(dev, stream))
        else:
            st = lib.delta_rule_recurrent_step(*common, _ptr(S), _ptr(o), B, H, Dk, Dv,
                                               _dtype_code(q), _stream(dev, stream))
    else:
        opts = dr_step_opts(g=g.data_ptr() if gated else None,
                            scale=1.0 if scale is None else float(scale),
                            flags=DR_QK_L2NORM if l2norm else 0,
                            gk=None if gk is None else gk.data_ptr())
        st = lib.delta_rule_recurrent_step_ex(*common, _ptr(S), _ptr(o), B, H, Dk, Dv,
                                              ctypes.byref(opts), _dtype_code(q),
                                              _stream(dev, stream))
    _check(st)
    return o


def delta_rule_recurrent_step(q, k, v, beta, S, *, o=None, scale=None,
                              use_qk_l2norm_in_kernel=False, stream=None):
    """One decode token: q, k ``[B,H,Dk]``; v ``[B,H,Dv]``; beta ``[B,H]``;
    S ``[B,H,Dv,Dk]`` float32, updated in place.  Returns o ``[B,H,Dv]``.
    ``scale`` and ``use_qk_l2norm_in_kernel`` as in the chunked forward."""
    return _step_call(False, q, k, v, beta, None, S, o, stream, scale, use_qk_l2norm_in_kernel)


def gated_delta_rule_recurrent_step(q, k, v, beta, g, S, *, o=None, scale=None,
                                    use_qk_l2norm_in_kernel=False, stream=None):
    """One decode token of the gated rule: as ``delta_rule_recurrent_step``
    plus g ``[B,H]`` float32, the log forget gate of this token."""
    return _step_call(True, q, k, v, beta, g, S, o, stream, scale, use_qk_l2norm_in_kernel)


def delta_rule_chunk_bwd(q, k, v, beta, do, S0=None, dS_T=None, *, workspace=None,
                         need_dS0=True, checkpoints_ready=False, stream=None):
    """Gradients of ``delta_rule_chunk_fwd`` (plain rule) for upstream
    gradients ``do`` ``[B,T,H,Dv]`` (dtype of q) and ``dS_T`` ``[B,H,Dv,Dk]``
    float32 or None.  Returns a dict with dq, dk, dv, dbeta (dtype of q) and
    dS0 (float32, or None when ``need_dS0`` is False).  ``workspace`` (a
    uint8 GPU tensor of at least ``delta_rule_chunk_bwd_workspace_bytes``
    bytes) holds the forward checkpoints; it is allocated when not given.
    ``checkpoints_ready``: the workspace already holds them, written by
    ``delta_rule_chunk_fwd_checkpointed`` for these same inputs, so the
    checkpointing forward pass is skipped."""
    return _bwd_call(q, k, v, beta, None, do, S0, dS_T, workspace, need_dS0, stream,
                     checkpoints_ready)


def gated_delta_rule_chunk_bwd(q, k, v, beta, g, do, S0=None, dS_T=None, *, workspace=None,
                               need_dS0=True, checkpoints_ready=False, stream=None):
    """Gradients of ``gated_delta_rule_chunk_fwd``: as ``delta_rule_chunk_bwd``
    with g ``[B,T,H]`` float32 (the log forget gate) among the inputs; the
    dict also holds dg (float32 ``[B,T,H]``)."""
    if g is None:
        raise ValueError("the gated backward needs g")
    return _bwd_call(q, k, v, beta, g, do, S0, dS_T, workspace, need_dS0, stream,
                     checkpoints_ready)


def delta_rule_chunk_fwd_checkpointed(q, k, v, beta, S0=None, *, g=None,
                                      output_final_state=True, o=None, S_T=None,
                                      workspace=None, stream=None):
    """The forward of the plain rule (or, with ``g``, the gated rule) that
    also writes every chunk's incoming state into the backward's
    ``workspace`` (allocated when None), at the backward's chunk length (32
    tokens for bfloat16, 16 for float32).  Returns ``(o, S_T, workspace)``;
    pass that workspace with ``checkpoints_ready=True`` to the backward of the
    same inputs, which then skips its checkpointing forward pass."""
    torch = _torch()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("the chunked forward needs GPU tensors")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    code = _dtype_code(q)
    _need(q, "q", (B, T, H, Dk), dt, dev)
    _need(k, "k", (B, T, H, Dk), dt, dev)
    _need(v, "v", (B, T, H, Dv), dt, dev)
    _need(beta, "beta", (B, T, H), dt, dev)
    if S0 is not None:
        _need(S0, "S0", (B, H, Dv, Dk), torch.float32, dev)
    if g is not None:
        _need(g, "g", (B, T, H), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=dt, device=dev)
    else:
        _need(o, "o", (B, T, H, Dv), dt, dev)
    if output_final_state and S_T is None:
        S_T = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev)
    elif S_T is not None:
        _need(S_T, "S_T", (B, H, Dv, Dk), torch.float32, dev)
    lib = load_library()
    nbytes = int(lib.delta_rule_chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, code))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace must be a GPU tensor of at least {nbytes} bytes")
    nws = workspace.numel() * workspace.element_size()
    st = lib.delta_rule_chunk_fwd_checkpointed(
        _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S0), _ptr(o), _ptr(S_T),
        _ptr(workspace), nws, B, T, H, Dk, Dv, code, _stream(dev, stream))
    _check(st)
    return o, S_T, workspace


def _bwd_call(q, k, v, beta, g, do, S0, dS_T, workspace, need_dS0, stream,
              checkpoints_ready=False):
    torch = _torch()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("the backward needs GPU tensors")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    code = _dtype_code(q)
    _need(q, "q", (B, T, H, Dk), dt, dev)
    _need(k, "k", (B, T, H, Dk), dt, dev)
    _need(v, "v", (B, T, H, Dv), dt, dev)
    _need(beta, "beta", (B, T, H), dt, dev)
    _need(do, "do", (B, T, H, Dv), dt, dev)
    if S0 is not None:
        _need(S0, "S0", (B, H, Dv, Dk), torch.float32, dev)
    if dS_T is not None:
        _need(dS_T, "dS_T", (B, H, Dv, Dk), torch.float32, dev)
    if g is not None:
        _need(g, "g", (B, T, H), torch.float32, dev)
    lib = load_library()
    nbytes = int(lib.delta_rule_chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, code))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace must be a GPU tensor of at least {nbytes} bytes")
    out = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
           "dbeta": torch.empty_like(beta),
           "dS0": torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev)
           if need_dS0 else None}
    nws = workspace.numel() * workspace.element_size()
    if checkpoints_ready:
        if g is not None:
            out["dg"] = torch.empty_like(g)
        st = lib.delta_rule_chunk_bwd_ex(
            _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S0), _ptr(do), _ptr(dS_T),
            _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dbeta"]),
            _ptr(out.get("dg")), _ptr(out["dS0"]), _ptr(workspace), nws, B, T, H, Dk, Dv,
            DR_BWD_CHECKPOINTS_READY, code, _stream(dev, stream))
    elif g is None:
        st = lib.delta_rule_chunk_bwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(S0), _ptr(do), _ptr(dS_T),
            _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dbeta"]),
            _ptr(out["dS0"]), _ptr(workspace), nws, B, T, H, Dk, Dv, code, _stream(dev, stream))
    else:
        out["dg"] = torch.empty_like(g)
        st = lib.gated_delta_rule_chunk_bwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S0), _ptr(do), _ptr(dS_T),
            _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dbeta"]),
            _ptr(out["dg"]), _ptr(out["dS0"]), _ptr(workspace), nws, B, T, H, Dk, Dv, code,
            _stream(dev, stream))
    _check(st)
    return out


def kda_bwd_workspace_bytes(B, T, H, Dk, Dv, num_seqs=None):
    """Bytes of device workspace ``kda_bwd`` needs (``num_seqs``: the number
    of packed sequences, or None for B sequences of T tokens)."""
    n = B if num_seqs is None else num_seqs
    return int(load_library().kda_bwd_workspace_bytes(B, T, H, Dk, Dv, n))


def kda_bwd(q, k, v, beta, gk, do, S0=None, dS_T=None, *, scale=None, cu_seqlens=None,
            workspace=None, need_dS0=True, stream=None):
    """Gradients of ``kda_fwd`` (without the in-kernel L2 norm) for upstream
    gradients ``do`` ``[B,T,H,Dv]`` (dtype of q) and ``dS_T`` float32 or
    None, for any log decay gk, erased channels included (``kda_bwd``).
    ``scale`` and ``cu_seqlens`` as in the forward.  Returns a dict with dq,
    dk, dv, dbeta (dtype of q), dgk (float32 ``[B,T,H,Dk]``) and dS0 (float32,
    or None when ``need_dS0`` is False).  ``workspace``: a uint8 GPU tensor of
    at least ``kda_bwd_workspace_bytes`` bytes, allocated when None.  With
    ``cu_seqlens``, tokens outside every sequence get zero gradients."""
    torch = _torch()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("the backward needs GPU tensors")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    code = _dtype_code(q)
    _need(q, "q", (B, T, H, Dk), dt, dev)
    _need(k, "k", (B, T, H, Dk), dt, dev)
    _need(v, "v", (B, T, H, Dv), dt, dev)
    _need(beta, "beta", (B, T, H), dt, dev)
    _need(gk, "gk", (B, T, H, Dk), torch.float32, dev)
    _need(do, "do", (B, T, H, Dv), dt, dev)
    nseq = B
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError("packed sequences (cu_seqlens) need a batch of 1")
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
            raise ValueError("cu_seqlens must be a 1-D tensor of num_seqs + 1 offsets")
        if cu_seqlens.dtype != torch.int32:
            cu_seqlens = cu_seqlens.to(torch.int32)
        nseq = cu_seqlens.numel() - 1
        _need(cu_seqlens, "cu_seqlens", (nseq + 1,), torch.int32, dev)
    if S0 is not None:
        _need(S0, "S0", (nseq, H, Dv, Dk), torch.float32, dev)
    if dS_T is not None:
        _need(dS_T, "dS_T", (nseq, H, Dv, Dk), torch.float32, dev)
    lib = load_library()
    nbytes = int(lib.kda_bwd_workspace_bytes(B, T, H, Dk, Dv, nseq))
    if nbytes < 0:
        raise NotImplementedError(f"kda_bwd does not support Dk={Dk}, Dv={Dv}")
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace must be a GPU tensor of at least {nbytes} bytes")
    alloc = torch.zeros if cu_seqlens is not None else torch.empty
    out = {"dq": alloc(q.shape, dtype=dt, device=dev), "dk": alloc(k.shape, dtype=dt, device=dev),
           "dv": alloc(v.shape, dtype=dt, device=dev),
           "dbeta": alloc(beta.shape, dtype=dt, device=dev),
           "dgk": alloc(gk.shape, dtype=torch.float32, device=dev),
           "dS0": torch.empty((nseq, H, Dv, Dk), dtype=torch.float32, device=dev)
           if need_dS0 else None}
    st = lib.kda_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(gk), _ptr(S0), _ptr(do),
                     _ptr(dS_T), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                     _ptr(out["dbeta"]), _ptr(out["dgk"]), _ptr(out["dS0"]),
                     None if cu_seqlens is None else ctypes.c_void_p(cu_seqlens.data_ptr()),
                     nseq if cu_seqlens is not None else 0,
                     1.0 if scale is None else float(scale), _ptr(workspace),
                     workspace.numel() * workspace.element_size(), B, T, H, Dk, Dv, code,
                     _stream(dev, stream))
    _check(st)
    return out


def kda_recurrent_step(q, k, v, beta, gk, S, *, o=None, scale=None,
                       use_qk_l2norm_in_kernel=False, stream=None):
    """One decode token of Kimi Delta Attention: as
    ``delta_rule_recurrent_step`` plus gk ``[B,H,Dk]`` float32, the log decay
    of each key channel (column j of S is scaled by exp(gk[j]) before the
    token)."""
    return _step_call(False, q, k, v, beta, None, S, o, stream, scale, use_qk_l2norm_in_kernel,
                      gk)
