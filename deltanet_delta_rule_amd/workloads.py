"""Seeded synthetic workloads for the delta-rule operator.

This module draws inputs only.  It holds none of the operator's arithmetic and
imports nothing else from this package, so both the HIP path and the fp64
oracle can be fed from it.  Every tensor is drawn in fp32 on the CPU from a
``torch.Generator`` seeded per workload, shaped and distributed as follows:

* draw order: q_raw, k_raw, v, beta_raw, S0 (all standard normal);
* q, k: L2-normalised along the head dimension (x / max(||x||, 1e-12)),
  after a SiLU for the small-model workload, or left raw (feature "raw") for
  the tests of the kernel's own normalisation option; by default the operator
  does not normalise (the DeltaNet layer feeds it SiLU + L2-normalised keys and
  queries: "Parallelizing Linear Transformers with the Delta Rule over Sequence
  Length", section 3 "DeltaNet transformer");
* v: standard normal;
* beta = sigmoid(beta_raw), doubled for the negative-eigenvalue workload, one
  scalar per (token, head) (fla ``fla/layers/delta_net.py``: ``b_proj`` then
  ``sigmoid``, times 2 when ``allow_neg_eigval``);
* S0: zero, or 0.02 * N(0,1) in fp32 where the workload carries a state in;
* gated workloads (gate_amax > 0) then draw, per head, A ~ U(0, gate_amax)
  and, per (token, head), a ~ N(0,1), and set the log forget gate
  g = -A softplus(a + 1) (the gated layer of the houmin.site page,
  "infra/delta-net", section "Gated DeltaNet": alpha = exp(-exp(A_log)
  softplus(W_alpha x + dt_bias)) with A = exp(A_log) drawn from U(0,16) and
  dt_bias = 1; a stands in for W_alpha x);
* KDA workloads (kda=True) draw a per (token, head, key channel) instead, so
  the log decay gk = -A softplus(a + 1) is a vector over the key channels
  (hada.io digest, section "Kimi Delta Attention : attenuation par canal":
  the scalar gate becomes a diagonal over the key dimension);
* q, k, v, beta are then rounded once to the workload dtype (round to nearest
  even); S0 and g stay fp32.

Named workloads (sizes are the whole job on one GPU):

``tiny_fp32``     B1 H2 T64 d16, chunk 16, fp32
``small_model``   B4 H8 T2048 d64, chunk 64, bf16, SiLU + L2 features
``layer_1p3b``    B8 H16 T2048 d128, chunk 64, bf16 (hidden 2048, 16 heads)
``long_prefill``  B1 H16 T32768 d128, chunk 64, bf16, S0 != 0, beta in (0,2)
``decode``        B128 H16 d128, 256 single-token steps, bf16, S0 != 0
``gated_layer_1p3b``  the layer_1p3b shape with the gated rule (A up to 16)
``gated_decode``  the decode workload with the gated rule
``kda_decode``    the decode workload with per-key-channel decay (A up to 1)
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import torch

BASE_SEED = 20240606


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int          # tokens per sequence (decode: number of steps)
    Dk: int
    Dv: int
    chunk: int      # chunk length (decode: unused)
    dtype: str      # "f32" or "bf16"
    feature: str    # "l2" or "silu_l2"
    beta_scale: float
    s0_std: float
    seed: int
    decode: bool = False
    gate_amax: float = 0.0  # > 0: gated rule, per-head A ~ U(0, gate_amax)
    kda: bool = False       # with gate_amax > 0: one log decay per key channel

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", B=1, H=2, T=64, Dk=16, Dv=16, chunk=16,
                          dtype="f32", feature="l2", beta_scale=1.0,
                          s0_std=0.0, seed=BASE_SEED + 0),
    "small_model": Workload("small_model", B=4, H=8, T=2048, Dk=64, Dv=64,
                            chunk=64, dtype="bf16", feature="silu_l2",
                            beta_scale=1.0, s0_std=0.0, seed=BASE_SEED + 1),
    "layer_1p3b": Workload("layer_1p3b", B=8, H=16, T=2048, Dk=128, Dv=128,
                           chunk=64, dtype="bf16", feature="l2",
                           beta_scale=1.0, s0_std=0.0, seed=BASE_SEED + 2),
    "long_prefill": Workload("long_prefill", B=1, H=16, T=32768, Dk=128,
                             Dv=128, chunk=64, dtype="bf16", feature="l2",
                             beta_scale=2.0, s0_std=0.02, seed=BASE_SEED + 3),
    "decode": Workload("decode", B=128, H=16, T=256, Dk=128, Dv=128, chunk=1,
                       dtype="bf16", feature="l2", beta_scale=1.0,
                       s0_std=0.02, seed=BASE_SEED + 4, decode=True),
    "gated_layer_1p3b": Workload("gated_layer_1p3b", B=8, H=16, T=2048, Dk=128,
                                 Dv=128, chunk=64, dtype="bf16", feature="l2",
                                 beta_scale=1.0, s0_std=0.0,
                                 seed=BASE_SEED + 5, gate_amax=16.0),
    "gated_decode": Workload("gated_decode", B=128, H=16, T=256, Dk=128,
                             Dv=128, chunk=1, dtype="bf16", feature="l2",
                             beta_scale=1.0, s0_std=0.02, seed=BASE_SEED + 6,
                             decode=True, gate_amax=16.0),
    "kda_decode": Workload("kda_decode", B=128, H=16, T=256, Dk=128,
                           Dv=128, chunk=1, dtype="bf16", feature="l2",
                           beta_scale=1.0, s0_std=0.02, seed=BASE_SEED + 7,
                           decode=True, gate_amax=1.0, kda=True),
}


def _features(x: torch.Tensor, feature: str) -> torch.Tensor:
    if feature == "raw":
        return x  # left for the kernel's own normalisation option
    if feature == "silu_l2":
        x = x * torch.sigmoid(x)
    elif feature != "l2":
        raise ValueError(f"unknown feature map {feature!r}")
    return torch.nn.functional.normalize(x, p=2.0, dim=-1, eps=1e-12)


def generate(w: Workload) -> dict:
    """Draw one workload.  Returns CPU tensors:

    chunk workloads: q, k [B,T,H,Dk]; v [B,T,H,Dv]; beta [B,T,H] in the
    workload dtype; S0 [B,H,Dv,Dk] fp32 or None; g [B,T,H] fp32 (gated
    workloads) or None; gk [B,T,H,Dk] fp32 (KDA workloads) or None.
    decode workloads: the same with the leading two axes read as
    [steps, B] (q, k [steps,B,H,Dk] ...), i.e. step-major.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    lead = (w.T, w.B) if w.decode else (w.B, w.T)
    q_raw = torch.randn(*lead, w.H, w.Dk, generator=g, dtype=torch.float32)
    k_raw = torch.randn(*lead, w.H, w.Dk, generator=g, dtype=torch.float32)
    v = torch.randn(*lead, w.H, w.Dv, generator=g, dtype=torch.float32)
    beta_raw = torch.randn(*lead, w.H, generator=g, dtype=torch.float32)
    if w.s0_std > 0:
        S0 = w.s0_std * torch.randn(w.B, w.H, w.Dv, w.Dk, generator=g,
                                    dtype=torch.float32)
    else:
        S0 = None
    gl = gk = None
    if w.gate_amax > 0:
        A = w.gate_amax * torch.rand(w.H, generator=g, dtype=torch.float32)
        if w.kda:
            a = torch.randn(*lead, w.H, w.Dk, generator=g, dtype=torch.float32)
            gk = (-A[:, None] * torch.nn.functional.softplus(a + 1.0)).contiguous()
        else:
            a = torch.randn(*lead, w.H, generator=g, dtype=torch.float32)
            gl = (-A * torch.nn.functional.softplus(a + 1.0)).contiguous()
    q = _features(q_raw, w.feature)
    k = _features(k_raw, w.feature)
    beta = w.beta_scale * torch.sigmoid(beta_raw)
    dt = w.torch_dtype
    out = {
        "q": q.to(dt).contiguous(),
        "k": k.to(dt).contiguous(),
        "v": v.to(dt).contiguous(),
        "beta": beta.to(dt).contiguous(),
        "S0": S0,
        "g": gl,
    }
    if gk is not None:
        out["gk"] = gk
    return out


def get(name: str, **overrides) -> Workload:
    """A named workload, optionally with fields overridden (e.g. a shorter T
    for a test that the oracle must finish in seconds)."""
    w = WORKLOADS[name]
    return w.with_(**overrides) if overrides else w


__all__ = ["Workload", "WORKLOADS", "generate", "get", "BASE_SEED"]
