#!/usr/bin/env python3
"""Throughput of the delta-rule forward on one MI355X.

One step = one ``delta_rule_chunk_fwd`` over the 1.3B-scale layer shape
(B=8, H=16, T=2048, d_k=d_v=128, chunk 64, bf16 inputs, fp32 state, final
state returned) with inputs already resident in HBM.  W untimed warm-up
steps, then K timed steps between two device synchronisations.  The GPU
raises its clock over the first tens of milliseconds of sustained work (the
benchmark step takes ~84 us per launch in the first 8 ms and settles at
~71 us after ~20 ms), so the default W = 1500 (~0.1 s) and every other line
below runs its step back to back for 0.1 s before its timed region: each
figure is the steady-state rate, not the ramp's.  Prints ONE JSON line on
stdout:

  value        tokens/s = B*T*K / wall time of the K steps
  roofline     the fused chunk kernel against HBM bandwidth (its roofline
               bound: arithmetic intensity 170 flop/B is below the MI355X
               ridge of ~315 flop/B), from the mean launch time: one pair of
               HIP events on the launch stream around the K back-to-back
               steps, elapsed / K; mfma_frac gives the same time against the
               dense bf16 MFMA peak
  cpu_baseline the fp64 CPU oracle on the host cores (reported, not a target),
               with a single-thread figure on a sample of heads beside it
  small_model  the small-model config (B4 H8 T2048 d64, SiLU + L2 features),
               mean launch time and its HBM / MFMA fractions
  parity       the timed run's outputs against that oracle run
  decode       256 back-to-back single-token steps of the decode workload
               (B=128, H=16, d=128), HBM bytes per step and tokens/s
  gated        the gated rule (per-token log forget gate) on the layer shape
               (chunked forward) and on the decode workload
  qk_l2norm    the layer shape with raw q, k normalised inside the kernel
  backward     delta_rule_chunk_bwd on the layer shape (checkpointing forward
               and reverse pass), time per call and ratio to the forward launch;
               with "gated" inside it, gated_delta_rule_chunk_bwd likewise, and
               "one_sequence", one sequence of the layer shape (B = 1, the
               two-pass reverse schedule for few heads), "training_step", and
               "kda", kda_bwd on the layer shape with per-channel decay
  kda          per-key-channel decay: decode steps and the chunked forward
  long_prefill the long-prefill config (B1 H16 T32768) through the
               segment-parallel schedule, with the plain schedule beside it

Options: --gpus N (only 1: the library runs on one GPU), --steps K,
--warmup W, --no-cpu-baseline, --no-decode, --no-small-model, --no-gated, --no-backward,
--no-long-prefill (its segment passes launch the benchmark's kernel on
other shapes; counter and trace runs of the benchmark line skip it),
--copy-calib BYTES (also time a
plain device copy of that size, for counter calibration runs).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("delta-rule fwd tokens/sec at H=16,d=128,T=2048; "
          "% bf16 MFMA / HBM roofline")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, published (256 CU x 2.4 GHz x 4096)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "chunk_fwd_layer_1p3b_traffic.txt")
KERNEL_SOURCES = ["deltanet_delta_rule_amd/csrc/chunk_fwd.hpp",
                  "deltanet_delta_rule_amd/csrc/chunk_fwd.hip",
                  "deltanet_delta_rule_amd/csrc/chunk_fwd_d128_c64.hip",
                  "deltanet_delta_rule_amd/csrc/dr_common.hpp",
                  "deltanet_delta_rule_amd/build.py"]  # compile flags
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "recurrent_step_decode_traffic.txt")
DECODE_SOURCES = ["deltanet_delta_rule_amd/csrc/recurrent_step.hip",
                  "deltanet_delta_rule_amd/csrc/dr_common.hpp",
                  "deltanet_delta_rule_amd/build.py"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def timed_steps(torch, step, reps):
    """Seconds per step of `reps` back-to-back steps, from one pair of HIP
    events on the current stream around all of them (an event pair around
    every step would put its own gap between the launches)."""
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        step()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps / 1e3


SETTLE_S = 0.1  # seconds of back-to-back work before a timed region


def settle(torch, step, seconds=SETTLE_S):
    """Run `step` back to back for about `seconds` so that the timed region
    that follows starts at the GPU's steady clock; returns the number of runs.
    Batches of 8 runs end in a synchronisation, so that the host never queues
    far ahead of the device."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            step()
        n += 8
        torch.cuda.synchronize()
    return n


def chunk_work(w):
    """Algorithmic MFMA flops and HBM bytes of one chunk_fwd call.

    flops per token-head: 2C(3Dk + 2Dv) + 6 Dk Dv (the products K K^T, Q K^T,
    T K; T V, (QK^T.M) E; W S^T, Q S^T, E^T K of the chunk form with full
    C x C tiles).  bytes: q, k, v, beta read and o written once in the input
    dtype, S0 read and S_T written once in fp32."""
    th = w.B * w.T * w.H
    e = 2 if w.dtype == "bf16" else 4
    flops = th * (2 * w.chunk * (3 * w.Dk + 2 * w.Dv) + 6 * w.Dk * w.Dv)
    nbytes = th * e * (2 * w.Dk + w.Dv + 1) + th * e * w.Dv
    if w.gate_amax > 0:  # fp32 log gates: one per token-head, or per key channel
        nbytes += th * 4 * (w.Dk if w.kda else 1)
    nbytes += 4 * w.B * w.H * w.Dv * w.Dk * ((1 if w.s0_std > 0 else 0) + 1)
    return flops, nbytes


def decode_bytes(w):
    """HBM bytes of one decode step: S read and written (fp32), q, k, v, beta
    read and o written in the input dtype, plus the fp32 log gate when gated
    (one per head, or one per key channel with per-channel decay)."""
    e = 2 if w.dtype == "bf16" else 4
    bh = w.B * w.H
    gate = 0 if w.gate_amax <= 0 else (4 * w.Dk if w.kda else 4)
    return bh * (8 * w.Dv * w.Dk + e * (2 * w.Dk + w.Dv + 1) + e * w.Dv + gate)


def source_digest(sources=KERNEL_SOURCES):
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(path=TRAFFIC_FILE, sources=KERNEL_SOURCES):
    """HBM bytes per launch from a committed counter summary, or None when
    the kernel sources changed since the counters were taken."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
    if kv.get("kernel_source_sha256") != source_digest(sources):
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def repeat_timed(fn, min_s=10.0, max_runs=200):
    """Run fn() back to back until min_s seconds of it have been timed (at
    least once); returns (mean seconds per run, runs, total seconds)."""
    total, runs = 0.0, 0
    while runs == 0 or (total < min_s and runs < max_runs):
        t0 = time.perf_counter()
        fn()
        total += time.perf_counter() - t0
        runs += 1
    return total / runs, runs, total


def run_cpu_single_thread(x, w, heads=16):
    """The fp64 oracle on one host thread over a bounded sample of the
    workload: the first `heads` (batch, head) pairs at full length."""
    import numpy as np

    from oracle import delta_rule_ref
    sel = [(b, h) for b in range(w.B) for h in range(w.H)][:heads]
    pick = lambda t: np.stack([t[b, :, h].double().numpy() for b, h in sel], axis=1)[None]
    q, k, v, beta = (pick(x[n]) for n in ("q", "k", "v", "beta"))
    S0 = None if x["S0"] is None else np.stack([x["S0"][b, h].double().numpy()
                                                for b, h in sel])[None]
    dt, runs, total = repeat_timed(lambda: delta_rule_ref(q, k, v, beta, S0, nthreads=1))
    # tokens/s of the whole workload at this rate: every (batch, head) pair
    # costs the same, and a token is all H heads of one batch row
    return {
        "value": len(sel) * w.T / w.H / dt,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{len(sel)} of the {w.B * w.H} heads of {w.name}, full T = {w.T}, "
                  f"{runs} runs in {total:.1f} s, scaled to tokens of all {w.H} heads",
    }


def run_cpu_baseline(x, w, o_gpu, st_gpu):
    """The fp64 oracle on the whole workload (all heads, full T), timed
    around the oracle call only with inputs already widened to fp64, repeated
    for about ten seconds (the first call's outputs give the parity)."""
    import numpy as np

    from oracle import delta_rule_ref
    q, k, v, beta = (x[n].double().numpy() for n in ("q", "k", "v", "beta"))
    S0 = None if x["S0"] is None else x["S0"].double().numpy()
    nt = cpu_threads()
    o_ref, s_ref = delta_rule_ref(q, k, v, beta, S0, nthreads=nt)
    dt, runs, total = repeat_timed(lambda: delta_rule_ref(q, k, v, beta, S0, nthreads=nt))
    og = o_gpu.double().cpu().numpy()
    sg = st_gpu.double().cpu().numpy()
    par = {
        "o_rel_err": float(np.max(np.abs(og - o_ref)) / np.max(np.abs(o_ref))),
        "S_T_rel_err": float(np.max(np.abs(sg - s_ref)) / np.max(np.abs(s_ref))),
        "tol": 2e-2 if w.dtype == "bf16" else 1e-4,
        "reference": "fp64 CPU oracle, whole workload",
    }
    base = {
        "value": w.B * w.T / dt,
        "unit": "tokens/s",
        "cores": nt,
        "kind": "oracle",
        "sample": (f"whole {w.name} workload ({w.B * w.H} heads x {w.T} tokens), "
                   f"{runs} runs in {total:.1f} s"),
    }
    return base, par


def bench_decode(torch, dr, W, reps=3, name="decode", **over):
    w = W.get(name, **over)
    x = W.generate(w)
    dev = torch.device("cuda:0")
    d = {n: (None if t is None else t.to(dev)) for n, t in x.items()}
    S = d["S0"].clone()
    outs = [torch.empty((w.B, w.H, w.Dv), dtype=w.torch_dtype, device=dev)
            for _ in range(w.T)]

    def run():
        for t in range(w.T):
            if d.get("gk") is not None:
                dr.kda_recurrent_step(d["q"][t], d["k"][t], d["v"][t], d["beta"][t], d["gk"][t],
                                      S, o=outs[t])
            elif d["g"] is None:
                dr.delta_rule_recurrent_step(d["q"][t], d["k"][t], d["v"][t], d["beta"][t], S,
                                             o=outs[t])
            else:
                dr.gated_delta_rule_recurrent_step(d["q"][t], d["k"][t], d["v"][t],
                                                   d["beta"][t], d["g"][t], S, o=outs[t])

    settle(torch, run)  # the state resets before every timed run
    times = []
    for _ in range(reps):
        S.copy_(d["S0"])  # reset outside the timed region
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        run()
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e) / 1e3)
    t = sorted(times)[len(times) // 2]
    per_step = t / w.T
    gbs = decode_bytes(w) / per_step / 1e9
    res = {
        "workload": (f"{w.name} B{w.B} H{w.H} d{w.Dk}, {w.T} steps, bf16 in, fp32 state"
                     + ("" if w.gate_amax <= 0 else
                        ", per-channel log decay fp32" if w.kda else ", log gates fp32")),
        "tokens_per_s": w.B * w.T / t,
        "us_per_step": per_step * 1e6,
        "hbm_gbs_algorithmic": gbs,
        "hbm_frac": gbs / HBM_PEAK_GBS,
        "algorithmic_bytes_per_step": decode_bytes(w),
    }
    traffic = measured_traffic(DECODE_TRAFFIC_FILE, DECODE_SOURCES)
    if name == "decode" and not over and traffic is not None:
        res["traffic"] = traffic
    return res


def bench_gated_chunk(torch, dr, W, reps=20, name="gated_layer_1p3b", l2=False):
    """A chunked-forward variant on the layer shape (mean launch time with HIP
    events on the launch stream): the gated rule, or with l2 the plain rule
    on raw q, k normalised inside the kernel."""
    w = W.get(name, feature="raw") if l2 else W.get(name)
    x = W.generate(w)
    dev = torch.device("cuda:0")
    d = {n: (None if t is None else t.to(dev)) for n, t in x.items()}
    o = torch.empty((w.B, w.T, w.H, w.Dv), dtype=w.torch_dtype, device=dev)
    st = torch.empty((w.B, w.H, w.Dv, w.Dk), dtype=torch.float32, device=dev)
    # the segment-parallel schedule's workspace (where the shape has a plan:
    # the small model), allocated once, before timing
    need = dr.chunk_fwd_workspace_bytes(w.B, w.T, w.H, w.Dk, w.Dv, w.chunk, w.torch_dtype)
    ws = torch.empty(need, dtype=torch.uint8, device=dev) if need > 0 else False

    def step():
        if d["g"] is None:
            dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["S0"], chunk=w.chunk,
                                    o=o, S_T=st, use_qk_l2norm_in_kernel=l2, workspace=ws)
        else:
            dr.gated_delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["S0"],
                                          chunk=w.chunk, o=o, S_T=st,
                                          use_qk_l2norm_in_kernel=l2, workspace=ws)

    settle(torch, step)
    launch_s = timed_steps(torch, step, reps)
    flops, nbytes = chunk_work(w)
    what = ("raw q, k normalised in the kernel, fp32 state" if l2 else
            "fp32 log gates and state" if d["g"] is not None else
            f"{w.feature} features, fp32 state")
    return {
        "workload": f"{w.name} B{w.B} H{w.H} T{w.T} d{w.Dk} chunk {w.chunk}, {w.dtype} in, {what}",
        "tokens_per_s": w.B * w.T / launch_s,
        "mean_launch_us": round(launch_s * 1e6, 2),
        "hbm_frac": round(nbytes / launch_s / 1e9 / HBM_PEAK_GBS, 4),
        "mfma_frac": round(flops / launch_s / 1e12 / BF16_PEAK_TFLOPS, 4),
        "algorithmic_bytes_per_launch": nbytes,
        "algorithmic_flops_per_launch": flops,
    }


def bench_kda_sequence(torch, dr, W, reps=10):
    """kda_fwd (chunked kernel) on the layer shape with per-channel decay:
    mean call time with HIP events on the launch stream."""
    w = W.get("layer_1p3b", gate_amax=16.0, kda=True, chunk=32)
    x = W.generate(w)
    dev = torch.device("cuda:0")
    d = {n: (None if t is None else t.to(dev)) for n, t in x.items()}
    o = torch.empty((w.B, w.T, w.H, w.Dv), dtype=w.torch_dtype, device=dev)
    st = torch.empty((w.B, w.H, w.Dv, w.Dk), dtype=torch.float32, device=dev)

    def step():
        dr.kda_fwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], None, o=o, S_T=st)

    settle(torch, step)
    launch_s = timed_steps(torch, step, reps)
    flops, nbytes = chunk_work(w)
    return {
        "workload": (f"layer_1p3b B{w.B} H{w.H} T{w.T} d{w.Dk} chunk {w.chunk}, bf16 in, "
                     "per-channel log decay fp32 (A up to 16), fp32 state"),
        "tokens_per_s": w.B * w.T / launch_s,
        "mean_launch_us": round(launch_s * 1e6, 2),
        "hbm_frac": round(nbytes / launch_s / 1e9 / HBM_PEAK_GBS, 4),
        "mfma_frac": round(flops / launch_s / 1e12 / BF16_PEAK_TFLOPS, 4),
    }


def bench_long_prefill(torch, dr, W, reps=20):
    """delta_rule_chunk_fwd on the long-prefill config (B1 H16 T32768, beta in
    (0,2), S0 != 0): the segment-parallel schedule the binding picks for it,
    and the plain schedule (workspace=False) for comparison; mean call time
    with HIP events on the launch stream (the workspace is allocated before
    timing)."""
    w = W.get("long_prefill")
    x = W.generate(w)
    dev = torch.device("cuda:0")
    d = {n: (None if t is None else t.to(dev)) for n, t in x.items()}
    o = torch.empty((w.B, w.T, w.H, w.Dv), dtype=w.torch_dtype, device=dev)
    st = torch.empty((w.B, w.H, w.Dv, w.Dk), dtype=torch.float32, device=dev)
    need = dr.chunk_fwd_workspace_bytes(w.B, w.T, w.H, w.Dk, w.Dv, w.chunk)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def timed(workspace):
        def step():
            dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["S0"], chunk=w.chunk,
                                    o=o, S_T=st, workspace=workspace)
        settle(torch, step)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        for _ in range(reps):
            step()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps / 1e3

    t_seg, t_plain = timed(ws if need > 0 else False), timed(False)
    _, nbytes = chunk_work(w)
    return {
        "workload": (f"long_prefill B{w.B} H{w.H} T{w.T} d{w.Dk} chunk {w.chunk}, bf16 in, "
                     "beta in (0,2), S0 != 0, fp32 state"),
        "tokens_per_s": w.B * w.T / t_seg,
        "mean_call_us": round(t_seg * 1e6, 2),
        "workspace_bytes": need,
        "plain_schedule_us": round(t_plain * 1e6, 2),
        "hbm_frac_algorithmic": round(nbytes / t_seg / 1e9 / HBM_PEAK_GBS, 4),
    }


def bench_backward(torch, dr, W, reps=10, name="layer_1p3b", B=None):
    """delta_rule_chunk_bwd (gated_delta_rule_chunk_bwd for a gated workload)
    on the layer shape (or B of its sequences): the checkpointing forward pass
    plus the reverse pass, with upstream gradients for o and S_T (mean time
    per call with HIP events on the launch stream)."""
    w = W.get(name) if B is None else W.get(name, B=B)
    x = W.generate(w)
    dev = torch.device("cuda:0")
    d = {n: (None if t is None else t.to(dev)) for n, t in x.items()}
    gen = torch.Generator(device="cpu").manual_seed(11)
    do = torch.randn(w.B, w.T, w.H, w.Dv, generator=gen).to(w.torch_dtype).to(dev)
    dst = torch.randn(w.B, w.H, w.Dv, w.Dk, generator=gen).to(dev)
    lib = dr.load_library()
    code = dr.DR_BF16 if w.dtype == "bf16" else dr.DR_F32
    ws = torch.empty(int(lib.delta_rule_chunk_bwd_workspace_bytes(w.B, w.T, w.H, w.Dk, w.Dv,
                                                                  code)),
                     dtype=torch.uint8, device=dev)

    def step():
        if d.get("g") is None:
            dr.delta_rule_chunk_bwd(d["q"], d["k"], d["v"], d["beta"], do, d["S0"], dst,
                                    workspace=ws)
        else:
            dr.gated_delta_rule_chunk_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], do,
                                          d["S0"], dst, workspace=ws)

    settle(torch, step)
    t = timed_steps(torch, step, reps)
    return {
        "workload": (f"{w.name} B{w.B} H{w.H} T{w.T} d{w.Dk}, bf16 in, fp32 state; "
                     "checkpointing forward + reverse pass (output allocation inside)"
                     + ("; reverse pass as the recursion pass (in segments whose maps are "
                        "chained, for at most 32 (b, h)) then the products pass over runs of "
                        "chunks (few heads)" if w.B * w.H <= 64 else
                        "; reverse walk split over two streams (recursion over the last "
                        "21/32 of the chunks, then the first 11/32, beside the single pass "
                        "over the last 21/32)" if w.B * w.H <= 128 else "")),
        "tokens_per_s": w.B * w.T / t,
        "mean_call_us": round(t * 1e6, 2),
        "vs_forward_launch": None,
        "workspace_bytes": int(ws.numel()),
    }


def bench_kda_backward(torch, dr, W, reps=5):
    """kda_bwd on the layer shape with per-channel decay drawn with A up to 16
    (the kda_fwd line's inputs), upstream gradients for o and S_T: mean time
    per call with HIP events on the launch stream (outputs allocated inside)."""
    w = W.get("layer_1p3b", gate_amax=16.0, kda=True, chunk=32)
    x = W.generate(w)
    dev = torch.device("cuda:0")
    d = {n: (None if t is None else t.to(dev)) for n, t in x.items()}
    gen = torch.Generator(device="cpu").manual_seed(11)
    do = torch.randn(w.B, w.T, w.H, w.Dv, generator=gen).to(w.torch_dtype).to(dev)
    dst = torch.randn(w.B, w.H, w.Dv, w.Dk, generator=gen).to(dev)
    ws = torch.empty(dr.kda_bwd_workspace_bytes(w.B, w.T, w.H, w.Dk, w.Dv), dtype=torch.uint8,
                     device=dev)

    def step():
        dr.kda_bwd(d["q"], d["k"], d["v"], d["beta"], d["gk"], do, d["S0"], dst, workspace=ws)

    settle(torch, step)
    t = timed_steps(torch, step, reps)
    return {
        "workload": (f"layer_1p3b B{w.B} H{w.H} T{w.T} d{w.Dk}, bf16 in, per-channel log decay "
                     "fp32 (A up to 16), fp32 state; token-serial: forward with a checkpoint "
                     "every 16 tokens, then blocks in reverse with their states recomputed, "
                     "and a reduce over the row tiles"),
        "tokens_per_s": w.B * w.T / t,
        "mean_call_us": round(t * 1e6, 2),
        "vs_kda_forward": None,
        "workspace_bytes": int(ws.numel()),
    }


def bench_training_step(torch, dr, W, reps=10, name="layer_1p3b"):
    """The chunked work of a training step on the layer shape: the forward
    (chunk 64) then the backward that forms its own checkpoints, against the
    forward that keeps the checkpoints in the backward's workspace (chunk 32,
    delta_rule_chunk_fwd_checkpointed) then the backward that reuses them
    (DR_BWD_CHECKPOINTS_READY); mean time per step and per call with HIP
    events on the launch stream, upstream gradients for o and S_T."""
    w = W.get(name)
    x = W.generate(w)
    dev = torch.device("cuda:0")
    d = {n: (None if t is None else t.to(dev)) for n, t in x.items()}
    gen = torch.Generator(device="cpu").manual_seed(11)
    do = torch.randn(w.B, w.T, w.H, w.Dv, generator=gen).to(w.torch_dtype).to(dev)
    dst = torch.randn(w.B, w.H, w.Dv, w.Dk, generator=gen).to(dev)
    lib = dr.load_library()
    ws = torch.empty(int(lib.delta_rule_chunk_bwd_workspace_bytes(w.B, w.T, w.H, w.Dk, w.Dv,
                                                                  dr.DR_BF16)),
                     dtype=torch.uint8, device=dev)
    o = torch.empty((w.B, w.T, w.H, w.Dv), dtype=w.torch_dtype, device=dev)
    st = torch.empty((w.B, w.H, w.Dv, w.Dk), dtype=torch.float32, device=dev)
    args = (d["q"], d["k"], d["v"], d["beta"])

    def fwd():
        dr.delta_rule_chunk_fwd(*args, d["S0"], chunk=w.chunk, o=o, S_T=st, workspace=False)

    def bwd():
        dr.delta_rule_chunk_bwd(*args, do, d["S0"], dst, workspace=ws)

    def fwd_ck():
        dr.delta_rule_chunk_fwd_checkpointed(*args, d["S0"], o=o, S_T=st, workspace=ws)

    def bwd_reuse():
        dr.delta_rule_chunk_bwd(*args, do, d["S0"], dst, workspace=ws, checkpoints_ready=True)

    def plain_step():
        fwd()
        bwd()

    def ck_step():
        fwd_ck()
        bwd_reuse()

    res = {}
    for key, fn in (("forward_then_backward_us", plain_step),
                    ("checkpointed_forward_then_backward_us", ck_step),
                    ("checkpointed_forward_us", fwd_ck)):
        settle(torch, fn)
        res[key] = round(timed_steps(torch, fn, reps) * 1e6, 2)
    fwd_ck()  # the checkpoints of these inputs, then the backward alone on them
    settle(torch, bwd_reuse)
    res["backward_reusing_checkpoints_us"] = round(timed_steps(torch, bwd_reuse, reps) * 1e6, 2)
    res["workload"] = (f"{w.name} B{w.B} H{w.H} T{w.T} d{w.Dk}, bf16 in, fp32 state; "
                       "forward (chunk 64) + backward, against the checkpointing forward "
                       "(chunk 32) + the backward on its checkpoints")
    return res


def sweep_schedules(torch, dr, W):
    """Chunked vs token-serial forward over sequence length and head dimension
    (plain rule, bf16, H = 16, B = max(1, 16384 / T) sequences, chunk 64, no
    segment schedule): one JSON line per shape with the median call time of
    each schedule (HIP events on the launch stream) and their ratio."""
    for d in (64, 128):
        for T in (16, 64, 256, 1024, 4096, 16384, 32768):
            B = max(1, 16384 // T)
            w = W.get("layer_1p3b", B=B, T=T, Dk=d, Dv=d, seed=31000 + T + d)
            x = W.generate(w)
            dd = {n: (None if t is None else t.cuda()) for n, t in x.items()}
            o = torch.empty((w.B, w.T, w.H, w.Dv), dtype=w.torch_dtype, device="cuda")
            st = torch.empty((w.B, w.H, w.Dv, w.Dk), dtype=torch.float32, device="cuda")
            res = {}
            for serial in (False, True):
                def step():
                    dr.delta_rule_chunk_fwd(dd["q"], dd["k"], dd["v"], dd["beta"], None,
                                            chunk=64, o=o, S_T=st, fused_recurrent=serial,
                                            workspace=False)
                for _ in range(2):
                    step()
                torch.cuda.synchronize()
                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(10)]
                for a, b in ev:
                    a.record()
                    step()
                    b.record()
                torch.cuda.synchronize()
                ts = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
                res["serial" if serial else "chunked"] = ts[len(ts) // 2]
            print(json.dumps({"d": d, "T": T, "B": B, "H": w.H,
                              "chunked_us": round(res["chunked"], 1),
                              "serial_us": round(res["serial"], 1),
                              "speedup": round(res["serial"] / res["chunked"], 2)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=1500,
                    help="untimed steps before the K timed ones (the default is ~0.1 s "
                         "of work, enough for the clock to settle)")
    ap.add_argument("--workload", default="layer_1p3b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-beyond-cache", action="store_true",
                    help="skip the decode run with a state larger than the Infinity Cache "
                         "(it launches the decode kernel on another shape)")
    ap.add_argument("--no-small-model", action="store_true",
                    help="skip the small-model (B4 H8 T2048 d64) line")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward line")
    ap.add_argument("--no-long-prefill", action="store_true",
                    help="skip the long-prefill line")
    ap.add_argument("--no-gated", action="store_true",
                    help="skip the gated-rule lines (chunked layer shape and decode)")
    ap.add_argument("--sweep", action="store_true",
                    help="only print the chunked vs token-serial sweep over T and d")
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="also run a device copy of this many bytes (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the delta-rule kernels shard by "
              "(batch, head) with no communication, and the library runs on a "
              "single MI355X. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import deltanet_delta_rule_amd as dr
    from deltanet_delta_rule_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.sweep:
        sweep_schedules(torch, dr, W)
        return
    dev = torch.device("cuda:0")
    w = W.get(args.workload)
    log(f"generating {w.name}: B{w.B} H{w.H} T{w.T} Dk{w.Dk} Dv{w.Dv} C{w.chunk} {w.dtype}")
    x = W.generate(w)
    d = {n: (None if t is None else t.to(dev)) for n, t in x.items()}
    o = torch.empty((w.B, w.T, w.H, w.Dv), dtype=w.torch_dtype, device=dev)
    st = torch.empty((w.B, w.H, w.Dv, w.Dk), dtype=torch.float32, device=dev)

    def step():
        dr.delta_rule_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["S0"], chunk=w.chunk,
                                o=o, S_T=st)

    if args.copy_calib:
        # a plain elementwise kernel of known traffic: reads n*4 bytes, writes n*4
        n = args.copy_calib // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 2.0, out=dst)
        torch.cuda.synchronize()
        log(f"copy calibration: {n * 4} bytes read, {n * 4} bytes written per launch")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    # the K steps run back to back; one pair of HIP events on the launch
    # stream (the current one) brackets them, so the mean launch duration is
    # their elapsed time / K (dispatch gaps between launches included)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for i in range(K):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_s = ev0.elapsed_time(ev1) / K / 1e3
    log(f"{K} steps: {wall * 1e3 / K:.3f} ms/step wall, {launch_s * 1e6:.1f} us/launch (events)")

    flops, nbytes = chunk_work(w)
    achieved = nbytes / launch_s / 1e9
    traffic = measured_traffic()
    roof = {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "kernel": "chunk_fwd_ws_kernel<bf16, Dk=128, C=64, NW=4> (4 state + 4 preparation waves)",
        "algorithmic_bytes_per_launch": nbytes,
        "mean_launch_us": round(launch_s * 1e6, 2),
        "mfma_frac": round(flops / launch_s / 1e12 / BF16_PEAK_TFLOPS, 4),
        "algorithmic_flops_per_launch": flops,
    }
    out = {
        "metric": METRIC,
        "value": w.B * w.T * K / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "Dk": w.Dk,
                   "Dv": w.Dv, "chunk": w.chunk, "state": "fp32",
                   "parallelism": "single GPU"},
        "roofline": roof,
    }
    if not args.no_small_model:
        log("small model: B4 H8 T2048 d64 chunked forward")
        out["small_model"] = bench_gated_chunk(torch, dr, W, name="small_model")
        out["small_model"]["kernel"] = (
            "segment-parallel schedule, 8 segments of 256 tokens per sequence: "
            "chunk_fwd_ws_kernel<bf16, Dk=64, C=32, NW=4> with map rows (12 waves), "
            "seg_chain_kernel<64>, chunk_fwd_ws_kernel<bf16, Dk=64, C=32, NW=4> (outputs)")
    if not args.no_decode:
        log("decode: 256 steps of B128 H16 d128")
        out["decode"] = bench_decode(torch, dr, W)
        # the 128 MiB state of the decode config fits the 256 MB Infinity
        # Cache; with 512 sequences (512 MiB) it cannot, so this rate is
        # bounded by DRAM
        if not args.no_beyond_cache:
            log("decode beyond the Infinity Cache: 64 steps of B512 H16 d128")
            out["decode"]["beyond_infinity_cache"] = bench_decode(torch, dr, W, B=512, T=64)
    if not args.no_gated:
        log("gated rule: layer shape chunked forward, then 256 decode steps")
        out["gated"] = {"chunk": bench_gated_chunk(torch, dr, W)}
        if not args.no_decode:
            out["gated"]["decode"] = bench_decode(torch, dr, W, name="gated_decode")
        if not args.no_decode:
            log("per-key-channel decay (KDA): 256 decode steps")
            out["kda"] = {"decode": bench_decode(torch, dr, W, name="kda_decode")}
        log("per-key-channel decay (KDA): layer shape sequence forward")
        out.setdefault("kda", {})["sequence"] = bench_kda_sequence(torch, dr, W)
        log("in-kernel q/k L2 norm: layer shape chunked forward")
        out["qk_l2norm"] = {"chunk": bench_gated_chunk(torch, dr, W, name="layer_1p3b", l2=True)}
    if not args.no_long_prefill:
        log("long prefill: B1 H16 T32768, segment-parallel schedule")
        out["long_prefill"] = bench_long_prefill(torch, dr, W)
    if not args.no_backward:
        log("backward: layer shape")
        out["backward"] = bench_backward(torch, dr, W)
        out["backward"]["vs_forward_launch"] = round(
            out["backward"]["mean_call_us"] / roof["mean_launch_us"], 2)
        if not args.no_gated:
            log("backward: gated rule, layer shape")
            out["backward"]["gated"] = bench_backward(torch, dr, W, name="gated_layer_1p3b")
        log("backward: one sequence of the layer shape (two-pass schedule)")
        out["backward"]["one_sequence"] = bench_backward(torch, dr, W, B=1)
        log("training step: forward + backward, with and without reused checkpoints")
        out["backward"]["training_step"] = bench_training_step(torch, dr, W)
        ts = out["backward"]["training_step"]
        ts["backward_reusing_vs_forward_launch"] = round(
            ts["backward_reusing_checkpoints_us"] / roof["mean_launch_us"], 2)
        if not args.no_gated:
            log("backward: KDA, layer shape (token-serial)")
            kb = out["backward"]["kda"] = bench_kda_backward(torch, dr, W)
            kf = out.get("kda", {}).get("sequence")
            if kf:
                kb["vs_kda_forward"] = round(kb["mean_call_us"] / kf["mean_launch_us"], 2)
    if not args.no_cpu_baseline:
        log("cpu baseline: fp64 oracle on the whole workload, then on one thread")
        torch.cuda.synchronize()
        out["cpu_baseline"], out["parity"] = run_cpu_baseline(x, w, o.cpu(), st.cpu())
        out["cpu_baseline"]["single_thread"] = run_cpu_single_thread(x, w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
