#!/usr/bin/env python3
"""Throughput of the MI355X Mamba-3 recurrence: prefill tokens/s/layer and decode
state-updates/s, with roofline fractions and the CPU oracle timed alongside.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long|siso|mimo|decode]

One "step" is one call of the hot path over one batch of synthetic input: a
whole-layer prefill (all heads) for the prefill workloads, or one single-token
decode step over all (sequence, head) pairs for the decode workload.  Inputs are
generated on the device from a fixed seed and are resident in HBM before timing.
Prints ONE JSON line.  The headline `value` is the requested workload, by
default the largest one-GPU configuration: the long-context MIMO prefill
(b=1, L=65536, 32 heads, P=64, N=128, R=4).  Its K timed steps are repeated
three times and `value` / `ms_per_step` are the mean of the three.  The other
configurations (SISO and MIMO prefill, MIMO decode) and the pages' other decode
settings are measured in the same run under "secondary", and the float64 CPU
oracle is timed on a bounded sample of every configuration ("cpu_baseline" for
the headline, "cpu_baselines" for all).
"""
from __future__ import annotations

import argparse
import json
import hashlib
import math
import os
import sys
import time

import torch

import state_space_sequence_02_amd as m3
from state_space_sequence_02_amd import inputs

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA, vendor figure
METRIC = "prefill tokens/s/layer + decode state-updates/s; % of HBM / MFMA roofline"


def esize(w):
    return 2 if w.dtype == "bf16" else 4


def prefill_bytes_per_token_head(w) -> int:
    """Algorithmic bytes: every input read once, y written once."""
    es, R, N, P = esize(w), w.rank, w.dstate, w.headdim
    return R * P * es + 2 * R * N * es + 8 + (N // 2) * 4 * (1 if w.rotation else 0) + R * P * es


def gated_bytes_per_token_head(w) -> int:
    """Algorithmic bytes of the gated call: y [R x P] is replaced by the gate
    input z [P] read and out [P] written."""
    es, R, P = esize(w), w.rank, w.headdim
    return prefill_bytes_per_token_head(w) - R * P * es + 2 * P * es


def gated_readout_torch(y, z, w_y, w_z):
    """The gated readout as plain torch ops (the unfused alternative):
    sum_r w_y y silu(w_z z) over the rank axis, in fp32."""
    g = torch.nn.functional.silu(w_z * z.float().unsqueeze(-2))
    return (w_y * y.float() * g).sum(dim=-2).to(y.dtype)


def prologue_torch(B, C, dt, theta_raw, bias_B, bias_C, eps):
    """The prologue as plain torch ops (the unfused alternative): RMS norm of
    B and C over N in fp32 plus the biases, rounded back to the input dtype,
    and the angle dt * theta_raw."""
    def norm(v, bias):
        f = v.float()
        return (f * torch.rsqrt(f.square().mean(dim=-1, keepdim=True) + eps) + bias).to(v.dtype)
    return norm(B, bias_B), norm(C, bias_C), dt.unsqueeze(-1) * theta_raw


def prefill_flops_per_token_head(w, q) -> float:
    """Algorithmic flops of the chunked form with q tokens/chunk (causal blocks only)."""
    R, N, P = w.rank, w.dstate, w.headdim
    return (q + 1) * R * R * (N + P) + 4 * N * P * R


def backward_bytes_per_token_head(w) -> int:
    """Algorithmic bytes of the backward: the forward inputs and dy read once,
    every gradient (fp32) written once.  The stored forward states (the
    workspace) are the implementation's, not counted."""
    es, R, N, P = esize(w), w.rank, w.dstate, w.headdim
    rot = (N // 2) * 4 if w.rotation else 0
    reads = R * P * es + 2 * R * N * es + 8 + rot + R * P * es
    writes = R * P * 4 + 2 * R * N * 4 + 8 + rot
    return reads + writes


def bench_backward(w, steps, warmup, reps=1):
    """One step = one m3_scan_backward over the whole layer (all heads), from
    seeded inputs and cotangents resident on the device."""
    dev = torch.device("cuda")
    d = inputs.make_prefill_inputs(w, seed=0, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(91)
    dy = torch.randn(d["x"].shape, generator=g, device=dev).to(d["x"].dtype)
    dh = torch.randn((w.batch, w.nheads, w.dstate, w.headdim), generator=g, device=dev)
    dcode = m3.M3_BF16 if w.dtype == "bf16" else m3.M3_FP32
    shape = m3.make_shape(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank, 0, dcode)
    ws = torch.empty(m3.backward_workspace_bytes(shape), dtype=torch.uint8, device=dev)

    def step(i):
        m3.scan_backward(d["x"], d["B"], d["C"], d["dt"], d["A"], d["lam"], d["theta"], dy=dy, dh_out=dh,
                         workspace=ws)

    r = _timed(step, steps, warmup, reps)
    tok = w.batch * w.seqlen
    nbytes = tok * w.nheads * backward_bytes_per_token_head(w) + w.batch * w.nheads * w.dstate * w.headdim * 8
    del d, ws
    return dict(r, tokens_per_s=tok / (r["ms"] * 1e-3), bytes=nbytes,
                gbs_launch=nbytes / (r["ms_launch"] * 1e-3) / 1e9,
                workspace_bytes=m3.backward_workspace_bytes(shape))


def bench_copy(nbytes, steps=200, warmup=30):
    """A plain device-to-device copy of `nbytes` (read once, written once) by
    torch, three buffer pairs in rotation: what streaming the decode's state
    costs with no arithmetic, as a practical ceiling beside the 8 TB/s peak."""
    n = nbytes // 4
    bufs = [(torch.randn(n, device="cuda"), torch.empty(n, device="cuda")) for _ in range(3)]

    def step(i):
        dst, src = bufs[i % 3][1], bufs[i % 3][0]
        dst.copy_(src)

    r = _timed(step, steps, warmup)
    del bufs
    return dict(us_per_launch=round(r["ms_launch"] * 1e3, 2), bytes_moved=2 * nbytes,
                gbs=round(2 * nbytes / (r["ms_launch"] * 1e-3) / 1e9, 1),
                hbm_frac=round(2 * nbytes / (r["ms_launch"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))


def decode_bytes_per_update(w, state_bytes=4) -> int:
    es, R, N, P = esize(w), w.rank, w.dstate, w.headdim
    return (2 * N * P * state_bytes + R * P * es + 2 * R * N * es + R * N * es + R * P * es + 8 + (N // 2) * 4
            + R * P * es)


def table2_intensity(n, p, r):
    """The paper's 2-byte decode arithmetic-intensity model (Table 2)."""
    return (4 * n * p * r + n * p - p * r) / (2 * (1 + 2 * n * r + p * r + n * p))


class StepTimer:
    """HIP events on the current stream (the stream the library launches on):
    one before every step and one after the last, plus (bracket=True) one right
    after every step, so that each launch's own duration is measured apart from
    the gap before the next launch."""

    def __init__(self, steps, bracket=False):
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        self.after = [torch.cuda.Event(enable_timing=True) for _ in range(steps)] if bracket else None

    def mark(self, i):
        self.ev[i].record(torch.cuda.current_stream())

    def mark_after(self, i):
        if self.after is not None:
            self.after[i].record(torch.cuda.current_stream())

    def result(self):
        self.ev[-1].synchronize()
        per = [self.ev[i].elapsed_time(self.ev[i + 1]) for i in range(len(self.ev) - 1)]
        total = self.ev[0].elapsed_time(self.ev[-1])
        per_sorted = sorted(per)
        out = dict(ms=total / len(per), ms_median=per_sorted[len(per) // 2], ms_min=per_sorted[0])
        if self.after is not None:
            own = sorted(self.ev[i].elapsed_time(self.after[i]) for i in range(len(self.after)))
            out.update(ms_launch=sum(own) / len(own), ms_launch_median=own[len(own) // 2])
        return out


PREWARM_S = 0.3


def _timed(step, steps, warmup, reps=1):
    """Times `steps` back-to-back steps (the throughput) `reps` times, then the
    same number again with an event right after each launch (each launch's own
    duration, which is what the kernel-trace profile reports; the extra events
    lengthen the steps of that loop, so it gives no throughput).  `ms` is the
    mean step over the repetitions; `ms_reps` lists each repetition's mean.

    Before the `warmup` untimed steps the step runs for PREWARM_S seconds of
    wall time: the GPU takes tens of milliseconds of steady work to reach its
    running clocks, longer than a few hundred 50 us steps."""
    t_end = time.perf_counter() + PREWARM_S
    i = 0
    while time.perf_counter() < t_end:
        for _ in range(16):
            step(i)
            i += 1
        torch.cuda.synchronize()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    runs = []
    for bracket in [False] * reps + [True]:
        t = StepTimer(steps, bracket)
        for i in range(steps):
            t.mark(i)
            step(i)
            t.mark_after(i)
        t.mark(steps)
        runs.append(t.result())
        torch.cuda.synchronize()
    timed, br = runs[:-1], runs[-1]
    out = dict(ms=sum(r["ms"] for r in timed) / len(timed), ms_reps=[r["ms"] for r in timed],
               ms_median=sorted(r["ms_median"] for r in timed)[len(timed) // 2],
               ms_min=min(r["ms_min"] for r in timed),
               ms_launch=br["ms_launch"], ms_launch_median=br["ms_launch_median"])
    return out


def bench_prefill(w, steps, warmup, chunk=0, nsets=2, gate=None, prologue=None, reps=1, kernel=0):
    """One step = one m3_scan_prefill over the whole layer (all heads), with the
    final state exported; `nsets` input sets alternate so a step cannot be served
    from the last-level cache left warm by the previous one.  gate="fused": one
    m3_scan_prefill_gated (z, w_y, w_z) per step; gate="torch": m3_scan_prefill
    then the same readout in torch ops.  prologue="fused": one
    m3_scan_prefill_prologue (raw angles, B/C biases) per step; "torch": the
    prologue in torch ops, then m3_scan_prefill.  kernel: 0 the library's choice,
    or m3.M3_KERNEL_PER_CHUNK / M3_KERNEL_STREAM (m3_debug_set_prefill_kernel)."""
    m3.debug_set_prefill_kernel(kernel)
    try:
        return _bench_prefill(w, steps, warmup, chunk, nsets, gate, prologue, reps)
    finally:
        m3.debug_set_prefill_kernel(0)


def _bench_prefill(w, steps, warmup, chunk, nsets, gate, prologue, reps):
    dev = torch.device("cuda")
    sets = [inputs.make_prefill_inputs(w, seed=s, device=dev) for s in range(nsets)]
    if prologue:
        g = torch.Generator(device=dev)
        g.manual_seed(79)
        for s in sets:
            s["theta"] = (torch.rand(s["theta"].shape, generator=g, device=dev) * 2 - 1) * math.pi
        pbB = torch.randn((w.nheads, w.rank, w.dstate), generator=g, device=dev) * 0.5
        pbC = torch.randn((w.nheads, w.rank, w.dstate), generator=g, device=dev) * 0.5
    if gate:
        g = torch.Generator(device=dev)
        g.manual_seed(77)
        for s in sets:
            s["z"] = torch.randn((w.batch, w.seqlen, w.nheads, w.headdim), generator=g, device=dev).to(w.torch_dtype)
        wy = torch.randn((w.nheads, w.rank, w.headdim), generator=g, device=dev)
        wz = torch.rand((w.nheads, w.rank, w.headdim), generator=g, device=dev) + 0.5
        outs = [torch.empty((w.batch, w.seqlen, w.nheads, w.headdim), dtype=w.torch_dtype, device=dev)
                for _ in sets]
    dcode = m3.M3_BF16 if w.dtype == "bf16" else m3.M3_FP32
    shape = m3.make_shape(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank, chunk, dcode)
    ws = torch.zeros(m3.prefill_prologue_workspace_bytes(shape) if prologue == "fused" else
                     m3.prefill_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    q_used = m3.prefill_chunk_used(shape, "gated" if gate == "fused" else "prologue" if prologue == "fused" else "plain")
    if q_used == 0:
        raise m3.M3Error(2, f"the library takes no chunk {chunk} for {w.name}")
    staged = prologue == "fused" and m3.prefill_prologue_mode(shape) == m3.M3_PROLOGUE_STAGED
    used = (m3.prefill_prologue_kernel_used(shape) if prologue == "fused" else
            m3.prefill_gated_kernel_used(shape) if gate == "fused" else m3.prefill_kernel_used(shape))
    kern = "stream_kernel" if used == m3.M3_KERNEL_STREAM else "prefill_kernel"
    if staged:
        kern = "prologue stage + " + kern
    ys = [torch.empty_like(s["x"]) for s in sets]
    hs = [torch.empty((w.batch, w.nheads, w.dstate, w.headdim), dtype=torch.float32, device=dev)
          for _ in sets]

    def step(i):
        d = sets[i % nsets]
        if prologue == "fused":
            m3.scan_prefill_prologue(d["x"], d["B"], d["C"], d["dt"], d["A"], d["lam"], d["theta"],
                                     y=ys[i % nsets], h_out=hs[i % nsets], chunk=chunk, workspace=ws,
                                     eps=1e-6, bias_B=pbB, bias_C=pbC)
            return
        if prologue == "torch":
            Bh, Ch, phi = prologue_torch(d["B"], d["C"], d["dt"], d["theta"], pbB, pbC, 1e-6)
            m3.scan_prefill(d["x"], Bh, Ch, d["dt"], d["A"], d["lam"], phi,
                            y=ys[i % nsets], h_out=hs[i % nsets], chunk=chunk, workspace=ws)
            return
        if gate == "fused":
            m3.scan_prefill_gated(d["x"], d["B"], d["C"], d["dt"], d["A"], d["lam"], d["theta"], z=d["z"],
                                  w_y=wy, w_z=wz, out=outs[i % nsets], h_out=hs[i % nsets], chunk=chunk,
                                  workspace=ws)
            return
        m3.scan_prefill(d["x"], d["B"], d["C"], d["dt"], d["A"], d["lam"], d["theta"],
                        y=ys[i % nsets], h_out=hs[i % nsets], chunk=chunk, workspace=ws)
        if gate == "torch":
            outs[i % nsets].copy_(gated_readout_torch(ys[i % nsets], d["z"], wy, wz))

    r = _timed(step, steps, warmup, reps)
    if m3.prefill_status(ws) != 0:
        raise RuntimeError("a prefill look-back wait gave up during the benchmark")
    ms = r["ms"]
    tok = w.batch * w.seqlen
    bpt = gated_bytes_per_token_head(w) if gate else prefill_bytes_per_token_head(w)
    nbytes = tok * w.nheads * bpt + w.batch * w.nheads * w.dstate * w.headdim * 4
    flops = tok * w.nheads * prefill_flops_per_token_head(w, q_used)
    del sets, ys, hs, ws
    msl = r["ms_launch"]
    return dict(r, tokens_per_s=tok / (ms * 1e-3), chunk=q_used, bytes=nbytes, flops=flops, kernel=kern,
                gbs=nbytes / (ms * 1e-3) / 1e9, tflops=flops / (ms * 1e-3) / 1e12,
                gbs_launch=nbytes / (msl * 1e-3) / 1e9, tflops_launch=flops / (msl * 1e-3) / 1e12)


# The paper page's Table 6 decode settings (128 sequences x 32 heads, P = 64):
# name -> (state dtype between steps, overrides of the decode workload).
DECODE_SETTINGS = {
    "mimo": (torch.float32, {}),
    "mimo_bf16_state": (torch.bfloat16, {}),
    "mimo_n64": (torch.float32, dict(dstate=64)),
    "siso_n128": (torch.float32, dict(rank=1)),
    "siso_n64": (torch.float32, dict(rank=1, dstate=64)),
}


def bench_decode(w, steps, warmup, nstate=3, state_dtype=torch.float32, gated=False, prologue=False, reps=1):
    """One step = one m3_decode_step over all (sequence, head) pairs; >= 3 state
    buffers (384 MiB at the 128-sequence shape) rotate so a step cannot be served
    from the 256 MB last-level cache left warm by the previous step.  gated:
    m3_decode_step_gated with a gate input per step and rank weights.  prologue:
    m3_decode_step_prologue with raw angles and B/C biases."""
    dev = torch.device("cuda")
    S = w.steps
    d = inputs.make_decode_inputs(w, seed=0, device=dev)
    if gated:
        g = torch.Generator(device=dev)
        g.manual_seed(78)
        zs = torch.randn((S, w.batch, w.nheads, w.headdim), generator=g, device=dev).to(w.torch_dtype)
        wy = torch.randn((w.nheads, w.rank, w.headdim), generator=g, device=dev)
        wz = torch.rand((w.nheads, w.rank, w.headdim), generator=g, device=dev) + 0.5
        out = torch.empty((w.batch, w.nheads, w.headdim), dtype=w.torch_dtype, device=dev)
    if prologue:
        g = torch.Generator(device=dev)
        g.manual_seed(80)
        d["theta"] = (torch.rand(d["theta"].shape, generator=g, device=dev) * 2 - 1) * math.pi
        pbB = torch.randn((w.nheads, w.rank, w.dstate), generator=g, device=dev) * 0.5
        pbC = torch.randn((w.nheads, w.rank, w.dstate), generator=g, device=dev) * 0.5
    hs = [torch.zeros((w.batch, w.nheads, w.dstate, w.headdim), dtype=state_dtype, device=dev)
          for _ in range(nstate)]
    y = torch.empty_like(d["x"][0])

    def step(i):
        s = i % S
        kw = dict(B_prev=d["B"][s - 1], x_prev=d["x"][s - 1]) if s else {}
        if prologue:
            m3.decode_step_prologue(hs[i % nstate], d["x"][s], d["B"][s], d["C"][s], d["dt"][s], d["A"],
                                    d["lam"][s], d["theta"][s], y=y, eps=1e-6, bias_B=pbB, bias_C=pbC, **kw)
            return
        if gated:
            m3.decode_step_gated(hs[i % nstate], d["x"][s], d["B"][s], d["C"][s], d["dt"][s], d["A"],
                                 d["lam"][s], d["theta"][s], z=zs[s], w_y=wy, w_z=wz, out=out, **kw)
            return
        m3.decode_step(hs[i % nstate], d["x"][s], d["B"][s], d["C"][s], d["dt"][s], d["A"],
                       d["lam"][s], d["theta"][s], y=y, **kw)

    r = _timed(step, steps, warmup, reps)
    ms = r["ms"]
    upd = w.batch * w.nheads
    nbytes = upd * decode_bytes_per_update(w, 2 if state_dtype == torch.bfloat16 else 4)
    if gated:   # y [R x P] replaced by z [P] read and out [P] written
        nbytes += upd * (2 * w.headdim - w.rank * w.headdim) * esize(w)
    del d, hs
    return dict(r, updates_per_s=upd / (ms * 1e-3), tokens_per_s=w.batch / (ms * 1e-3),
                bytes=nbytes, gbs=nbytes / (ms * 1e-3) / 1e9,
                gbs_launch=nbytes / (r["ms_launch"] * 1e-3) / 1e9)


PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "state_space_sequence_02_amd", "csrc")


def kernel_source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(name):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary for this kernel and workload, or None when there is none or the
    kernel's source has changed since the counters were taken."""
    path = os.path.join(PROFILES, f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_digest") != kernel_source_digest(rec.get("sources", [])):
        return None
    return rec.get("bytes_per_launch")


_ORACLE_THREADS = None


def cpu_baseline(w, target_s=10.0):
    """The float64 CPU oracle, as it stands, on a bounded sample of the same
    workload (about target_s seconds on all host cores), scaled to the metric's
    unit.  Prefill: one sequence, min(cores, H) heads, over a prefix of the
    sequence long enough to take about target_s (the oracle's time is linear in
    the tokens and the heads), drawn with the workload's distributions; decode:
    a subset of the sequences, all heads, 16 successive steps."""
    import numpy as np
    import oracle
    global _ORACLE_THREADS
    if _ORACLE_THREADS is None:   # (a run with an explicit count changes the default)
        _ORACLE_THREADS = oracle.max_threads()
    nthreads = _ORACLE_THREADS
    if w.steps:   # decode: a subset of (sequence, head) pairs over 16 steps
        d = inputs.make_decode_inputs(w, seed=0, device="cpu", steps=16)
        def run(npairs):
            seqs = list(range(min(npairs, w.batch)))
            sub = {k: (v[:, seqs] if (v is not None and k != "A") else v) for k, v in d.items()}
            t0 = time.perf_counter()
            oracle.decode_steps(np.zeros((len(seqs), w.nheads, w.dstate, w.headdim)), sub["x"], sub["B"],
                                sub["C"], sub["dt"], sub["A"], sub["lam"], sub["theta"], nthreads=nthreads)
            return time.perf_counter() - t0, len(seqs) * w.nheads * 16
        dt1, u1 = run(1)
        n = max(1, min(w.batch, int(target_s / max(dt1, 1e-3))))
        el, upd = run(n)
        return dict(value=upd / el, unit="state-updates/s", cores=nthreads, kind="oracle",
                    sample=f"{n} sequences x {w.nheads} heads x 16 steps of the {w.name} workload")
    nh = min(nthreads, w.nheads)

    def run(nheads, L, threads=nthreads):
        d = inputs.make_prefill_inputs(w, seed=0, device="cpu", batch=1, seqlen=L)
        heads = list(range(nheads))
        o = {k: (None if v is None else (v[heads] if k == "A" else v[:, :, heads]).double().numpy())
             for k, v in d.items()}
        t0 = time.perf_counter()
        oracle.scan(**o, nthreads=threads)
        return time.perf_counter() - t0
    Lc = min(w.seqlen, 256)
    tc = run(nh, Lc)
    Ls = int(min(w.seqlen, max(Lc, Lc * target_s / max(tc, 1e-3))))
    el = run(nh, Ls)
    tokens_per_s = (Ls * nh / w.nheads) / el
    L1 = min(w.seqlen, max(64, Ls // 8))
    el1 = run(1, L1, threads=1)   # one head on one core
    return dict(value=tokens_per_s, unit="tokens/s/layer", cores=nthreads, kind="oracle",
                sample=f"1 sequence x {nh} of {w.nheads} heads x the first {Ls} of {w.seqlen} tokens, "
                       "scaled to a full layer",
                value_1thread=(L1 / w.nheads) / el1)


PREFILL_SOURCES = {"prefill_kernel": ["m3_fused_kernel.h", "m3_device.h", "m3_internal.h"],
                   "stream_kernel": ["m3_stream.hip", "m3_fused_kernel.h", "m3_device.h", "m3_internal.h"]}
DECODE_SOURCES = ["m3_decode.hip", "m3_device.h", "m3_internal.h"]


def prefill_chunk_for(w, requested):
    """The chunk a prefill workload runs at: the requested one when the library
    takes it, else the largest it takes below it (the long workload's 128-token
    chunk is 512 (token, rank) rows, which do not fit one compute unit)."""
    dcode = m3.M3_BF16 if w.dtype == "bf16" else m3.M3_FP32
    shape = m3.make_shape(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank, requested, dcode)
    if requested == 0 or m3.prefill_chunk_used(shape) == requested:
        return requested
    return min(requested, m3.prefill_max_chunk(shape))


def prefill_line(w, rr):
    return dict(tokens_per_s_layer=rr["tokens_per_s"], us=round(rr["ms"] * 1e3, 1),
                us_median=round(rr["ms_median"] * 1e3, 1), chunk=rr["chunk"], kernel=rr["kernel"],
                us_per_launch=round(rr["ms_launch"] * 1e3, 1),
                hbm_frac=round(rr["gbs_launch"] / HBM_PEAK_GBS, 4),
                mfma_frac=round(rr["tflops_launch"] / MFMA_BF16_PEAK_TFS, 4))


def decode_line(wl, rr, state="fp32"):
    return dict(state_updates_per_s=rr["updates_per_s"], us_per_step=round(rr["ms"] * 1e3, 1),
                us_median=round(rr["ms_median"] * 1e3, 1), us_per_launch=round(rr["ms_launch"] * 1e3, 1),
                hbm_gbs=round(rr["gbs_launch"], 1), hbm_frac=round(rr["gbs_launch"] / HBM_PEAK_GBS, 4),
                state=state, dstate=wl.dstate, rank=wl.rank)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--reps", type=int, default=3, help="repetitions of the timed steps (mean reported)")
    ap.add_argument("--workload", default="long", choices=["long", "siso", "mimo", "decode", "tiny"])
    ap.add_argument("--chunk", type=int, default=-1,
                    help="prefill tokens per chunk (-1: the configuration's; 0: library default)")
    ap.add_argument("--kernel", default="auto", choices=["auto", "per_chunk", "stream"],
                    help="prefill kernel of the headline line (auto: the one the library takes)")
    ap.add_argument("--prologue", action="store_true",
                    help="headline prefill through m3_scan_prefill_prologue (raw angles, B/C biases)")
    ap.add_argument("--backward", action="store_true",
                    help="headline: the backward (m3_scan_backward, every gradient) at the prefill workload's shape")
    ap.add_argument("--decode-setting", default="mimo", choices=sorted(DECODE_SETTINGS),
                    help="decode workload only: which of the Table 6 decode settings is the headline")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(heads and sequences shard with no communication; see the design notes).",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    m3.load_library()
    torch.cuda.synchronize()

    w = inputs.WORKLOADS[args.workload]
    if w.steps:
        state_dtype, kw = DECODE_SETTINGS[args.decode_setting]
        w = inputs.workload("decode", **kw)
        r = bench_decode(w, args.steps * 10, args.warmup * 10, state_dtype=state_dtype, reps=args.reps)
        value, unit, ms = r["updates_per_s"], "state-updates/s", r["ms"]
        traffic = measured_traffic("decode_kernel_decode" if args.decode_setting == "mimo"
                                   else f"decode_kernel_{args.decode_setting}")
        roof = dict(bound="hbm", achieved=round(r["gbs_launch"], 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(r["gbs_launch"] / HBM_PEAK_GBS, 4), traffic=traffic, kernel="decode_kernel",
                    algorithmic_bytes_per_launch=r["bytes"], us_per_launch=round(r["ms_launch"] * 1e3, 2))
        config = dict(workload=f"decode: {w.batch} seq x {w.nheads} heads, N={w.dstate}, P={w.headdim}, "
                               f"R={w.rank}, bf16 in, {'bf16' if state_dtype == torch.bfloat16 else 'fp32'} state",
                      batch=w.batch, nheads=w.nheads, dstate=w.dstate, headdim=w.headdim, rank=w.rank,
                      state_buffers=3)
        steps_done = args.steps * 10
    elif args.backward:
        r = bench_backward(w, args.steps, args.warmup, reps=args.reps)
        value, unit, ms = r["tokens_per_s"], "tokens/s/layer", r["ms"]
        roof = dict(bound="hbm", achieved=round(r["gbs_launch"], 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(r["gbs_launch"] / HBM_PEAK_GBS, 4), traffic=None,
                    kernel="m3_scan_backward (five launches)", algorithmic_bytes_per_launch=r["bytes"],
                    us_per_launch=round(r["ms_launch"] * 1e3, 2))
        config = dict(workload=f"{w.name} backward: b={w.batch}, L={w.seqlen}, H={w.nheads}, P={w.headdim}, "
                               f"N={w.dstate}, R={w.rank}, {w.dtype} in, fp32 gradients",
                      batch=w.batch, seq_len=w.seqlen, nheads=w.nheads, dstate=w.dstate,
                      headdim=w.headdim, rank=w.rank, workspace_bytes=r["workspace_bytes"])
        steps_done = args.steps
    else:
        requested = w.chunk if args.chunk < 0 else args.chunk
        chunk = prefill_chunk_for(w, requested)
        kernel = {"auto": 0, "per_chunk": m3.M3_KERNEL_PER_CHUNK, "stream": m3.M3_KERNEL_STREAM}[args.kernel]
        r = bench_prefill(w, args.steps, args.warmup, chunk=chunk, reps=args.reps, kernel=kernel,
                          prologue="fused" if args.prologue else None)
        value, unit, ms = r["tokens_per_s"], "tokens/s/layer", r["ms"]
        traffic = measured_traffic(f"{r['kernel']}_{w.name}_q{r['chunk']}")
        roof = dict(bound="hbm", achieved=round(r["gbs_launch"], 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(r["gbs_launch"] / HBM_PEAK_GBS, 4), traffic=traffic,
                    kernel=r["kernel"],
                    algorithmic_bytes_per_launch=r["bytes"],
                    us_per_launch=round(r["ms_launch"] * 1e3, 2),
                    mfma_tflops=round(r["tflops_launch"], 2),
                    mfma_frac=round(r["tflops_launch"] / MFMA_BF16_PEAK_TFS, 4),
                    algorithmic_flops_per_launch=r["flops"])
        config = dict(workload=f"{w.name} prefill{' with the prologue' if args.prologue else ''}: b={w.batch}, L={w.seqlen}, H={w.nheads}, P={w.headdim}, "
                               f"N={w.dstate}, R={w.rank}, {w.dtype} in, fp32 state",
                      batch=w.batch, seq_len=w.seqlen, nheads=w.nheads, dstate=w.dstate,
                      headdim=w.headdim, rank=w.rank, chunk=r["chunk"], chunk_requested=requested)
        if requested and r["chunk"] != requested:
            config["chunk_note"] = (f"the configuration's {requested}-token chunk is {requested * w.rank} "
                                    f"(token, rank) rows, which do not fit one compute unit; the largest "
                                    f"chunk the library takes is used (the result does not depend on it)")
        steps_done = args.steps
    out = dict(metric=METRIC, value=value, unit=unit, n_gpus=1, steps=steps_done, warmup=args.warmup,
               ms_per_step=ms, ms_reps=r["ms_reps"], reps=args.reps, ms_median=r["ms_median"], ms_min=r["ms_min"],
               higher_is_better=True, scaling="weak", vs_baseline=None,
               dtype="bf16" if w.dtype == "bf16" else "f32", data="synthetic (seeded, on device)",
               config=config, roofline=roof)
    if not args.no_secondary:
        sec = {}
        for name, q in (("siso", 64), ("siso", 0), ("mimo", 64), ("long", 128)):
            if name == args.workload and (q == 0) == (args.chunk == 0):
                continue
            wl = inputs.WORKLOADS[name]
            steps = args.steps if name != "long" else max(3, args.steps // 4)
            key = f"{name}_prefill" + ("_default_chunk" if q == 0 else "")
            sec[key] = prefill_line(wl, bench_prefill(wl, steps, max(2, args.warmup // 5),
                                                      chunk=prefill_chunk_for(wl, q)))
        # the N = 128 workloads on the per-chunk kernel, beside the streaming
        # kernel the library takes for them
        for name in ("long", "mimo"):
            wl = inputs.WORKLOADS[name]
            steps = args.steps if name != "long" else max(3, args.steps // 4)
            sec[f"{name}_prefill_per_chunk_kernel"] = prefill_line(
                wl, bench_prefill(wl, steps, max(2, args.warmup // 5), chunk=prefill_chunk_for(wl, wl.chunk),
                                  kernel=m3.M3_KERNEL_PER_CHUNK))
        wd = inputs.WORKLOADS["decode"]
        if args.workload != "decode":
            rd = bench_decode(wd, 200, 30)
            sec["mimo_decode"] = dict(decode_line(wd, rd),
                                      table2_intensity=round(table2_intensity(wd.dstate, wd.headdim, wd.rank), 2))
        # the paper page's Table 6 decode settings: SISO and MIMO, state size 64
        # or 128, fp32 or bf16 state (128 sequences x 32 heads, P=64)
        def dec(name, setting):
            state_dtype, kw = DECODE_SETTINGS[setting]
            wl = inputs.workload("decode", **kw)
            rr = bench_decode(wl, 200, 30, state_dtype=state_dtype)
            sec[name] = dict(decode_line(wl, rr, "bf16" if state_dtype == torch.bfloat16 else "fp32"),
                             traffic=measured_traffic(f"decode_kernel_{setting}"))
        dec("mimo_decode_bf16_state", "mimo_bf16_state")
        dec("mimo_decode_n64", "mimo_n64")
        dec("siso_decode_n128", "siso_n128")
        dec("siso_decode_n64", "siso_n64")
        # torch's device copy of the decode states' bytes (N=64 fp32 or N=128
        # bf16: 64 MiB; N=128 fp32: 128 MiB), read once and written once
        sec["device_copy_64MiB"] = bench_copy(64 << 20)
        sec["device_copy_128MiB"] = bench_copy(128 << 20)
        # the gated readout (rank contraction + rank-expanded SiLU gate) fused
        # into the kernels, and the prefill's unfused alternative
        wm = inputs.WORKLOADS["mimo"]
        rf = bench_prefill(wm, args.steps, max(2, args.warmup // 5), chunk=64, gate="fused")
        rt = bench_prefill(wm, args.steps, max(2, args.warmup // 5), chunk=64, gate="torch")
        sec["mimo_prefill_gated"] = dict(prefill_line(wm, rf), us_unfused_torch_readout=round(rt["ms"] * 1e3, 1))
        rw = bench_decode(wd, 200, 30, nstate=1)
        sec["mimo_decode_warm"] = dict(us_per_launch=round(rw["ms_launch"] * 1e3, 1),
                                       state_updates_per_s=rw["updates_per_s"],
                                       note="one state buffer reused every step, so the 128 MiB state "
                                            "could be served from the 256 MB last-level cache")
        rg = bench_decode(wd, 200, 30, gated=True)
        sec["mimo_decode_gated"] = decode_line(wd, rg)
        # the prologue (BCNorm + B/C biases + angle = dt x raw angle) through
        # m3_scan_prefill_prologue, and the unfused alternative (the prologue in
        # torch ops first): fused into the per-chunk kernel on the SISO
        # workload and into the streaming kernel on the MIMO workload
        for name in ("siso", "mimo"):
            ws_ = inputs.WORKLOADS[name]
            pf = bench_prefill(ws_, args.steps, max(2, args.warmup // 5), chunk=64, prologue="fused")
            pt = bench_prefill(ws_, args.steps, max(2, args.warmup // 5), chunk=64, prologue="torch")
            sec[f"{name}_prefill_prologue"] = dict(prefill_line(ws_, pf),
                                                   us_unfused_torch_prologue=round(pt["ms"] * 1e3, 1))
        rp = bench_decode(wd, 200, 30, prologue=True)
        sec["mimo_decode_prologue"] = decode_line(wd, rp)
        # the backward of the recurrence (every gradient), at the SISO and MIMO
        # prefill shapes
        for name in ("siso", "mimo"):
            wl = inputs.WORKLOADS[name]
            rb = bench_backward(wl, 3, 1)
            sec[f"{name}_backward"] = dict(tokens_per_s_layer=rb["tokens_per_s"], us=round(rb["ms"] * 1e3, 1),
                                           us_per_launch=round(rb["ms_launch"] * 1e3, 1),
                                           hbm_frac=round(rb["gbs_launch"] / HBM_PEAK_GBS, 4),
                                           algorithmic_bytes_per_launch=rb["bytes"],
                                           workspace_bytes=rb["workspace_bytes"])
        out["secondary"] = sec
    if not args.no_cpu_baseline:
        base = {}
        for name in ("tiny", "siso", "mimo", "decode", "long"):
            base[name] = cpu_baseline(inputs.WORKLOADS[name], target_s=1.0 if name == "tiny" else 10.0)
        out["cpu_baseline"] = base[args.workload]
        out["cpu_baselines"] = base
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
