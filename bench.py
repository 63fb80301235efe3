#!/usr/bin/env python3
"""Benchmark of the selective-scan hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step is one full pass of the path over one batch of synthetic input: for the
prefill workloads one ssm_scan_fwd call (chunk summaries, carry scan, rescan with
the fused epilogue); for the decode workload one token for every layer and
sequence (one ssm_step call per layer, as a model would issue them). Inputs are
drawn with the seeded recipe of ``workloads`` and are resident in HBM before the
timed region starts. W untimed warm-up steps are followed by exactly K timed
steps bracketed by device synchronisation. Prints one JSON line.

By default all five workloads run, one after another, each with its own timing,
roofline and CPU baseline (the "workloads" key); the headline fields are the
long-context prefill's (batch 1, L = 262144, 8192 channels, N = 16, bf16 inputs,
fp32 state), at which the throughput target is set. --workload NAME runs one.

Roofline: the dominant kernel's average duration is measured with HIP events
recorded by the library itself on the launch stream (ssm_scan_fwd_profiled), and
its algorithmic bytes against 8 TB/s are the headline (bound "hbm": the metric's
roofline). Beside it, "alu_view" gives the vector-ALU issue ceiling: VALU
instructions per element, and issue slots per element with a transcendental
charged two slots, against 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz, and what that
ceiling allows in elements/s and as a fraction of HBM peak. HBM traffic measured
with rocprofv3 counters is read from profiles/traffic.json when it was taken on
the current kernel source (by hash), else null.

With no variant flag the run ends with the 256k prefill's backward ("backward": ssm_scan_bwd,
and ssm_scan_bwd_saved from the training forward's stored states).

The CPU baseline is the fp64 oracle as it stands, run on a bounded sample of the
same workload (a subset of channels over the full sequence; channels are
independent) from as many threads as this process has host cores (its CPU affinity,
capped by a cgroup quota if one is set), with nproc and the CPU model recorded.

--fused times the same workload through ssm_scan_fwd_fused / ssm_step_fused instead:
x is the input of the MambaBlock's causal depthwise convolution (--conv-k taps,
default 4) and dt the raw dt projection output, and the convolution + silu and
softplus run inside the scan's load stage (decode: with the carried conv state).
--trap times the exponential-trapezoidal entry points (--trap-weight random: with the
per-step weight stream), --mimo R the MIMO ones (rank-R
inputs and outputs per channel; elements stay channel-steps, each with R outputs).
--backward times ssm_scan_bwd on a prefill workload, and with --fused ssm_scan_bwd_fused
(the gradients through the input stage as well), with --saved ssm_scan_bwd_saved from the
states ssm_scan_fwd_save stored (with --fused: ssm_scan_bwd_fused_saved from
ssm_scan_fwd_fused_save's; that forward timed apart). --one-call times the decode as one call
over all layers per token instead of one call per layer.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz: one fp32 VALU instruction per lane per clock
# (non-packed; the published 157.3 TFLOP/s counts packed fp32 FMAs as 4 flops).
VALU_PEAK_TLANE = 256 * 4 * 16 * 2.4e9 / 1e12
METRIC = "scan elements (batch·L·D_inner)/s at N=16; achieved HBM GB/s vs peak"
CSRC = "selective_state_space_49_amd/csrc/"
COMMON_HEADERS = [CSRC + "ssm_device.h", CSRC + "ssm_stream.h"]
KERNEL_SOURCES = {
    "real": [CSRC + "scan_real.hip", CSRC + "ssm_input_stage.h"],
    "complex": [CSRC + "scan_complex.hip"],
    "step": [CSRC + "step.hip", CSRC + "ssm_input_stage.h"],
    "bwd": [CSRC + "scan_bwd.hip", CSRC + "scan_real.hip", CSRC + "ssm_input_stage.h"],
    "mimo": [CSRC + "scan_mimo.hip", CSRC + "scan_real.hip"],
    "mimo_step": [CSRC + "scan_mimo.hip"],
}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def source_hash(kind: str) -> str:
    """Hash of the code (comments and whitespace removed) of a kernel kind's sources: the
    stored traffic of a kernel is reported only while this hash is the one it was
    counted under."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind] + COMMON_HEADERS:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------- algorithmic work
def prefill_bytes(s, io_bytes: int) -> float:
    """Each input read once, each output written once (never dA or dB)."""
    b, L, Dn, N = s.batch, s.L, s.d_inner, s.d_state
    c = 2 if s.complex_state else 1
    streams = 3 + (1 if s.gated else 0)                     # x, dt, (z), y
    return (b * L * Dn * streams * io_bytes + 2 * b * L * N * c * io_bytes
            + Dn * N * c * 4 + Dn * 4 + b * Dn * N * c * 4)


def prefill_lane_ops(s) -> float:
    """Vector-ALU instructions per scan element (one lane-op each; a transcendental
    counts as one instruction like any other). Real state, per state: dt*A, exp,
    (dt x)*B, fma (state), fma (output) = 5. Complex state, per state: dt*a, exp,
    dt*theta, fract, sin, cos, 2 mul (decay x rotation), 2 mul (dt x B), 4 fma (complex
    update), 2 fma (real part of C h) = 16. Per element: dt*x, D*x + acc; with bf16 I/O
    the widening of x and dt and the output conversion; gated: the gate (mul, exp, add,
    rcp, mul, mul) and, with bf16 I/O, the widening of z. The complex state spreads a
    channel over P = 4 lanes, each of which does the per-element work, plus the sum over
    its P lanes (2 DPP adds) and, with bf16 I/O, the widening of its share of the staged
    B and C rows (one per lane-step)."""
    bf16 = s.io == "bf16"
    per_state = 16 if s.complex_state else 5
    per_elem = 2 + (3 if bf16 else 0)
    if s.gated:
        per_elem += 6 + (1 if bf16 else 0)
    if s.complex_state:
        P = min(s.d_state, 4)
        per_elem = P * (per_elem + (P.bit_length() - 1) + (1 if bf16 else 0))
    return s.d_state * per_state + per_elem


def trap_lane_ops(N: int) -> float:
    """Extra VALU instructions per element of the exponential-trapezoidal update: per
    state one more fused multiply-add (the previous input term), per element w = dt/2,
    w x_prev and w x in place of dt x (two more)."""
    return N + 2


def mimo_prefill_bytes(s, io_bytes: int, R: int) -> float:
    """MIMO prefill: x, (z), y of R elements per channel-step, dt of one, B and C of N x R
    per step, A, D, h_final; each read or written once."""
    b, L, Dn, N = s.batch, s.L, s.d_inner, s.d_state
    streams = R * (2 + (1 if s.gated else 0)) + 1
    return (b * L * Dn * streams * io_bytes + 2 * b * L * N * R * io_bytes
            + Dn * N * 4 + Dn * 4 + b * Dn * N * 4)


def mimo_lane_ops(s, R: int, matrix: bool = False) -> float:
    """VALU instructions per channel-step of the MIMO update (one lane per channel).
    VALU path, per state: dt*A, exp, the R-term sum B x (one multiply, R-1 fused
    multiply-adds), the state's fused multiply-add, and R output fused multiply-adds =
    3 + 2R; per channel-step: dt*x[r] and D x[r] + acc[r] (2R). Matrix path (the prefill
    from rank 4: B x on the matrix cores), per state: dt*A, exp, dt*v, the state's fused
    multiply-add and R output fused multiply-adds = 4 + R; with bf16 I/O and at least 4
    states the output sums run on the matrix cores too, leaving per state dt*A, exp, dt*v,
    the state's fused multiply-add and half a conversion (the state packed to bf16 two
    at a time for the matrix operand) = 4.5. Per channel-step on the matrix path D x[r] +
    acc[r] (R). All: with bf16 I/O the widening of x and dt and the output conversion
    (R + 1 + ceil(R/2): outputs are packed two to an instruction); gated: the gate per
    output (6R) and, with bf16, the widening of z (R). The matrix operations (2 N R flops
    per channel-step for B x, 2 N R more for the outputs) are not VALU work. R = 1 gives
    prefill_lane_ops."""
    bf16 = s.io == "bf16"
    out_matrix = matrix and bf16 and s.d_state >= 4
    per_elem = (R if matrix else 2 * R) + ((R + 1 + (R + 1) // 2) if bf16 else 0)
    if s.gated:
        per_elem += 6 * R + (R if bf16 else 0)
    per_state = 4.5 if out_matrix else (4 + R) if matrix else (3 + 2 * R)
    return s.d_state * per_state + per_elem


def mimo_decode_bytes(s, io_bytes: int, R: int) -> float:
    """MIMO decode token for all layers: state read + write, x, (z), y of R elements and
    dt per channel, B and C of N x R per (layer, sequence), A, D."""
    Ln, S, Dn, N = s.n_layers, s.n_seq, s.d_inner, s.d_state
    return (Ln * S * Dn * N * 4 * 2 + Ln * S * Dn * (R * (2 + (1 if s.gated else 0)) + 1) * io_bytes
            + 2 * Ln * S * N * R * io_bytes + Ln * Dn * (N + 1) * 4)


def input_stage_bytes(s, io_bytes: int, K: int) -> float:
    """Extra bytes of the fused input stage: filter, biases, carried conv state in/out
    (the raw x and dt replace x and dt one for one)."""
    return s.d_inner * (K + (1 if K else 0) + 1) * 4 + 2 * s.batch * max(K - 1, 0) * s.d_inner * io_bytes


def input_stage_lane_ops(K: int) -> float:
    """Vector-ALU instructions per element of the fused input stage. softplus(dt + bias):
    add, mul, exp, add, sub, log, mul, rcp, mul, mul, compare, select, max, add = 14.
    Convolution: K fma, then silu (mul, exp, add, rcp, mul) = K + 5."""
    return 14 + (K + 5 if K else 0)


def decode_bytes(s, io_bytes: int) -> float:
    """Per token for all layers: state read + write, token inputs/outputs, A, D."""
    Ln, S, Dn, N = s.n_layers, s.n_seq, s.d_inner, s.d_state
    return (Ln * S * Dn * N * 4 * 2 + Ln * S * Dn * (4 if s.gated else 3) * io_bytes
            + 2 * Ln * S * N * io_bytes + Ln * Dn * (N + 1) * 4)


def backward_bytes(s, io_bytes: int) -> float:
    """Backward, each input read once and each gradient written once: x, dt, z, dy read,
    dx, ddt, dz written; B, C read and dB, dC (fp32) written; A, D, dA, dD. The states
    stored every 8 steps and read back are traffic of the method, not of the algorithm."""
    b, L, Dn, N = s.batch, s.L, s.d_inner, s.d_state
    streams = 3 + 2 * (1 if s.gated else 0) + 1 + 1          # x, dt, (z), dy / dx, ddt, (dz)
    return (b * L * Dn * streams * io_bytes + 2 * b * L * N * (io_bytes + 4)
            + 2 * Dn * (N + 1) * 4)


def backward_lane_ops(s, saved=False) -> float:
    """VALU instructions per element of the backward: a forward walk storing the states
    every 8 steps (4 per state + dt*x and widening; none with the training forward's
    states), the recomputation of each 4-step piece (the same, and once more for every
    second piece, whose start is not stored), and the backward step (12 per state: exp argument, exp, lam, a h, lam a h,
    dB and dC terms, B.lam, A.lam a h, dA, lam a, C.h; plus about 20 per element for the
    gate's derivative, dx, ddt, dz and conversions), plus the sums of dB and dC over the
    wave (2N values over 64 lanes: 2N - 1 exchanges of two or three instructions plus the
    last levels, 70 for N = 16)."""
    N = s.d_state
    walk = 4 * N + 3
    bfly = {1: 6, 2: 8, 4: 15, 8: 33, 16: 70}[N]
    return (0 if saved else walk) + 1.5 * walk + 12 * N + 20 + bfly


def decode_lane_ops(s) -> float:
    """Vector-ALU instructions per channel of a decode step: 5 per state as in prefill,
    dt*x, D*x + acc, the pairwise tree over the G = 4 lanes of a channel (2 adds), and
    with bf16 I/O the widening and conversion; gated: the gate and the widening of z."""
    bf16 = s.io == "bf16"
    per_elem = 2 + 2 + (3 if bf16 else 0)
    if s.gated:
        per_elem += 6 + (1 if bf16 else 0)
    return 5 * s.d_state + per_elem


# ----------------------------------------------------------------- runs
def run_backward(shape, steps, warmup, torch, ssm, workloads, chunk_len=0, conv_k=None,
                 saved=False):
    """One step = one ssm_scan_bwd call over the workload (dy ~ N(0, 1) in the I/O dtype);
    with conv_k, one ssm_scan_bwd_fused call (the input stage of a conv_k-tap filter:
    x and dt of the workload are then the raw x_in and dt_raw). saved: one
    ssm_scan_bwd_saved call (with conv_k, ssm_scan_bwd_fused_saved) from the states one
    ssm_scan_fwd_save (ssm_scan_fwd_fused_save) call stored (that forward is timed too,
    apart, and reported beside the backward)."""
    dev = "cuda"
    log("drawing inputs for", shape.name, "(backward)")
    d = workloads.make_scan_inputs(shape, dev)
    g = torch.Generator(device=dev).manual_seed(shape.seed + 29)
    dy = torch.randn(d["x"].shape, generator=g, device=dev).to(d["x"].dtype)
    b, L, Dn, N = shape.batch, shape.L, shape.d_inner, shape.d_state
    fused = conv_k is not None
    if fused:
        d.update(workloads.make_input_stage(shape, conv_k, dev))
        io = 1 if shape.io == "bf16" else 0
        need = (ssm.ssm_scan_bwd_fused_saved_workspace if saved else ssm.ssm_scan_bwd_fused_workspace)(
            b, L, Dn, N, conv_k, io, chunk_len)
    elif saved:
        need = ssm.ssm_scan_bwd_saved_workspace(b, L, Dn, N, chunk_len)
    else:
        need = ssm.ssm_scan_bwd_workspace(b, L, Dn, N, chunk_len)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    log("backward workspace", ws.numel() / 1e9, "GB")
    out = {}
    fwd_ms = None
    if saved:
        states = torch.empty(ssm._states_shape(b, L, Dn, N), dtype=torch.float32, device=dev)
        log("stored states", states.numel() * 4 / 1e9, "GB")
        fws = torch.empty(max(ssm.ssm_scan_fwd_save_workspace(b, L, Dn, N, chunk_len), 1),
                          dtype=torch.uint8, device=dev)
        yb = torch.empty_like(d["x"])
        # the fused training forward stores the scan's inputs u and dt as well
        u_st = torch.empty_like(d["x"]) if fused else None
        dt_st = torch.empty_like(d["x"]) if fused else None

        def fwd():
            if fused:
                ssm.ssm_scan_fwd_fused_save(d["x"], d["dt_raw"], d["A"], d["B"], d["C"], d["D"], d["z"],
                                            conv_w=d["conv_w"], conv_b=d["conv_b"],
                                            conv_state0=d["conv_state0"], dt_bias=d["dt_bias"], y=yb,
                                            states=states, u_out=u_st, dt_out=dt_st, chunk_len=chunk_len,
                                            workspace=fws, want_conv_state=False)
                return
            ssm.ssm_scan_fwd_save(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], y=yb,
                                  states=states, chunk_len=chunk_len, workspace=fws)
        for _ in range(max(warmup, 1)):
            fwd()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fwd()
        e1.record()
        torch.cuda.synchronize()
        fwd_ms = e0.elapsed_time(e1) / steps
        log("forward with stored states", round(fwd_ms, 4), "ms")

    def call():
        if saved and fused:
            ssm.ssm_scan_bwd_fused_saved(d["x"], d["dt_raw"], d["A"], d["B"], d["C"], d["D"], d["z"],
                                         states=states, u=u_st, dt=dt_st, conv_w=d["conv_w"], conv_b=d["conv_b"],
                                         conv_state0=d["conv_state0"], dt_bias=d["dt_bias"], dy=dy,
                                         chunk_len=chunk_len, workspace=ws, want_dh0=False,
                                         want_dconv_state0=False)
            return
        if saved:
            r = ssm.ssm_scan_bwd_saved(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"],
                                       states=states, dy=dy, chunk_len=chunk_len, workspace=ws,
                                       out=out, want_dh0=False)
            out.update(r)
            return
        if fused:
            ssm.ssm_scan_bwd_fused(d["x"], d["dt_raw"], d["A"], d["B"], d["C"], d["D"], d["z"],
                                   conv_w=d["conv_w"], conv_b=d["conv_b"], conv_state0=d["conv_state0"],
                                   dt_bias=d["dt_bias"], dy=dy, chunk_len=chunk_len, workspace=ws,
                                   want_dh0=False, want_dconv_state0=False)
            return
        r = ssm.ssm_scan_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], dy=dy,
                             chunk_len=chunk_len, workspace=ws, out=out, want_dh0=False)
        out.update(r)

    log("warmup", warmup)
    for _ in range(max(warmup, 1)):
        call()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log("timing", steps, "steps")
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        call()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1) / steps
    io_bytes = 2 if shape.io == "bf16" else 4
    nbytes, lane_ops = backward_bytes(shape, io_bytes), backward_lane_ops(shape, saved)
    if fused:
        # recompute of u, dt (x_in, dt_raw read; u, dt written) and the chain rule (x_in,
        # dt_raw, du, ddt read; dx_in, ddt_raw written): 10 more streams; the input stage
        # forward once more, and its backward: per tap an fma for a_t, dx_in and dw, silu'
        # (exp, add, rcp, sub, fma, 2 mul) and softplus' (add, mul, exp, add, rcp, mul, add).
        # From the fused training forward's u and dt (saved): the chain rule only.
        nbytes += (6 if saved else 10) * shape.elements * io_bytes
        lane_ops += (0 if saved else input_stage_lane_ops(conv_k)) + 3 * conv_k + 14
    phases = {"backward_call": gpu_ms}
    if saved:
        phases["forward_with_stored_states"] = fwd_ms
    info = {
        "wall_s": wall, "ms_per_step": wall / steps * 1e3, "phases_ms": phases,
        "elements_per_step": shape.elements, "bytes_per_step": nbytes,
        "lane_ops_per_elem": lane_ops, "chunk_len": chunk_len,
        "n_chunks": None, "dominant_ms": gpu_ms, "gpu_ms": gpu_ms,
        "kernel": ("ssm_scan_bwd_fused" if fused else "ssm_scan_bwd") + ("_saved" if saved else "")
                  + " (all launches)",
        "source": "bwd",
    }
    return info, d


def run_prefill(shape, steps, warmup, torch, ssm, workloads, chunk_len=0, conv_k=None, trap=False,
                mimo=0, lam=False):
    """conv_k None: ssm_scan_fwd; else ssm_scan_fwd_fused with a conv_k-tap filter.
    trap: ssm_scan_fwd_trap (exponential-trapezoidal), with an input before step 0.
    mimo R > 0: ssm_scan_fwd_mimo with rank-R projections."""
    dev = "cuda"
    log("drawing inputs for", shape.name)
    d = workloads.make_mimo_inputs(shape, mimo, dev) if mimo else workloads.make_scan_inputs(shape, dev)
    if trap:
        d.update(workloads.make_prev_input(shape.batch, shape.d_inner, shape.d_state, shape.io, dev))
        d["lam"] = (workloads.make_trap_weight((shape.batch, shape.L, shape.d_inner), shape.io, dev,
                                               kind="random") if lam else None)
    fused = conv_k is not None
    if fused:
        d.update(workloads.make_input_stage(shape, conv_k, dev))
        d["dt"] = None                      # the fused path reads dt_raw instead
    b, L, Dn, N = shape.batch, shape.L, shape.d_inner, shape.d_state
    cplx = shape.complex_state
    y = torch.empty_like(d["x"])
    hf = torch.empty((b, Dn, N) + ((2,) if cplx else ()), dtype=torch.float32, device=dev)
    T = chunk_len or (ssm.ssm_scan_fwd_c64_chunk_len(b, L, Dn, N) if cplx
                      else ssm.ssm_scan_fwd_mimo_chunk_len(b, L, Dn, N, mimo) if mimo
                      else ssm.ssm_scan_fwd_fused_chunk_len(b, L, Dn, N) if fused
                      else ssm.ssm_scan_fwd_chunk_len(b, L, Dn, N))
    ws_n = (ssm.ssm_scan_fwd_c64_workspace(b, L, Dn, N, T) if cplx
            else ssm.ssm_scan_fwd_mimo_workspace(b, L, Dn, N, mimo, T) if mimo
            else ssm.ssm_scan_fwd_workspace_ex(b, L, Dn, N, T))
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)
    fn = ssm.ssm_scan_fwd_c64_profiled if cplx else ssm.ssm_scan_fwd_profiled
    so = (torch.empty_like(d["conv_state0"]) if fused and d["conv_state0"] is not None else None)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for row in ev:                      # create the underlying HIP events
        for e in row:
            e.record()
    warm_ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in warm_ev:
        e.record()
    torch.cuda.synchronize()

    def call(events):
        if fused:
            ssm.ssm_scan_fwd_fused(d["x"], d["dt_raw"], d["A"], d["B"], d["C"], d["D"], d["z"], None,
                                   conv_w=d["conv_w"], conv_b=d["conv_b"],
                                   conv_state0=d["conv_state0"], dt_bias=d["dt_bias"], y=y,
                                   h_final=hf, conv_state_out=so, workspace=ws, chunk_len=T,
                                   events=[e.cuda_event for e in events])
        elif trap:
            ssm.ssm_scan_fwd_trap(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], None,
                                  d["x_prev"], d["B_prev"], lam=d["lam"], y=y, h_final=hf,
                                  workspace=ws, chunk_len=T, events=[e.cuda_event for e in events])
        elif mimo:
            ssm.ssm_scan_fwd_mimo(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], None,
                                  y=y, h_final=hf, workspace=ws, chunk_len=T,
                                  events=[e.cuda_event for e in events])
        else:
            fn(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], None, y=y, h_final=hf,
               workspace=ws, chunk_len=T, events=[e.cuda_event for e in events])

    log("warmup", warmup)
    for _ in range(warmup):
        call(warm_ev)
    torch.cuda.synchronize()
    log("timing", steps, "steps")
    t0 = time.perf_counter()
    for k in range(steps):
        call(ev[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    phases = {"summary": 0.0, "carry": 0.0, "rescan": 0.0}
    for row in ev:
        phases["summary"] += row[0].elapsed_time(row[1])
        phases["carry"] += row[1].elapsed_time(row[2])
        phases["rescan"] += row[2].elapsed_time(row[3])
    phases = {k: v / steps for k, v in phases.items()}
    gpu_ms = sum(phases.values())
    io_bytes = 2 if shape.io == "bf16" else 4
    elems = shape.elements
    nbytes = prefill_bytes(shape, io_bytes)
    lane_ops = prefill_lane_ops(shape)
    if fused:
        nbytes += input_stage_bytes(shape, io_bytes, conv_k)
        lane_ops += input_stage_lane_ops(conv_k)
    if trap:
        nbytes += shape.batch * (shape.d_inner + shape.d_state) * io_bytes   # x_prev, B_prev
        lane_ops += trap_lane_ops(shape.d_state)
        if lam:  # the weight stream: read once; widened, 1 - lam and one more product
            nbytes += elems * io_bytes
            lane_ops += 3 if shape.io == "bf16" else 2
    if mimo:
        nbytes = mimo_prefill_bytes(shape, io_bytes, mimo)
        lane_ops = mimo_lane_ops(shape, mimo, matrix=mimo >= 4)
    info = {
        "wall_s": wall, "ms_per_step": wall / steps * 1e3, "phases_ms": phases,
        "elements_per_step": elems, "bytes_per_step": nbytes,
        "lane_ops_per_elem": lane_ops, "chunk_len": T,
        "n_chunks": -(-L // T), "dominant_ms": phases["rescan"], "gpu_ms": gpu_ms,
        "kernel": "k_chunk_scan_c" if cplx else "k_mimo_scan" if mimo else "k_chunk_scan",
        "source": "complex" if cplx else "mimo" if mimo else "real",
    }
    return info, d


def run_decode(shape, steps, warmup, torch, ssm, workloads, graph=True, conv_k=None, trap=False,
               mimo=0, one_call=False, lam=False):
    """conv_k None: ssm_step; else ssm_step_fused with a conv_k-tap filter. trap:
    ssm_step_trap, given the previous token's x and B. mimo R > 0: ssm_step_mimo.
    one_call: each token is one call over all layers (n_layers = Ln: the [layers, seqs,
    ...] tensors as they are) instead of one call per layer."""
    dev = "cuda"
    Ln, S, Dn, N = shape.n_layers, shape.n_seq, shape.d_inner, shape.d_state
    par = workloads.make_decode_params(shape, dev)
    h = torch.zeros((Ln, S, Dn, N), device=dev)
    log("drawing", warmup + steps, "token steps of inputs")
    toks = [workloads.make_mimo_decode_step(shape, mimo, k, dev) if mimo
            else workloads.make_decode_step(shape, k, dev) for k in range(warmup + steps)]
    if trap:  # each token's weight (random in [0, 1]) or none (1/2)
        for k, t in enumerate(toks):
            t["lam"] = (workloads.make_trap_weight((Ln, S, Dn), shape.io, dev, kind="random", seed=100 + k)
                        if lam else None)
    fused = conv_k is not None
    if fused:
        ist = workloads.make_decode_input_stage(shape, conv_k, dev)
        for k, t in enumerate(toks):
            t["dt"] = workloads.make_decode_dt_raw(shape, k, dev)
        sl = lambda v, l: None if v is None else v[l:l + 1]
        ist_l = [{k: sl(v, l) for k, v in ist.items()} for l in range(Ln)]
    y = torch.empty(tuple(toks[0]["x"].shape), dtype=toks[0]["x"].dtype, device=dev)
    A_l = [par["A"][l:l + 1] for l in range(Ln)]
    D_l = [par["D"][l:l + 1] for l in range(Ln)]
    h_l = [h[l:l + 1] for l in range(Ln)]
    per_layer = [{k: (None if v is None else v[l:l + 1]) for k, v in t.items()} for t in toks
                 for l in range(Ln)]
    calls = 1 if one_call else Ln  # calls per token
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps * calls)]

    def call(t, pv, hh, A, D, p, yy):
        if fused:
            ssm.ssm_step_fused(hh, p["conv_state"], t["x"], t["dt"], A, t["B"], t["C"], D, t["z"],
                               conv_w=p["conv_w"], conv_b=p["conv_b"], dt_bias=p["dt_bias"], y_t=yy)
        elif trap:
            ssm.ssm_step_trap(hh, pv["x"], pv["B"], t["x"], t["dt"], A, t["B"], t["C"], D, t["z"],
                              lam_t=t["lam"], y_t=yy)
        elif mimo:
            ssm.ssm_step_mimo(hh, t["x"], t["dt"], A, t["B"], t["C"], D, t["z"], y_t=yy)
        else:
            ssm.ssm_step(hh, t["x"], t["dt"], A, t["B"], t["C"], D, t["z"], y_t=yy)

    def token(k, timed):
        for l in range(calls):
            if timed:
                ev[2 * ((k - warmup) * calls + l)].record()
            if one_call:
                pv = toks[k - 1] if k > 0 else {"x": None, "B": None}
                call(toks[k], pv, h, par["A"], par["D"], ist if fused else None, y)
            else:
                pv = per_layer[(k - 1) * Ln + l] if k > 0 else {"x": None, "B": None}
                call(per_layer[k * Ln + l], pv, h_l[l], A_l[l], D_l[l], ist_l[l] if fused else None,
                     y[l:l + 1])
            if timed:
                ev[2 * ((k - warmup) * calls + l) + 1].record()

    for k in range(warmup):
        token(k, False)
    torch.cuda.synchronize()
    if graph:
        # One captured graph per token: the Ln per-layer calls, bound to that token's
        # inputs (drawn beforehand), replayed back to back. Capture happens outside the
        # timed region; the graph holds no memset nodes.
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for k in range(warmup, warmup + steps):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    token(k, False)
                graphs.append(g)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        gev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        h.zero_()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        gev[0].record()
        for g in graphs:
            g.replay()
        gev[1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        kern = gev[0].elapsed_time(gev[1]) / (steps * calls)
    else:
        t0 = time.perf_counter()
        for k in range(warmup, warmup + steps):
            token(k, True)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        kern = sum(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps * calls)) / (steps * calls)
    io_bytes = 2 if shape.io == "bf16" else 4
    nbytes = decode_bytes(shape, io_bytes)
    lane_ops = decode_lane_ops(shape)
    if fused:
        K = conv_k
        nbytes += Ln * S * Dn * 2 * max(K - 1, 0) * io_bytes + Ln * Dn * (K + (1 if K else 0) + 1) * 4
        lane_ops += input_stage_lane_ops(K)
    if trap:
        nbytes += Ln * S * (Dn + N) * io_bytes   # the previous token's x and B
        lane_ops += trap_lane_ops(N)
        if lam:
            nbytes += Ln * S * Dn * io_bytes     # the token's weight
            lane_ops += 3 if shape.io == "bf16" else 2
    if mimo:
        nbytes = mimo_decode_bytes(shape, io_bytes, mimo)
        lane_ops = mimo_lane_ops(shape, mimo)
    info = {
        "wall_s": wall, "ms_per_step": wall / steps * 1e3,
        "elements_per_step": Ln * S * Dn, "bytes_per_step": nbytes,
        "lane_ops_per_elem": lane_ops, "dominant_ms": kern * calls, "per_call_ms": kern,
        "kernel": "k_mimo_step" if mimo else "k_step", "source": "mimo_step" if mimo else "step",
        "phases_ms": {"ssm_step_all_layers" if one_call else "ssm_step_per_layer": kern},
        "graph": graph, "calls_per_token": calls,
    }
    return info, None


def traffic_for(info, workload):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tab = json.load(f)
    ent = tab.get(workload)
    if not ent or ent.get("source_sha") != source_hash(info["source"]):
        return None
    return ent.get("hbm_bytes_per_launch")


# Elements in the oracle's CPU sample: about 1-2 s of wall time on 16 host threads
# (10-30 s of CPU work) for the real-state forward and backward; the complex oracle
# costs about 4 times more per element.
CPU_SAMPLE_ELEMS = 1 << 27


def sample_width(shape, elems):
    # channels to sample so that the whole sequence of every batch row gives ~elems
    return max(1, min(shape.d_inner, -(-elems // (shape.batch * max(shape.L, 1)))))


def cpu_baseline(shape, d, torch, workloads, threads, conv_k=None, trap=False, mimo=0):
    import oracle
    oracle.build(force=False)
    k = sample_width(shape, CPU_SAMPLE_ELEMS // (4 if shape.complex_state else 1))
    idx = workloads.sample_channels(shape.d_inner, k, seed=5).to("cuda")
    g = lambda t: None if t is None else t.index_select(2, idx).cpu()
    args = (g(d["x"]), g(d["dt"]), d["A"].index_select(0, idx).cpu(), d["B"].cpu(), d["C"].cpu(),
            d["D"].index_select(0, idx).cpu(), g(d["z"]))
    log("cpu baseline: oracle on", k, "channels x", shape.L, "steps x batch", shape.batch,
        "with", threads, "threads")
    t0 = time.perf_counter()
    if conv_k is not None:
        # the oracle's input stage on the sample (one thread), then its scan as above
        sel = lambda t: None if t is None else t.index_select(0, idx).cpu()
        u = (oracle.conv_silu(args[0], sel(d["conv_w"]), sel(d["conv_b"]),
                              g(d["conv_state0"]))[0] if conv_k else args[0])
        dts = oracle.softplus(g(d["dt_raw"]), sel(d["dt_bias"]))
        args = (u, dts) + args[2:]
    if trap or mimo:
        import threading
        import numpy as np
        xp = oracle.to_f64(d["x_prev"].index_select(1, idx).cpu()) if trap else None
        Bq = oracle.to_f64(d["B_prev"].cpu()) if trap else None
        lw = (oracle.to_f64(d["lam"].index_select(2, idx).cpu())
              if trap and d.get("lam") is not None else None)
        f = [oracle.to_f64(a) for a in args]
        parts = [p for p in np.array_split(np.arange(k), threads) if len(p)]

        def work(p):
            sub = lambda a: None if a is None else np.ascontiguousarray(a[:, :, p])
            if mimo:
                oracle.scan_mimo(sub(f[0]), sub(f[1]), f[2][p], f[3], f[4], f[5][p], sub(f[6]))
            else:
                oracle.scan_trap(sub(f[0]), sub(f[1]), f[2][p], f[3], f[4], f[5][p], sub(f[6]),
                                 x_prev=np.ascontiguousarray(xp[:, p]), B_prev=Bq,
                                 lam=None if lw is None else sub(lw))
        t0 = time.perf_counter()
        ts = [threading.Thread(target=work, args=(p,)) for p in parts]
        for t in ts: t.start()
        for t in ts: t.join()
    else:
        oracle.scan_threaded(*args, threads=threads, complex_state=shape.complex_state)
    dt = time.perf_counter() - t0
    elems = shape.batch * shape.L * k
    # The same oracle on one thread, over one thread's share of the sample (the first
    # k / threads channels), so that it takes about as long as the run above.
    k1 = max(1, k // threads)
    t1 = time.perf_counter()
    if trap or mimo:
        work(np.arange(k1))
    else:
        import numpy as np

        def one(t, dim):  # the first k1 channels (torch tensors, or numpy after the input stage)
            if t is None:
                return None
            v = t[:, :, :k1] if dim == 2 else t[:k1]
            return v.contiguous() if hasattr(v, "contiguous") else np.ascontiguousarray(v)
        oracle.scan_threaded(one(args[0], 2), one(args[1], 2), one(args[2], 0), args[3], args[4],
                             one(args[5], 0), one(args[6], 2), threads=1, complex_state=shape.complex_state)
    dt1 = time.perf_counter() - t1
    elems1 = shape.batch * shape.L * k1
    return {"value": elems / dt, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "sample": f"{k} of {shape.d_inner} channels over all {shape.L} steps x batch "
                      f"{shape.batch} ({elems} elements, {dt:.1f} s wall), fp64 sequential loop "
                      f"per channel{' (exponential-trapezoidal)' if trap else ''}"
                      f"{f' (MIMO, rank {mimo})' if mimo else ''}, channels split "
                      f"over {threads} threads",
            "value_1_core": elems1 / dt1,
            "sample_1_core": f"the first {k1} of those channels on one thread ({elems1} elements, "
                             f"{dt1:.1f} s wall)"}


def cpu_baseline_backward(shape, d, torch, workloads, threads, conv_k=None):
    """The oracle's backward on a channel sample over the full sequence, channel groups on
    several threads (dB and dC then cover the sampled channels only; the per-element work
    is the same)."""
    import threading
    import numpy as np
    import oracle
    oracle.build(force=False)
    k = sample_width(shape, CPU_SAMPLE_ELEMS // 2)
    idx = workloads.sample_channels(shape.d_inner, k, seed=5)
    g = lambda t: None if t is None else oracle.to_f64(t.index_select(2, idx.to(t.device)))
    x, dt, z = g(d["x"]), g(d["dt_raw"] if conv_k is not None else d["dt"]), g(d["z"])
    sel = lambda t: None if t is None else oracle.to_f64(t.index_select(0, idx.to(t.device)))
    if conv_k is not None:
        cw, cb, db, cs = sel(d["conv_w"]), sel(d["conv_b"]), sel(d["dt_bias"]), g(d["conv_state0"])
    A, B, C, D = (oracle.to_f64(d["A"].index_select(0, idx.to(d["A"].device))), oracle.to_f64(d["B"]),
                  oracle.to_f64(d["C"]), oracle.to_f64(d["D"].index_select(0, idx.to(d["D"].device))))
    dy = np.random.default_rng(3).normal(0, 1, x.shape)
    parts = [p for p in np.array_split(np.arange(k), threads) if len(p)]
    log("cpu baseline (backward): oracle on", k, "channels x", shape.L, "steps with", len(parts), "threads")

    def work(p):
        sub = lambda a: None if a is None else np.ascontiguousarray(a[:, :, p])
        if conv_k is not None:
            oracle.scan_fused_bwd(sub(x), sub(dt), A[p], B, C, D[p], sub(z),
                                  conv_w=None if cw is None else cw[p], conv_b=None if cb is None else cb[p],
                                  conv_state0=sub(cs), dt_bias=None if db is None else db[p], dy=sub(dy))
        else:
            oracle.scan_bwd(sub(x), sub(dt), A[p], B, C, D[p], sub(z), dy=sub(dy))

    t0 = time.perf_counter()
    ts = [threading.Thread(target=work, args=(p,)) for p in parts]
    for t in ts: t.start()
    for t in ts: t.join()
    dtm = time.perf_counter() - t0
    elems = shape.batch * shape.L * k
    t1 = time.perf_counter()
    work(parts[0])  # one thread's share on one thread, timed alone
    dt1 = time.perf_counter() - t1
    elems1 = shape.batch * shape.L * len(parts[0])
    return {"value": elems / dtm, "unit": "elements/s", "cores": len(parts), "kind": "oracle",
            "value_1_core": elems1 / dt1,
            "sample_1_core": f"the first {len(parts[0])} of those channels on one thread ({elems1} elements, "
                             f"{dt1:.1f} s wall)",
            "sample": f"{'backward through the input stage' if conv_k is not None else 'backward'}: "
                      f"{k} of {shape.d_inner} channels over all {shape.L} steps x batch "
                      f"{shape.batch} ({elems} elements, {dtm:.1f} s wall), fp64 loops per channel "
                      f"(forward keeping every state, then backward), channels split over "
                      f"{len(parts)} threads"}


def cpu_baseline_decode(shape, workloads, threads, conv_k=None, seqs=4, tokens=192, trap=False,
                        mimo=0):
    """The oracle's decode step (or, with conv_k, its fused step) for every layer on the
    first `seqs` sequences, `tokens` tokens in a row with the state carried, the layers
    split over host threads. Inputs are drawn once; the timed region is the oracle."""
    import threading
    import numpy as np
    import oracle
    oracle.build(force=False)
    Ln, Dn, N = shape.n_layers, shape.d_inner, shape.d_state
    S = min(seqs, shape.n_seq)
    par = workloads.make_decode_params(shape, "cpu")
    tok = (workloads.make_mimo_decode_step(shape, mimo, 0, "cpu") if mimo
           else workloads.make_decode_step(shape, 0, "cpu"))
    sl = lambda t: None if t is None else np.ascontiguousarray(oracle.to_f64(t[:, :S]))
    x, z, B, C = sl(tok["x"]), sl(tok["z"]), sl(tok["B"]), sl(tok["C"])
    A, D = oracle.to_f64(par["A"]), oracle.to_f64(par["D"])
    fused = conv_k is not None
    if fused:
        ist = workloads.make_decode_input_stage(shape, conv_k, "cpu")
        dt = sl(workloads.make_decode_dt_raw(shape, 0, "cpu"))
        f64 = lambda t: None if t is None else oracle.to_f64(t)
        cw, cb, db = f64(ist["conv_w"]), f64(ist["conv_b"]), f64(ist["dt_bias"])
        cs = sl(ist["conv_state"]) if ist["conv_state"] is not None else np.zeros((Ln, S, max(conv_k - 1, 0), Dn))
        if conv_k == 0:  # no convolution: the input stage is softplus(dt + bias) alone
            dt = np.stack([oracle.softplus(dt[l], db[l]) for l in range(Ln)])
    else:
        dt = sl(tok["dt"])
    h = np.zeros((Ln, S, Dn, N))
    groups = [(int(g[0]), int(g[-1]) + 1) for g in np.array_split(np.arange(Ln), min(threads, Ln)) if len(g)]
    log("cpu baseline (decode): oracle on", Ln, "layers x", S, "sequences x", tokens, "tokens with",
        len(groups), "threads")

    def work(l0, l1):
        r = slice(l0, l1)
        hh, cc = h[r], (cs[r] if fused else None)
        for _ in range(tokens):
            if fused and conv_k > 0:
                _, hh, cc = oracle.step_fused(hh, cc, x[r], dt[r], A[r], B[r], C[r], D[r], z if z is None else z[r],
                                              conv_w=cw[r], conv_b=None if cb is None else cb[r],
                                              dt_bias=None if db is None else db[r])
            elif mimo:
                _, hh = oracle.step_mimo(hh, x[r], dt[r], A[r], B[r], C[r], D[r], None if z is None else z[r])
            elif trap:  # the same token's x and B stand in for the previous token's
                _, hh = oracle.step_trap(hh, x[r], B[r], x[r], dt[r], A[r], B[r], C[r], D[r],
                                         None if z is None else z[r])
            else:
                _, hh = oracle.step(hh, x[r], dt[r], A[r], B[r], C[r], D[r], None if z is None else z[r])

    t0 = time.perf_counter()
    ts = [threading.Thread(target=work, args=g) for g in groups]
    for t in ts: t.start()
    for t in ts: t.join()
    dtm = time.perf_counter() - t0
    elems = Ln * S * Dn * tokens
    # one thread's share of the layers on one thread, timed alone
    n1 = max(1, Ln // len(groups))
    t1 = time.perf_counter()
    work(0, n1)
    dt1 = time.perf_counter() - t1
    elems1 = n1 * S * Dn * tokens
    what = ("fused decode step (conv + silu, softplus, scan)" if fused else
            "exponential-trapezoidal decode step" if trap else
            f"MIMO decode step (rank {mimo})" if mimo else "decode step")
    return {"value": elems / dtm, "unit": "elements/s", "cores": len(groups), "kind": "oracle",
            "sample": f"{what}: all {Ln} layers x {S} of {shape.n_seq} sequences x {Dn} channels, "
                      f"{tokens} tokens (token 0's inputs each time) with the state carried ({elems} "
                      f"elements, {dtm:.1f} s wall), "
                      f"fp64, layers split over {len(groups)} threads",
            "value_1_core": elems1 / dt1,
            "sample_1_core": f"the first {n1} of those layers on one thread ({elems1} elements, {dt1:.1f} s wall)"}


def trans_per_elem(shape, variant: dict) -> float:
    """Transcendental instructions (exp, log, rcp, sin, cos) among the VALU instructions
    per element: the hardware issues each in two slots (SQ_ACTIVE_INST_VALU charges it
    twice), so issue slots per element = VALU instructions + transcendentals. Real state:
    one exp per state; complex: exp, sin, cos per state; the gate exp + rcp per output;
    the input stage softplus (exp, log, rcp) and silu (exp, rcp); the backward: the
    forward walk, the recomputation and the adjoint update each one exp per state, and
    the gate's derivative (exp, rcp)."""
    N = shape.d_state
    g = 2 if getattr(shape, "gated", True) else 0
    if variant.get("backward"):
        t = 3 * N + g
        if variant.get("conv_k") is not None:
            t += 3 + (2 if variant["conv_k"] else 0) + 3
        return t
    R = variant.get("mimo") or 1
    t = (3 * N if getattr(shape, "complex_state", False) else N) + g * R
    if variant.get("conv_k") is not None:
        t += 3 + (2 if variant["conv_k"] else 0)
    return t


def host_cpus() -> dict:
    """The host cores this process may use: the CPU affinity set, capped by a cgroup CPU
    quota where one is set, plus nproc and the CPU model for the record."""
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    quota = None
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            q, per = f.read().split()[:2]
            if q != "max":
                quota = float(q) / float(per)
    except (OSError, ValueError):
        pass
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    usable = aff if quota is None else max(1, min(aff, int(quota + 0.5)))
    return {"nproc": os.cpu_count(), "affinity": aff, "cgroup_quota_cores": quota,
            "cpu_model": model, "threads": usable}


def measure(name, variant, steps, warmup, with_cpu, threads, cpus, torch, ssm, workloads,
            chunk_len=0, graph=True, one_call=False):
    """Run one workload (one configuration of the path) and return its record."""
    shape = workloads.WORKLOADS[name]
    is_decode = isinstance(shape, workloads.DecodeShape)
    conv_k, trap, mimo, backward = (variant.get("conv_k"), variant.get("trap", False),
                                    variant.get("mimo", 0), variant.get("backward", False))
    saved = backward and variant.get("saved", False)
    lam = trap and variant.get("lam", False)
    steps = max(1, steps if not is_decode else min(steps, 64))
    if is_decode:
        info, d = run_decode(shape, steps, warmup, torch, ssm, workloads, graph=graph, conv_k=conv_k,
                             trap=trap, mimo=mimo, one_call=one_call, lam=lam)
    elif backward:
        info, d = run_backward(shape, steps, warmup, torch, ssm, workloads, chunk_len, conv_k,
                               saved=saved)
    else:
        info, d = run_prefill(shape, steps, warmup, torch, ssm, workloads, chunk_len, conv_k,
                              trap=trap, mimo=mimo, lam=lam)
    elems_s = info["elements_per_step"] / (info["ms_per_step"] / 1e3)
    dom_s = info["dominant_ms"] / 1e3
    hbm_ach = info["bytes_per_step"] / dom_s / 1e9
    lane_ops = info["lane_ops_per_elem"]
    trans = trans_per_elem(shape, variant)
    slots = lane_ops + trans
    alu_ach = info["elements_per_step"] * lane_ops / dom_s / 1e12
    slot_ach = info["elements_per_step"] * slots / dom_s / 1e12
    traffic_key = name + (f"+input_stage_k{conv_k}" if conv_k is not None else "") + \
        ("+backward" if backward else "") + ("_saved" if saved else "") + ("+trap" if trap else "") + \
        ("_lam" if lam else "") + \
        (f"+mimo{mimo}" if mimo else "") + ("+one_call" if is_decode and one_call else "")
    # The metric names the HBM roofline: it is the headline bound for every workload;
    # the vector-ALU issue ceiling, which the bf16 and complex prefills reach first, is
    # reported beside it.
    roof = {"bound": "hbm", "achieved": round(hbm_ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(hbm_ach / HBM_PEAK_GBS, 4), "traffic": traffic_for(info, traffic_key),
            "kernel": info["kernel"],
            "kernel_ms": round(info["dominant_ms"] if not is_decode else info["per_call_ms"], 4),
            "bytes_per_launch": info["bytes_per_step"] if not is_decode else
            info["bytes_per_step"] / info["calls_per_token"],
            "alu_view": {
                "valu_instr_per_elem": lane_ops, "transcendental_per_elem": trans,
                "issue_slots_per_elem": slots,
                "achieved_T_instr_s": round(alu_ach, 2), "achieved_T_slots_s": round(slot_ach, 2),
                "peak_T_slots_s": round(VALU_PEAK_TLANE, 2),
                "frac_instr": round(alu_ach / VALU_PEAK_TLANE, 4),
                "frac_issue_slots": round(slot_ach / VALU_PEAK_TLANE, 4),
                "ceiling_elements_s": round(VALU_PEAK_TLANE * 1e12 / slots, 1),
                "ceiling_hbm_frac": round(VALU_PEAK_TLANE * 1e12 / slots * info["bytes_per_step"]
                                          / info["elements_per_step"] / 1e9 / HBM_PEAK_GBS, 4),
                "note": "issue slots charge a transcendental two, as SQ_ACTIVE_INST_VALU does; "
                        "transcendentals partly overlap other VALU issue, so frac_issue_slots can "
                        "pass 1 and the slot ceiling is a little below what the chip sustains"}}
    if is_decode:
        cfg = {"workload": shape.name, "n_layers": shape.n_layers, "n_seq": shape.n_seq,
               "d_inner": shape.d_inner, "d_state": shape.d_state, "io": shape.io, "state": "f32",
               "calls_per_step": info["calls_per_token"], "hip_graph_per_token": info["graph"]}
        if conv_k is not None:
            cfg["input_stage"] = {"conv_k": conv_k, "conv_silu": conv_k > 0, "softplus_dt": True,
                                  "entry_point": "ssm_step_fused"}
        if trap:
            cfg["discretisation"] = "exponential-trapezoidal (ssm_step_trap)"
            cfg["trap_weight"] = "random per token and channel" if lam else "1/2 (none given)"
        if mimo:
            cfg["mimo_rank"] = mimo
            cfg["entry_point"] = "ssm_step_mimo"
    else:
        cfg = {"workload": shape.name, "batch": shape.batch, "L": shape.L, "d_inner": shape.d_inner,
               "d_state": shape.d_state, "io": shape.io, "state": "c64" if shape.complex_state else "f32",
               "complex_state": shape.complex_state, "gated": shape.gated,
               "chunk_len": info["chunk_len"], "n_chunks": info["n_chunks"]}
        if conv_k is not None:
            cfg["input_stage"] = {"conv_k": conv_k, "conv_silu": conv_k > 0, "softplus_dt": True,
                                  "entry_point": "ssm_scan_fwd_fused"}
        if backward:
            cfg["pass"] = ("backward through the input stage from the fused training forward's stored "
                           "states (ssm_scan_bwd_fused_saved: dx_in, ddt_raw, dconv_w, dconv_b, ddt_bias, "
                           "dz, dA, dB, dC, dD)" if conv_k is not None and saved else
                           "backward through the input stage (ssm_scan_bwd_fused: dx_in, ddt_raw, dconv_w, "
                           "dconv_b, ddt_bias, dz, dA, dB, dC, dD)" if conv_k is not None else
                           "backward from the training forward's stored states (ssm_scan_bwd_saved: "
                           "dx, ddt, dz, dA, dB, dC, dD)" if saved else
                           "backward (ssm_scan_bwd: dx, ddt, dz, dA, dB, dC, dD)")
        if trap:
            cfg["discretisation"] = "exponential-trapezoidal (ssm_scan_fwd_trap)"
            cfg["trap_weight"] = "random per step and channel" if lam else "1/2 (none given)"
        if mimo:
            cfg["mimo_rank"] = mimo
            cfg["entry_point"] = "ssm_scan_fwd_mimo"
    whole = info["bytes_per_step"] / (info["ms_per_step"] / 1e3) / 1e9
    rec = {"value": round(elems_s, 1), "unit": "elements/s", "steps": steps, "warmup": warmup,
           "ms_per_step": round(info["ms_per_step"], 4), "config": cfg,
           "achieved_hbm_GBps_whole_step": round(whole, 1),
           "hbm_frac_whole_step": round(whole / HBM_PEAK_GBS, 4),
           "phases_ms": {k: round(v, 4) for k, v in info["phases_ms"].items()},
           "roofline": roof}
    if "summary" in info["phases_ms"]:
        # The chunk summaries walk back only until every state's decay reaches 2^-H
        # (H = 28 + the bit length of the chunk length), so their time depends on dt and
        # A: slow decay walks whole chunks.
        rec["summary_depends_on_inputs"] = ("chunk summaries walk back until the decay reaches "
                                            "2^-H (H = 28 + the bit length of the chunk length, "
                                            "41 at 256k); slower decay (smaller dt*|A|) walks more "
                                            "of each chunk")
    if mimo:
        rec["mimo_outputs_per_s"] = round(elems_s * mimo, 1)  # R outputs per channel-step
    cpu = None
    if with_cpu and not (is_decode and shape.complex_state):
        if is_decode:
            cpu = cpu_baseline_decode(shape, workloads, threads, conv_k, trap=trap, mimo=mimo)
        elif backward:
            cpu = cpu_baseline_backward(shape, d, torch, workloads, threads, conv_k)
        else:
            cpu = cpu_baseline(shape, d, torch, workloads, threads, conv_k, trap=trap, mimo=mimo)
        cpu.update({"nproc": cpus["nproc"], "cpu_model": cpus["cpu_model"],
                    "affinity_cores": cpus["affinity"], "cgroup_quota_cores": cpus["cgroup_quota_cores"]})
    rec["cpu_baseline"] = cpu
    del d
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def copy_ceiling(torch, nbytes=1 << 32, reps=5):
    """Practical HBM ceiling for context: a device-to-device copy of nbytes (read + write
    of nbytes each), best of reps, timed with events on the current stream."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    del src, dst
    torch.cuda.empty_cache()
    gbs = 2 * nbytes / (best / 1e3) / 1e9
    return {"GBps": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "what": f"device copy of {nbytes >> 30} GiB (read + write), best of {reps}, torch copy_"}


# The five workloads of the metric, in the order they run by default; the 256k prefill
# (the configuration the metric is quoted on) is the headline.
ALL_WORKLOADS = ["tiny_f32", "jamba_layer_prefill", "long_context_256k", "batched_decode",
                 "complex_rotation"]
HEADLINE = "long_context_256k"


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None,
                    help="one workload only (default: all five, the 256k prefill as the headline; "
                         "with --fused, --trap, --mimo or --backward: the 256k prefill)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="oracle threads (default: every host core this process may use)")
    ap.add_argument("--chunk-len", type=int, default=0,
                    help="prefill chunk length (0 = the library's own plan)")
    ap.add_argument("--no-graph", action="store_true",
                    help="decode: launch the per-layer calls eagerly instead of replaying one "
                         "captured HIP graph per token")
    ap.add_argument("--one-call", action="store_true",
                    help="decode: one call per token over all layers (n_layers = 28 in one "
                         "launch) instead of one call per layer")
    ap.add_argument("--fused", action="store_true",
                    help="through ssm_scan_fwd_fused / ssm_step_fused (conv + silu and softplus "
                         "fused into the load stage)")
    ap.add_argument("--conv-k", type=int, default=4, help="filter taps with --fused (0..4)")
    ap.add_argument("--trap", action="store_true",
                    help="the exponential-trapezoidal entry points (ssm_scan_fwd_trap, ssm_step_trap)")
    ap.add_argument("--trap-weight", choices=("none", "random"), default="none",
                    help="with --trap: no weight (1/2, the trapezoid rule) or a random weight in "
                         "[0, 1] per step and channel (the weight stream)")
    ap.add_argument("--mimo", type=int, default=0, metavar="R",
                    help="the MIMO entry points (ssm_scan_fwd_mimo, ssm_step_mimo) with rank R "
                         "(1, 2, 4 or 8)")
    ap.add_argument("--backward", action="store_true",
                    help="time ssm_scan_bwd (gradients of the prefill) on the prefill workload")
    ap.add_argument("--saved", action="store_true",
                    help="with --backward: ssm_scan_bwd_saved from ssm_scan_fwd_save's stored "
                         "states (with --fused: ssm_scan_bwd_fused_saved from "
                         "ssm_scan_fwd_fused_save's; the forward timed apart)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 1 GiB three times (reference for "
                         "the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this path is built and measured on a single "
              f"MI355X (asked for --gpus {args.gpus}). Across GPUs the channels would shard with no "
              f"exchange, or the sequence with one exchange of chunk summaries; neither is implemented.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import selective_state_space_49_amd as ssm
    import workloads
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        nbytes = 1 << 30
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "launches": 3}))
        return
    ssm.load_library()
    variant = {"conv_k": args.conv_k if args.fused else None, "trap": args.trap, "mimo": args.mimo,
               "backward": args.backward, "lam": args.trap_weight == "random",
               "saved": args.saved}
    is_variant = args.fused or args.trap or args.mimo or args.backward
    names = [args.workload] if args.workload else ([HEADLINE] if is_variant else ALL_WORKLOADS)
    for n in names:
        shape = workloads.WORKLOADS[n]
        is_decode = isinstance(shape, workloads.DecodeShape)
        if args.trap and (args.fused or args.backward or shape.complex_state):
            print("--trap applies to the real-state prefill and decode workloads, without --fused "
                  "or --backward", file=sys.stderr)
            sys.exit(2)
        if args.mimo and (args.mimo not in (1, 2, 4, 8) or args.fused or args.backward or args.trap
                          or shape.complex_state):
            print("--mimo R (R in 1, 2, 4, 8) applies to the real-state prefill and decode workloads, "
                  "without --fused, --backward or --trap", file=sys.stderr)
            sys.exit(2)
        if not is_decode and (args.backward or args.fused) and shape.complex_state:
            print("--backward and --fused apply to the real-state workloads", file=sys.stderr)
            sys.exit(2)
    cpus = host_cpus()
    threads = args.cpu_threads or cpus["threads"]
    recs = {}
    for n in names:
        log("workload", n)
        recs[n] = measure(n, variant, args.steps, args.warmup, not args.no_cpu_baseline, threads, cpus,
                          torch, ssm, workloads, args.chunk_len, graph=not args.no_graph,
                          one_call=args.one_call)
    head_name = HEADLINE if HEADLINE in recs else names[0]
    head = recs[head_name]
    io = head["config"]["io"]
    out = {
        "metric": METRIC, "value": head["value"], "unit": "elements/s", "n_gpus": 1,
        "steps": head["steps"], "warmup": head["warmup"], "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": io, "arithmetic": "fp32 state and fp32 arithmetic; inputs and outputs in " + io,
        "data": "synthetic (seeded, resident in HBM before timing)", "config": head["config"],
        "achieved_hbm_GBps_whole_step": head["achieved_hbm_GBps_whole_step"],
        "hbm_frac_whole_step": head["hbm_frac_whole_step"],
        "phases_ms": head["phases_ms"], "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
    }
    if "summary_depends_on_inputs" in head:
        out["summary_depends_on_inputs"] = head["summary_depends_on_inputs"]
    if "mimo_outputs_per_s" in head:
        out["mimo_outputs_per_s"] = head["mimo_outputs_per_s"]
    out["hbm_copy_ceiling"] = copy_ceiling(torch)
    if len(recs) > 1:
        out["workloads"] = {n: {k: v for k, v in r.items() if k not in ("steps", "warmup")}
                            for n, r in recs.items()}
    if not is_variant and not args.workload:
        # The default run also times the 256k prefill's backward (row f2): ssm_scan_bwd,
        # and ssm_scan_bwd_saved from the training forward's stored states (that forward
        # timed apart), each with its roofline record; the oracle's backward as baseline.
        back = {}
        for key, var, cpu in (("ssm_scan_bwd", {"backward": True}, True),
                              ("ssm_scan_bwd_saved", {"backward": True, "saved": True}, False)):
            log("workload", HEADLINE, key)
            r = measure(HEADLINE, var, args.steps, args.warmup, cpu and not args.no_cpu_baseline,
                        threads, cpus, torch, ssm, workloads, args.chunk_len)
            back[key] = {k: v for k, v in r.items() if k not in ("steps", "warmup")}
        out["backward"] = back
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
