"""Seeded synthetic inputs for the selective state-space scan.

This module draws the random tensors that both sides of every comparison consume:
the fp64 oracle (``oracle/``) and the HIP library (``selective_state_space_49_amd``).
It holds the five workload shapes and the value distributions of their inputs and
nothing of the scan's arithmetic. Neither side imports the other; both import this.

Shapes come from the pages: hidden 4096 with expand 2 gives 8192 inner channels and
a 16-wide state (the ``MambaBlock`` defaults and the model config dict of
"【大模型】- Jamba 混合 SSM-Transformer", sections 4.1 "Mamba 层" and 6.3 "长序列性能"),
256k tokens is the context window that "Jamba — SSM-Transformer Híbrido" quotes for
one 80 GB GPU (section "O Problema"), and 28 Mamba layers is its layer count for a
4-block Jamba (section "O bloco Jamba").

Distributions (``N(mu, s)`` means mean mu, standard deviation s):
  x, z ~ N(0, 1);  dt = softplus(N(-1, 0.5));  A = -exp(N(0, 0.5)) per (channel, state);
  B, C ~ N(0, 1) per (batch, step, state);  D ~ N(1, 0.1) per channel.
Complex-state workload: a = exp(N(0, 0.5)), theta ~ U(-pi, pi), A = (-a, theta) as
(re, im); Re/Im of B and C each ~ N(0, 1).

Input stage of the MambaBlock (fused entry points; a generator of its own, seeded
seed + 17, so the draws above do not change): the convolution filter and bias
~ U(-1/sqrt(K), 1/sqrt(K)) per channel (PyTorch's default Conv1d initialisation for a
depthwise filter, fan-in K); dt_bias ~ N(0, 0.1) per channel; the carried conv state
~ N(0, 1); the raw step dt_raw ~ N(-1, 0.5) (so softplus(dt_raw + dt_bias) follows the
dt recipe above). x doubles as the convolution's input. Draw order: conv_w, conv_b,
dt_bias, conv_state0, dt_raw.

Every draw is made in float32 and then rounded to the I/O dtype (round-to-nearest-
even for bfloat16), so both sides read exactly the same bits. The draw order within a
call is fixed: A, D, x, z, dt, B, C. Large tensors are drawn in fixed-size slabs so
that host and device memory stay bounded; the slab size is part of the recipe.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional

import torch

__all__ = [
    "ScanShape", "DecodeShape", "WORKLOADS", "SCAN_WORKLOADS", "io_torch_dtype",
    "make_scan_inputs", "make_decode_params", "make_decode_step", "make_h0",
    "sample_channels", "SLAB_ELEMS", "make_input_stage", "make_decode_input_stage",
    "make_decode_dt_raw", "make_mimo_inputs", "make_mimo_decode_step", "make_trap_weight",
]

# Elements drawn per randn call for big tensors (fixed: part of the seeded recipe).
SLAB_ELEMS = 1 << 27


@dataclass(frozen=True)
class ScanShape:
    """A prefill workload: x, dt, z, y are [batch, L, d_inner]; B, C [batch, L, d_state]."""
    name: str
    batch: int
    L: int
    d_inner: int
    d_state: int
    io: str                  # "f32" or "bf16": dtype of x, dt, z, B, C and y
    complex_state: bool = False
    gated: bool = True       # z present (silu gate) or not
    seed: int = 0

    @property
    def elements(self) -> int:
        """Scan elements (batch * L * d_inner): the unit of the throughput metric."""
        return self.batch * self.L * self.d_inner

    def scaled(self, **kw) -> "ScanShape":
        return replace(self, **kw)


@dataclass(frozen=True)
class DecodeShape:
    """A decode workload: one token per (layer, sequence) per step, state in place."""
    name: str
    n_layers: int
    n_seq: int
    d_inner: int
    d_state: int
    steps: int
    io: str
    gated: bool = True
    complex_state: bool = False
    seed: int = 0

    def scaled(self, **kw) -> "DecodeShape":
        return replace(self, **kw)


WORKLOADS = {
    # Tiny oracle check: batch 1, L=64, 16 channels, N=4, all fp32.
    "tiny_f32": ScanShape("tiny_f32", 1, 64, 16, 4, "f32", seed=1000),
    # Jamba-shaped Mamba layer prefill: batch 2, L=4096, 8192 channels, N=16, bf16 I/O.
    "jamba_layer_prefill": ScanShape("jamba_layer_prefill", 2, 4096, 8192, 16, "bf16", seed=1001),
    # Long-context prefill at the 256k window: batch 1, L=262144, 8192 channels, N=16.
    "long_context_256k": ScanShape("long_context_256k", 1, 262144, 8192, 16, "bf16", seed=1002),
    # Batched decode: 28 layers x 256 sequences x 8192 channels, N=16, 512 steps.
    "batched_decode": DecodeShape("batched_decode", 28, 256, 8192, 16, 512, "bf16", seed=1003),
    # Complex diagonal state: batch 4, L=8192, 4096 channels, N=16 complex, no gate.
    "complex_rotation": ScanShape("complex_rotation", 4, 8192, 4096, 16, "bf16",
                                  complex_state=True, gated=False, seed=1004),
}
SCAN_WORKLOADS = [k for k, v in WORKLOADS.items() if isinstance(v, ScanShape)]


def io_torch_dtype(io: str) -> torch.dtype:
    if io == "f32":
        return torch.float32
    if io == "bf16":
        return torch.bfloat16
    raise ValueError(f"unknown io dtype {io!r}")


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, mean: float, std: float, g, device, out_dtype) -> torch.Tensor:
    """N(mean, std) drawn in float32 slab by slab, rounded to out_dtype."""
    shape = tuple(int(s) for s in shape)
    n = math.prod(shape)
    out = torch.empty(n, dtype=out_dtype, device=device)
    for s0 in range(0, n, SLAB_ELEMS):
        s1 = min(n, s0 + SLAB_ELEMS)
        v = torch.randn(s1 - s0, generator=g, device=device, dtype=torch.float32)
        v.mul_(std).add_(mean)
        out[s0:s1] = v.to(out_dtype)
    return out.view(shape)


def _softplus_normal(shape, mean, std, g, device, out_dtype) -> torch.Tensor:
    """softplus(N(mean, std)) in float32, rounded to out_dtype (the dt recipe)."""
    shape = tuple(int(s) for s in shape)
    n = math.prod(shape)
    out = torch.empty(n, dtype=out_dtype, device=device)
    for s0 in range(0, n, SLAB_ELEMS):
        s1 = min(n, s0 + SLAB_ELEMS)
        v = torch.randn(s1 - s0, generator=g, device=device, dtype=torch.float32)
        v.mul_(std).add_(mean)
        out[s0:s1] = torch.nn.functional.softplus(v).to(out_dtype)
    return out.view(shape)


def _uniform(shape, lo, hi, g, device) -> torch.Tensor:
    v = torch.rand(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return v.mul_(hi - lo).add_(lo)


def make_scan_inputs(shape: ScanShape, device="cpu", seed: Optional[int] = None) -> dict:
    """Draw one prefill workload's inputs.

    Returns a dict with x, dt, z (None when not gated), B, C in the I/O dtype,
    A (float32 [d_inner, d_state], or [d_inner, d_state, 2] as (re, im) for the
    complex state) and D (float32 [d_inner]).
    """
    seed = shape.seed if seed is None else seed
    g = _gen(seed, device)
    io = io_torch_dtype(shape.io)
    b, L, Dn, N = shape.batch, shape.L, shape.d_inner, shape.d_state
    f32 = torch.float32
    if shape.complex_state:
        a = torch.exp(_normal((Dn, N), 0.0, 0.5, g, device, f32))
        theta = _uniform((Dn, N), -math.pi, math.pi, g, device)
        A = torch.stack([-a, theta], dim=-1).contiguous()
    else:
        A = -torch.exp(_normal((Dn, N), 0.0, 0.5, g, device, f32))
    D = _normal((Dn,), 1.0, 0.1, g, device, f32)
    x = _normal((b, L, Dn), 0.0, 1.0, g, device, io)
    z = _normal((b, L, Dn), 0.0, 1.0, g, device, io) if shape.gated else None
    dt = _softplus_normal((b, L, Dn), -1.0, 0.5, g, device, io)
    bc_shape = (b, L, N, 2) if shape.complex_state else (b, L, N)
    B = _normal(bc_shape, 0.0, 1.0, g, device, io)
    C = _normal(bc_shape, 0.0, 1.0, g, device, io)
    return {"x": x, "dt": dt, "z": z, "A": A, "B": B, "C": C, "D": D}


def make_prev_input(batch: int, d_inner: int, d_state: int, io: str = "f32", device="cpu",
                    seed: int = 29) -> dict:
    """The input before step 0 of an exponential-trapezoidal prefill: x_prev [batch,
    d_inner] and B_prev [batch, d_state], ~ N(0, 1) like x and B, in the I/O dtype."""
    g = _gen(seed, device)
    dt = torch.float32 if io == "f32" else torch.bfloat16
    return {"x_prev": _normal((batch, d_inner), 0.0, 1.0, g, device, dt),
            "B_prev": _normal((batch, d_state), 0.0, 1.0, g, device, dt)}


def make_trap_weight(shape, io: str = "f32", device="cpu", kind: str = "random",
                     seed: int = 37) -> torch.Tensor:
    """The weight of each step's current input in the exponential-trapezoidal rule, laid
    out like dt (shape = (batch, L, d_inner), or (n_layers, n_seq, d_inner) for a decode
    token), in the I/O dtype: kind "random" ~ U(0, 1) per element (drawn in float32 slab
    by slab), "half" = 1/2 (the trapezoid rule), "one" = 1 (Euler's step)."""
    shape = tuple(int(v) for v in shape)
    dt = torch.float32 if io == "f32" else torch.bfloat16
    if kind == "half":
        return torch.full(shape, 0.5, dtype=dt, device=device)
    if kind == "one":
        return torch.ones(shape, dtype=dt, device=device)
    if kind != "random":
        raise ValueError(f"unknown weight kind {kind!r}")
    g = _gen(seed, device)
    n = math.prod(shape)
    out = torch.empty(n, dtype=dt, device=device)
    for s0 in range(0, n, SLAB_ELEMS):
        s1 = min(n, s0 + SLAB_ELEMS)
        out[s0:s1] = torch.rand(s1 - s0, generator=g, device=device, dtype=torch.float32).to(dt)
    return out.view(shape)


def make_h0(batch: int, d_inner: int, d_state: int, complex_state=False, device="cpu",
            seed: int = 7) -> torch.Tensor:
    """A non-zero initial state ~ N(0, 1), float32 [batch, d_inner, d_state(, 2)]."""
    g = _gen(seed, device)
    shp = (batch, d_inner, d_state, 2) if complex_state else (batch, d_inner, d_state)
    return _normal(shp, 0.0, 1.0, g, device, torch.float32)


def make_decode_params(shape: DecodeShape, device="cpu", seed: Optional[int] = None) -> dict:
    """Per-layer parameters of a decode workload: A [n_layers, d_inner, d_state(, 2)], D."""
    seed = shape.seed if seed is None else seed
    g = _gen(seed, device)
    Ln, Dn, N = shape.n_layers, shape.d_inner, shape.d_state
    f32 = torch.float32
    if shape.complex_state:
        a = torch.exp(_normal((Ln, Dn, N), 0.0, 0.5, g, device, f32))
        theta = _uniform((Ln, Dn, N), -math.pi, math.pi, g, device)
        A = torch.stack([-a, theta], dim=-1).contiguous()
    else:
        A = -torch.exp(_normal((Ln, Dn, N), 0.0, 0.5, g, device, f32))
    D = _normal((Ln, Dn), 1.0, 0.1, g, device, f32)
    return {"A": A, "D": D}


def make_decode_step(shape: DecodeShape, step: int, device="cpu", seed: Optional[int] = None) -> dict:
    """Fresh single-token inputs for one decode step, for every (layer, sequence).

    x_t, dt_t, z_t: [n_layers, n_seq, d_inner]; B_t, C_t: [n_layers, n_seq, d_state(, 2)].
    Each step has its own generator (seed, step), so any step can be redrawn alone.
    """
    seed = shape.seed if seed is None else seed
    g = _gen(seed * 100003 + 1 + int(step), device)
    io = io_torch_dtype(shape.io)
    Ln, S, Dn, N = shape.n_layers, shape.n_seq, shape.d_inner, shape.d_state
    x = _normal((Ln, S, Dn), 0.0, 1.0, g, device, io)
    z = _normal((Ln, S, Dn), 0.0, 1.0, g, device, io) if shape.gated else None
    dt = _softplus_normal((Ln, S, Dn), -1.0, 0.5, g, device, io)
    bc = (Ln, S, N, 2) if shape.complex_state else (Ln, S, N)
    B = _normal(bc, 0.0, 1.0, g, device, io)
    C = _normal(bc, 0.0, 1.0, g, device, io)
    return {"x": x, "dt": dt, "z": z, "B": B, "C": C}


def sample_channels(n_total: int, k: int, seed: int = 11) -> torch.Tensor:
    """k distinct channel indices out of n_total, sorted, always including both ends."""
    k = min(k, n_total)
    g = _gen(seed, "cpu")
    idx = torch.randperm(n_total, generator=g)[:k]
    idx[0] = 0
    if k > 1:
        idx[1] = n_total - 1
    return torch.unique(idx)


def make_input_stage(shape: ScanShape, K: int, device="cpu", seed: Optional[int] = None,
                     with_state=True) -> dict:
    """Input-stage tensors of a prefill workload for a K-tap filter (K = 0: none):
    conv_w [d_inner, K], conv_b [d_inner], dt_bias [d_inner] (float32),
    conv_state0 [batch, K-1, d_inner] and dt_raw [batch, L, d_inner] (I/O dtype)."""
    seed = (shape.seed if seed is None else seed) + 17
    g = _gen(seed, device)
    io = io_torch_dtype(shape.io)
    b, L, Dn = shape.batch, shape.L, shape.d_inner
    out = {"conv_w": None, "conv_b": None, "conv_state0": None}
    if K > 0:
        bound = 1.0 / math.sqrt(K)
        out["conv_w"] = _uniform((Dn, K), -bound, bound, g, device)
        out["conv_b"] = _uniform((Dn,), -bound, bound, g, device)
    out["dt_bias"] = _normal((Dn,), 0.0, 0.1, g, device, torch.float32)
    if K > 1 and with_state:
        out["conv_state0"] = _normal((b, K - 1, Dn), 0.0, 1.0, g, device, io)
    out["dt_raw"] = _normal((b, L, Dn), -1.0, 0.5, g, device, io)
    return out


def make_decode_input_stage(shape: DecodeShape, K: int, device="cpu",
                            seed: Optional[int] = None) -> dict:
    """Per-layer input-stage parameters of a decode workload: conv_w [n_layers,
    d_inner, K], conv_b and dt_bias [n_layers, d_inner] (float32) and the initial conv
    state [n_layers, n_seq, K-1, d_inner] (I/O dtype)."""
    seed = (shape.seed if seed is None else seed) + 17
    g = _gen(seed, device)
    io = io_torch_dtype(shape.io)
    Ln, S, Dn = shape.n_layers, shape.n_seq, shape.d_inner
    out = {"conv_w": None, "conv_b": None, "conv_state": None}
    if K > 0:
        bound = 1.0 / math.sqrt(K)
        out["conv_w"] = _uniform((Ln, Dn, K), -bound, bound, g, device)
        out["conv_b"] = _uniform((Ln, Dn), -bound, bound, g, device)
    out["dt_bias"] = _normal((Ln, Dn), 0.0, 0.1, g, device, torch.float32)
    if K > 1:
        out["conv_state"] = _normal((Ln, S, K - 1, Dn), 0.0, 1.0, g, device, io)
    return out


def make_decode_dt_raw(shape: DecodeShape, step: int, device="cpu",
                       seed: Optional[int] = None) -> torch.Tensor:
    """The raw step dt_raw ~ N(-1, 0.5) [n_layers, n_seq, d_inner] of one decode step
    (its own generator per step, seeded from (seed + 17, step))."""
    seed = (shape.seed if seed is None else seed) + 17
    g = _gen(seed * 100003 + 1 + int(step), device)
    Ln, S, Dn = shape.n_layers, shape.n_seq, shape.d_inner
    return _normal((Ln, S, Dn), -1.0, 0.5, g, device, io_torch_dtype(shape.io))


def make_mimo_inputs(shape: ScanShape, rank: int, device="cpu", seed: Optional[int] = None) -> dict:
    """A prefill workload with MIMO projections of rank R: the plain scan's recipe with
    x, z ~ N(0, 1) of shape [batch, L, d_inner, R] and B, C ~ N(0, 1) of shape
    [batch, L, d_state, R]; dt ~ softplus(N(-1, 0.5)) [batch, L, d_inner]; A, D as
    make_scan_inputs. Drawn from its own generator (seed + 23)."""
    seed = (shape.seed if seed is None else seed) + 23
    g = _gen(seed, device)
    io = io_torch_dtype(shape.io)
    b, L, Dn, N, R = shape.batch, shape.L, shape.d_inner, shape.d_state, int(rank)
    f32 = torch.float32
    A = -torch.exp(_normal((Dn, N), 0.0, 0.5, g, device, f32))
    D = _normal((Dn,), 1.0, 0.1, g, device, f32)
    x = _normal((b, L, Dn, R), 0.0, 1.0, g, device, io)
    z = _normal((b, L, Dn, R), 0.0, 1.0, g, device, io) if shape.gated else None
    dt = _softplus_normal((b, L, Dn), -1.0, 0.5, g, device, io)
    B = _normal((b, L, N, R), 0.0, 1.0, g, device, io)
    C = _normal((b, L, N, R), 0.0, 1.0, g, device, io)
    return {"x": x, "dt": dt, "z": z, "A": A, "B": B, "C": C, "D": D}


def make_mimo_decode_step(shape: DecodeShape, rank: int, step: int, device="cpu",
                          seed: Optional[int] = None) -> dict:
    """One MIMO decode token for every (layer, sequence): x_t, z_t [n_layers, n_seq,
    d_inner, R]; dt_t [n_layers, n_seq, d_inner]; B_t, C_t [n_layers, n_seq, d_state, R];
    distributions as make_decode_step, its own generator per (seed + 23, step)."""
    seed = (shape.seed if seed is None else seed) + 23
    g = _gen(seed * 100003 + 1 + int(step), device)
    io = io_torch_dtype(shape.io)
    Ln, S, Dn, N, R = shape.n_layers, shape.n_seq, shape.d_inner, shape.d_state, int(rank)
    x = _normal((Ln, S, Dn, R), 0.0, 1.0, g, device, io)
    z = _normal((Ln, S, Dn, R), 0.0, 1.0, g, device, io) if shape.gated else None
    dt = _softplus_normal((Ln, S, Dn), -1.0, 0.5, g, device, io)
    B = _normal((Ln, S, N, R), 0.0, 1.0, g, device, io)
    C = _normal((Ln, S, N, R), 0.0, 1.0, g, device, io)
    return {"x": x, "dt": dt, "z": z, "B": B, "C": C}
