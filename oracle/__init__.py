"""fp64 CPU oracle for the selective state-space scan -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The HIP library never does, and this package
never imports the HIP library: the two share no code. The arithmetic lives in
``ssm_oracle.c`` (plain sequential loops in double precision, built with gcc -O2
-ffp-contract=off); this file only converts inputs to float64 and calls it.

Inputs are torch tensors or numpy arrays in any float dtype. bfloat16 values are
widened to float64 exactly (a bfloat16 is the top 16 bits of a float32). Outputs are
float64 numpy arrays. Layouts are those of ``ssm_oracle.c``.

Page references for what the loops compute are in ``ssm_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_LIB = os.path.join(_HERE, "libssm_oracle.so")
_lock = threading.Lock()
_lib = None

GCC_FLAGS = ["-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-std=c99"]


def build(force: bool = True) -> str:
    """Compile ssm_oracle.c into libssm_oracle.so with the host C compiler."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        i64, dp = ctypes.c_int64, ctypes.c_void_p
        for name in ("oracle_scan_f64", "oracle_scan_c128"):
            f = getattr(lib, name)
            f.argtypes = [i64, i64, i64, i64] + [dp] * 10
            f.restype = ctypes.c_int
        for name in ("oracle_step_f64", "oracle_step_c128"):
            f = getattr(lib, name)
            f.argtypes = [i64, i64, i64, i64] + [dp] * 9
            f.restype = ctypes.c_int
        lib.oracle_state_bytes.argtypes = [i64, i64, i64, i64]
        lib.oracle_state_bytes.restype = i64
        lib.oracle_conv_silu_f64.argtypes = [i64, i64, i64, i64] + [dp] * 6
        lib.oracle_conv_silu_f64.restype = ctypes.c_int
        lib.oracle_softplus_f64.argtypes = [i64, i64, dp, dp, dp]
        lib.oracle_softplus_f64.restype = ctypes.c_int
        lib.oracle_scan_bwd_f64.argtypes = [i64, i64, i64, i64] + [dp] * 18
        lib.oracle_scan_bwd_f64.restype = ctypes.c_int
        lib.oracle_input_stage_bwd_f64.argtypes = [i64, i64, i64, i64] + [dp] * 14
        lib.oracle_input_stage_bwd_f64.restype = ctypes.c_int
        lib.oracle_scan_trap_f64.argtypes = [i64, i64, i64, i64] + [dp] * 13
        lib.oracle_scan_trap_f64.restype = ctypes.c_int
        lib.oracle_step_trap_f64.argtypes = [i64, i64, i64, i64] + [dp] * 12
        lib.oracle_step_trap_f64.restype = ctypes.c_int
        lib.oracle_scan_mimo_f64.argtypes = [i64] * 5 + [dp] * 10
        lib.oracle_scan_mimo_f64.restype = ctypes.c_int
        lib.oracle_step_mimo_f64.argtypes = [i64] * 5 + [dp] * 9
        lib.oracle_step_mimo_f64.restype = ctypes.c_int
        _lib = lib
        return lib


def to_f64(a) -> np.ndarray:
    """Exact widening of a tensor/array to a contiguous float64 numpy array."""
    if a is None:
        return None
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous()
            if a.dtype == torch.bfloat16:
                bits = a.view(torch.int16).numpy().view(np.uint16).astype(np.uint32) << 16
                return bits.view(np.float32).astype(np.float64)
            return a.numpy().astype(np.float64)
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def scan(x, dt, A, B, C, D, z=None, h0=None):
    """Real-state prefill. x, dt, z: [b, L, Dn]; B, C: [b, L, N]; A: [Dn, N]; D: [Dn];
    h0: [b, Dn, N] or None. Returns (y [b, L, Dn], h_final [b, Dn, N]) in float64."""
    x, dt, A, B, C, D, z, h0 = map(to_f64, (x, dt, A, B, C, D, z, h0))
    b, L, Dn = x.shape
    N = A.shape[1]
    _check(dt, (b, L, Dn), "dt"); _check(B, (b, L, N), "B"); _check(C, (b, L, N), "C")
    _check(A, (Dn, N), "A"); _check(D, (Dn,), "D")
    if z is not None: _check(z, (b, L, Dn), "z")
    if h0 is not None: _check(h0, (b, Dn, N), "h0")
    y = np.empty((b, L, Dn)); hf = np.empty((b, Dn, N))
    rc = _load().oracle_scan_f64(b, L, Dn, N, _p(x), _p(dt), _p(A), _p(B), _p(C), _p(D),
                                 _p(z), _p(h0), _p(y), _p(hf))
    if rc != 0:
        raise RuntimeError("oracle_scan_f64 failed")
    return y, hf


def scan_complex(x, dt, A, B, C, D, z=None, h0=None):
    """Complex-state prefill. A: [Dn, N, 2] (re, im); B, C: [b, L, N, 2];
    h0: [b, Dn, N, 2]. Returns (y [b, L, Dn], h_final [b, Dn, N, 2])."""
    x, dt, A, B, C, D, z, h0 = map(to_f64, (x, dt, A, B, C, D, z, h0))
    b, L, Dn = x.shape
    N = A.shape[1]
    _check(dt, (b, L, Dn), "dt"); _check(B, (b, L, N, 2), "B"); _check(C, (b, L, N, 2), "C")
    _check(A, (Dn, N, 2), "A"); _check(D, (Dn,), "D")
    if z is not None: _check(z, (b, L, Dn), "z")
    if h0 is not None: _check(h0, (b, Dn, N, 2), "h0")
    y = np.empty((b, L, Dn)); hf = np.empty((b, Dn, N, 2))
    rc = _load().oracle_scan_c128(b, L, Dn, N, _p(x), _p(dt), _p(A), _p(B), _p(C), _p(D),
                                  _p(z), _p(h0), _p(y), _p(hf))
    if rc != 0:
        raise RuntimeError("oracle_scan_c128 failed")
    return y, hf


def step(h, x, dt, A, B, C, D, z=None):
    """One decode token. h: [Ln, S, Dn, N]; x, dt, z: [Ln, S, Dn]; B, C: [Ln, S, N];
    A: [Ln, Dn, N]; D: [Ln, Dn]. Returns (y [Ln, S, Dn], h_new) without touching h."""
    h = to_f64(h).copy()
    x, dt, A, B, C, D, z = map(to_f64, (x, dt, A, B, C, D, z))
    Ln, S, Dn = x.shape
    N = h.shape[-1]
    _check(h, (Ln, S, Dn, N), "h"); _check(B, (Ln, S, N), "B"); _check(C, (Ln, S, N), "C")
    _check(A, (Ln, Dn, N), "A"); _check(D, (Ln, Dn), "D"); _check(dt, (Ln, S, Dn), "dt")
    if z is not None: _check(z, (Ln, S, Dn), "z")
    y = np.empty((Ln, S, Dn))
    rc = _load().oracle_step_f64(Ln, S, Dn, N, _p(h), _p(x), _p(dt), _p(A), _p(B), _p(C),
                                 _p(D), _p(z), _p(y))
    if rc != 0:
        raise RuntimeError("oracle_step_f64 failed")
    return y, h


def step_complex(h, x, dt, A, B, C, D, z=None):
    """Complex decode token. h: [Ln, S, Dn, N, 2]; A: [Ln, Dn, N, 2]; B, C: [Ln, S, N, 2]."""
    h = to_f64(h).copy()
    x, dt, A, B, C, D, z = map(to_f64, (x, dt, A, B, C, D, z))
    Ln, S, Dn = x.shape
    N = h.shape[-2]
    _check(h, (Ln, S, Dn, N, 2), "h"); _check(B, (Ln, S, N, 2), "B")
    _check(C, (Ln, S, N, 2), "C"); _check(A, (Ln, Dn, N, 2), "A"); _check(D, (Ln, Dn), "D")
    y = np.empty((Ln, S, Dn))
    rc = _load().oracle_step_c128(Ln, S, Dn, N, _p(h), _p(x), _p(dt), _p(A), _p(B), _p(C),
                                  _p(D), _p(z), _p(y))
    if rc != 0:
        raise RuntimeError("oracle_step_c128 failed")
    return y, h


def state_bytes(n_layers: int, channels: int, d_state: int, bytes_per_value: int) -> int:
    """Size of a fixed-size SSM state in bytes (independent of sequence length)."""
    return int(_load().oracle_state_bytes(n_layers, channels, d_state, bytes_per_value))


def scan_bwd(x, dt, A, B, C, D, z=None, h0=None, dy=None, dh_final=None):
    """Gradients of sum(dy * y) + sum(dh_final * h_final) of the real-state prefill.
    Returns a dict with dx, ddt, dz (None when ungated) [b, L, Dn]; dA [Dn, N];
    dB, dC [b, L, N]; dD [Dn]; dh0 [b, Dn, N]."""
    x, dt, A, B, C, D, z, h0, dy, dh_final = map(to_f64, (x, dt, A, B, C, D, z, h0, dy, dh_final))
    b, L, Dn = x.shape
    N = A.shape[1]
    _check(dt, (b, L, Dn), "dt"); _check(B, (b, L, N), "B"); _check(C, (b, L, N), "C")
    _check(A, (Dn, N), "A"); _check(D, (Dn,), "D"); _check(dy, (b, L, Dn), "dy")
    if z is not None: _check(z, (b, L, Dn), "z")
    if h0 is not None: _check(h0, (b, Dn, N), "h0")
    if dh_final is not None: _check(dh_final, (b, Dn, N), "dh_final")
    g = {k: np.empty(shp) for k, shp in [("dx", (b, L, Dn)), ("ddt", (b, L, Dn)), ("dA", (Dn, N)),
                                         ("dB", (b, L, N)), ("dC", (b, L, N)), ("dD", (Dn,)),
                                         ("dh0", (b, Dn, N))]}
    g["dz"] = np.empty((b, L, Dn)) if z is not None else None
    rc = _load().oracle_scan_bwd_f64(b, L, Dn, N, _p(x), _p(dt), _p(A), _p(B), _p(C), _p(D), _p(z),
                                     _p(h0), _p(dy), _p(dh_final), _p(g["dx"]), _p(g["ddt"]),
                                     _p(g["dA"]), _p(g["dB"]), _p(g["dC"]), _p(g["dD"]), _p(g["dz"]),
                                     _p(g["dh0"]))
    if rc != 0:
        raise RuntimeError("oracle_scan_bwd_f64 failed")
    return g


def conv_silu(x, w, cb=None, state0=None):
    """Causal depthwise convolution over time, then silu (the MambaBlock's input stage).
    x: [b, L, Dn]; w: [Dn, K]; cb: [Dn] or None; state0: [b, K-1, Dn] or None (zeros).
    Returns (u [b, L, Dn], state_out [b, K-1, Dn] = the last K-1 inputs)."""
    x, w, cb, state0 = map(to_f64, (x, w, cb, state0))
    b, L, Dn = x.shape
    K = w.shape[1]
    _check(w, (Dn, K), "conv_w")
    if cb is not None: _check(cb, (Dn,), "conv_b")
    if state0 is not None: _check(state0, (b, K - 1, Dn), "conv_state0")
    u = np.empty((b, L, Dn)); so = np.empty((b, K - 1, Dn))
    if _load().oracle_conv_silu_f64(b, L, Dn, K, _p(x), _p(w), _p(cb), _p(state0), _p(u), _p(so)) != 0:
        raise RuntimeError("oracle_conv_silu_f64 failed")
    return u, so


def softplus(raw, bias=None):
    """softplus(raw + bias) with bias [Dn] broadcast over the leading dimensions."""
    raw, bias = to_f64(raw), to_f64(bias)
    Dn = raw.shape[-1]
    if bias is not None: _check(bias, (Dn,), "dt_bias")
    out = np.empty(raw.shape)
    rows = raw.size // Dn if Dn else 0
    if _load().oracle_softplus_f64(rows, Dn, _p(raw), _p(bias), _p(out)) != 0:
        raise RuntimeError("oracle_softplus_f64 failed")
    return out


def scan_fused(x_in, dt_raw, A, B, C, D, z=None, h0=None, conv_w=None, conv_b=None,
               conv_state0=None, dt_bias=None):
    """The MambaBlock's input stage followed by the real-state scan:
    u = silu(causal conv(x_in)), dt = softplus(dt_raw + dt_bias), then scan(u, dt, ...).
    Returns (y, h_final, conv_state_out)."""
    u, so = conv_silu(x_in, conv_w, conv_b, conv_state0)
    y, hf = scan(u, softplus(dt_raw, dt_bias), A, B, C, D, z, h0)
    return y, hf, so


def input_stage_bwd(x_in, dt_raw, du, ddt, conv_w=None, conv_b=None, conv_state0=None,
                    dt_bias=None, want_dstate0=True):
    """Gradients through the input stage (oracle_input_stage_bwd_f64): given du =
    dLoss/du and ddt = dLoss/ddt for u = silu(conv(x_in)), dt = softplus(dt_raw + bias),
    returns a dict dx_in, ddt_raw [b, L, Dn]; dconv_w [Dn, K], dconv_b, ddt_bias [Dn]
    (None without conv_w, conv_b, dt_bias); dconv_state0 [b, K-1, Dn] (None for K < 2
    or when not wanted). conv_w None: no convolution (u = x_in)."""
    x_in, dt_raw, du, ddt, w, cb, s0, bias = map(
        to_f64, (x_in, dt_raw, du, ddt, conv_w, conv_b, conv_state0, dt_bias))
    b, L, Dn = x_in.shape
    K = 0 if w is None else w.shape[1]
    if w is not None: _check(w, (Dn, K), "conv_w")
    if cb is not None: _check(cb, (Dn,), "conv_b")
    if s0 is not None: _check(s0, (b, K - 1, Dn), "conv_state0")
    if bias is not None: _check(bias, (Dn,), "dt_bias")
    out = {"dx_in": np.empty((b, L, Dn)), "ddt_raw": np.empty((b, L, Dn)),
           "dconv_w": np.empty((Dn, K)) if K else None,
           "dconv_b": np.empty(Dn) if (K and cb is not None) else None,
           "ddt_bias": np.empty(Dn) if bias is not None else None,
           "dconv_state0": np.empty((b, K - 1, Dn)) if (K > 1 and want_dstate0) else None}
    if _load().oracle_input_stage_bwd_f64(
            b, L, Dn, K, _p(x_in), _p(dt_raw), _p(w), _p(cb), _p(s0), _p(bias), _p(du), _p(ddt),
            _p(out["dx_in"]), _p(out["ddt_raw"]), _p(out["dconv_w"]), _p(out["dconv_b"]),
            _p(out["ddt_bias"]), _p(out["dconv_state0"])) != 0:
        raise RuntimeError("oracle_input_stage_bwd_f64 failed")
    return out


def scan_fused_bwd(x_in, dt_raw, A, B, C, D, z=None, h0=None, conv_w=None, conv_b=None,
                   conv_state0=None, dt_bias=None, dy=None, dh_final=None):
    """Gradients of sum(dy y) + sum(dh_final h_final) for scan_fused: the scan's
    backward (scan_bwd) on u = silu(conv(x_in)) and dt = softplus(dt_raw + bias), then
    input_stage_bwd. conv_w None: no convolution (u = x_in). Returns scan_bwd's dict
    without dx, ddt, plus input_stage_bwd's entries."""
    u = x_in if conv_w is None else conv_silu(x_in, conv_w, conv_b, conv_state0)[0]
    dt = softplus(dt_raw, dt_bias)
    g = scan_bwd(u, dt, A, B, C, D, z, h0, dy=dy, dh_final=dh_final)
    out = input_stage_bwd(x_in, dt_raw, g.pop("dx"), g.pop("ddt"), conv_w, conv_b, conv_state0,
                          dt_bias)
    out.update(g)
    return out


def step_fused(h, conv_state, x_in, dt_raw, A, B, C, D, z=None, conv_w=None, conv_b=None,
               dt_bias=None):
    """One decode token through the input stage and the scan, per layer:
    conv_state [Ln, S, K-1, Dn]; conv_w [Ln, Dn, K]; conv_b, dt_bias [Ln, Dn] or None.
    Returns (y, h_new, conv_state_new) without touching the inputs."""
    x_in, dt_raw, conv_state, conv_w, conv_b, dt_bias = map(
        to_f64, (x_in, dt_raw, conv_state, conv_w, conv_b, dt_bias))
    Ln, S, Dn = x_in.shape
    K = conv_w.shape[2]
    _check(conv_w, (Ln, Dn, K), "conv_w"); _check(conv_state, (Ln, S, K - 1, Dn), "conv_state")
    u = np.empty((Ln, S, Dn)); dt = np.empty((Ln, S, Dn)); cs = np.empty((Ln, S, K - 1, Dn))
    for l in range(Ln):
        ul, cs[l] = conv_silu(x_in[l][:, None, :], conv_w[l], None if conv_b is None else conv_b[l],
                              conv_state[l])
        u[l] = ul[:, 0, :]
        dt[l] = softplus(dt_raw[l], None if dt_bias is None else dt_bias[l])
    y, hn = step(h, u, dt, A, B, C, D, z)
    return y, hn, cs


def scan_threaded(x, dt, A, B, C, D, z=None, h0=None, threads: int = 1, complex_state=False):
    """The same oracle loop run on disjoint channel subsets from `threads` threads.

    Channels are independent, so this computes exactly what ``scan`` computes; it is
    how the benchmark times the oracle on several host cores (ctypes releases the GIL).
    """
    x, dt, A, B, C, D, z, h0 = map(to_f64, (x, dt, A, B, C, D, z, h0))
    Dn = x.shape[2]
    parts = [p for p in np.array_split(np.arange(Dn), max(1, threads)) if len(p)]
    fn = scan_complex if complex_state else scan
    results = [None] * len(parts)

    def work(k, idx):
        sub = lambda a: None if a is None else np.ascontiguousarray(a[:, :, idx])
        results[k] = fn(sub(x), sub(dt), A[idx], B, C, D[idx], sub(z),
                        None if h0 is None else np.ascontiguousarray(h0[:, idx]))

    ts = [threading.Thread(target=work, args=(k, idx)) for k, idx in enumerate(parts)]
    for t in ts: t.start()
    for t in ts: t.join()
    y = np.concatenate([r[0] for r in results], axis=2)
    hf = np.concatenate([r[1] for r in results], axis=1)
    return y, hf


def _check(a, shape, name):
    if tuple(a.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(a.shape)}")


def scan_trap(x, dt, A, B, C, D, z=None, h0=None, x_prev=None, B_prev=None, lam=None):
    """Real-state prefill with the exponential-trapezoidal discretisation. As scan(),
    plus the input before step 0: x_prev [b, Dn] and B_prev [b, N] (None: zero), and
    the weight of each step's current input lam [b, L, Dn] (None: 1/2, the trapezoid
    rule; 1 is Euler's step). Returns (y [b, L, Dn], h_final [b, Dn, N])."""
    x, dt, A, B, C, D, z, h0, x_prev, B_prev, lam = map(
        to_f64, (x, dt, A, B, C, D, z, h0, x_prev, B_prev, lam))
    b, L, Dn = x.shape
    N = A.shape[1]
    _check(dt, (b, L, Dn), "dt"); _check(B, (b, L, N), "B"); _check(C, (b, L, N), "C")
    _check(A, (Dn, N), "A"); _check(D, (Dn,), "D")
    if z is not None: _check(z, (b, L, Dn), "z")
    if h0 is not None: _check(h0, (b, Dn, N), "h0")
    if x_prev is not None: _check(x_prev, (b, Dn), "x_prev")
    if B_prev is not None: _check(B_prev, (b, N), "B_prev")
    if lam is not None: _check(lam, (b, L, Dn), "lam")
    y = np.empty((b, L, Dn)); hf = np.empty((b, Dn, N))
    rc = _load().oracle_scan_trap_f64(b, L, Dn, N, _p(x), _p(dt), _p(A), _p(B), _p(C), _p(D),
                                      _p(z), _p(h0), _p(x_prev), _p(B_prev), _p(lam), _p(y), _p(hf))
    if rc != 0:
        raise RuntimeError("oracle_scan_trap_f64 failed")
    return y, hf


def step_trap(h, x_prev, B_prev, x, dt, A, B, C, D, z=None, lam=None):
    """One exponential-trapezoidal decode token. h: [Ln, S, Dn, N]; x_prev, x, dt, z,
    lam: [Ln, S, Dn]; B_prev, B, C: [Ln, S, N]; A: [Ln, Dn, N]; D: [Ln, Dn]. x_prev and
    B_prev are the previous token's x and B (None: no previous input); lam the weight
    of the current input (None: 1/2). Returns (y [Ln, S, Dn], h_new) without touching h."""
    h = to_f64(h).copy()
    x_prev, B_prev, x, dt, A, B, C, D, z, lam = map(to_f64, (x_prev, B_prev, x, dt, A, B, C, D, z, lam))
    Ln, S, Dn = x.shape
    N = h.shape[-1]
    _check(h, (Ln, S, Dn, N), "h"); _check(B, (Ln, S, N), "B"); _check(C, (Ln, S, N), "C")
    _check(A, (Ln, Dn, N), "A"); _check(D, (Ln, Dn), "D"); _check(dt, (Ln, S, Dn), "dt")
    if z is not None: _check(z, (Ln, S, Dn), "z")
    if x_prev is not None: _check(x_prev, (Ln, S, Dn), "x_prev")
    if B_prev is not None: _check(B_prev, (Ln, S, N), "B_prev")
    if lam is not None: _check(lam, (Ln, S, Dn), "lam")
    y = np.empty((Ln, S, Dn))
    rc = _load().oracle_step_trap_f64(Ln, S, Dn, N, _p(h), _p(x_prev), _p(B_prev), _p(x), _p(dt),
                                      _p(lam), _p(A), _p(B), _p(C), _p(D), _p(z), _p(y))
    if rc != 0:
        raise RuntimeError("oracle_step_trap_f64 failed")
    return y, h


def scan_mimo(x, dt, A, B, C, D, z=None, h0=None):
    """Real-state prefill with MIMO projections of rank R. x, z: [b, L, Dn, R];
    dt: [b, L, Dn]; B, C: [b, L, N, R]; A: [Dn, N]; D: [Dn]; h0: [b, Dn, N] or None.
    Returns (y [b, L, Dn, R], h_final [b, Dn, N])."""
    x, dt, A, B, C, D, z, h0 = map(to_f64, (x, dt, A, B, C, D, z, h0))
    b, L, Dn, R = x.shape
    N = A.shape[1]
    _check(dt, (b, L, Dn), "dt"); _check(B, (b, L, N, R), "B"); _check(C, (b, L, N, R), "C")
    _check(A, (Dn, N), "A"); _check(D, (Dn,), "D")
    if z is not None: _check(z, (b, L, Dn, R), "z")
    if h0 is not None: _check(h0, (b, Dn, N), "h0")
    y = np.empty((b, L, Dn, R)); hf = np.empty((b, Dn, N))
    rc = _load().oracle_scan_mimo_f64(b, L, Dn, N, R, _p(x), _p(dt), _p(A), _p(B), _p(C), _p(D),
                                      _p(z), _p(h0), _p(y), _p(hf))
    if rc != 0:
        raise RuntimeError("oracle_scan_mimo_f64 failed")
    return y, hf


def step_mimo(h, x, dt, A, B, C, D, z=None):
    """One MIMO decode token. h: [Ln, S, Dn, N]; x, z: [Ln, S, Dn, R]; dt: [Ln, S, Dn];
    B, C: [Ln, S, N, R]; A: [Ln, Dn, N]; D: [Ln, Dn]. Returns (y [Ln, S, Dn, R], h_new)
    without touching h."""
    h = to_f64(h).copy()
    x, dt, A, B, C, D, z = map(to_f64, (x, dt, A, B, C, D, z))
    Ln, S, Dn, R = x.shape
    N = h.shape[-1]
    _check(h, (Ln, S, Dn, N), "h"); _check(B, (Ln, S, N, R), "B"); _check(C, (Ln, S, N, R), "C")
    _check(A, (Ln, Dn, N), "A"); _check(D, (Ln, Dn), "D"); _check(dt, (Ln, S, Dn), "dt")
    if z is not None: _check(z, (Ln, S, Dn, R), "z")
    y = np.empty((Ln, S, Dn, R))
    rc = _load().oracle_step_mimo_f64(Ln, S, Dn, N, R, _p(h), _p(x), _p(dt), _p(A), _p(B), _p(C),
                                      _p(D), _p(z), _p(y))
    if rc != 0:
        raise RuntimeError("oracle_step_mimo_f64 failed")
    return y, h
