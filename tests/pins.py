"""Pins for the fp64 oracle: checks against definitions that do not share its code.

Each ``pin_*`` function takes the oracle module (or a stand-in with the same
functions) and raises AssertionError when the oracle disagrees with something the
pages or plain mathematics fix:

  brute force   the state written out as an explicit selective convolution,
                y_t = sum_{s<=t} sum_n C_t[n] exp(A_n (S_t - S_s)) dt_s B_s[n] x_s
                      + sum_n C_t[n] exp(A_n S_t) h0[n] + D x_t, then the gate,
                with S_t the running sum of dt. It uses exp of a sum of dt where
                the recurrence multiplies exps, so the two are independent.
  convolution   the time-invariant case (constant dt, B, C) must equal a causal
                convolution with kernel K_k = sum_n C_n exp(k dt A_n) dt B_n; the
                pages tie the structured SSM of S4 to a long convolution
                ("Jamba — SSM-Transformer Híbrido", section "Um SSM em uma página").
  closed forms  a geometric series (one state, constant inputs); dt = 0 keeps the
                state fixed; the complex state with no decay is a pure rotation
                e^{i theta t} (the data-dependent rotary embedding of the Mamba-3
                item on complex-valued state updates, same page).
  invariants    linearity in x; splitting a sequence and resuming from h_final
                (the state is all that carries over); L decode steps equal one
                prefill; a NaN stays inside its channel; the complex variant with
                theta = 0 equals the real one.
  printed value the fixed-size state arithmetic of the memory-budget section
                (tests/golden/state_memory.json).
  backward      central finite differences of sum(dy y) + sum(dh_final h_final)
                through the forward oracle, for every element of every input, against
                the backward oracle's gradients.
  trapezoid     the exponential-trapezoidal discretisation (the reading of the
                Mamba-3 item on the same page, and of the key-terms rows that say it
                subsumes Euler's): each step's two input taps, weighted lam and 1 - lam,
                written out as a sum with exp of summed dt, for the default weight 1/2
                and for random weights; weight 1 is the Euler scan and its decode step;
                with A = 0 and weight 1/2 the state is exactly numpy's trapezoid rule
                over the samples B x on the time grid; against the closed-form solution
                of the continuous ODE the error falls about 4x per halved step at
                weight 1/2 (second order) and 2x at weight 1, as Euler's does;
                split/resume with the previous input passed on, and L decode steps,
                bit for bit, with random weights.
  MIMO          the reading of Mamba-3's matrix-valued projections (B_t, C_t of size
                N x R, R inputs and outputs per channel): rank 1 is the scan above
                bit for bit; with no skip, gate or initial state each output is the
                sum over inputs of rank-1 scans (superposition, since the state is
                linear in the input); the explicit convolution with exp of summed dt;
                split/resume and L decode steps bit for bit.
  input stage   the MambaBlock's causal depthwise convolution against numpy's
                np.convolve (a true convolution, so the taps go in reversed) and an
                impulse response; the carried conv state against the plain
                concatenation of two calls' inputs; softplus against numpy's
                logaddexp(0, v) and its identities softplus(v) - softplus(-v) = v,
                softplus(0) = log 2; the fused scan with an identity filter and an
                inverse-softplus step against the plain scan of silu(x); L fused
                decode steps against one fused prefill.

The pins draw their own inputs with numpy; they test only the oracle.
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def silu(z):
    return z / (1.0 + np.exp(-z))


def tiny_real(seed, b=2, L=24, Dn=3, N=4, gated=True, with_h0=True):
    r = np.random.default_rng(seed)
    x = r.normal(0, 1, (b, L, Dn))
    z = r.normal(0, 1, (b, L, Dn)) if gated else None
    dt = np.log1p(np.exp(r.normal(-1, 0.5, (b, L, Dn))))
    A = -np.exp(r.normal(0, 0.5, (Dn, N)))
    B = r.normal(0, 1, (b, L, N))
    C = r.normal(0, 1, (b, L, N))
    D = r.normal(1, 0.1, Dn)
    h0 = r.normal(0, 1, (b, Dn, N)) if with_h0 else None
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=D, z=z, h0=h0)


def tiny_complex(seed, b=2, L=20, Dn=3, N=4, gated=False, with_h0=True):
    r = np.random.default_rng(seed)
    x = r.normal(0, 1, (b, L, Dn))
    z = r.normal(0, 1, (b, L, Dn)) if gated else None
    dt = np.log1p(np.exp(r.normal(-1, 0.5, (b, L, Dn))))
    A = np.stack([-np.exp(r.normal(0, 0.5, (Dn, N))), r.uniform(-np.pi, np.pi, (Dn, N))], -1)
    B = r.normal(0, 1, (b, L, N, 2))
    C = r.normal(0, 1, (b, L, N, 2))
    D = r.normal(1, 0.1, Dn)
    h0 = r.normal(0, 1, (b, Dn, N, 2)) if with_h0 else None
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=D, z=z, h0=h0)


def brute_real(x, dt, A, B, C, D, z=None, h0=None):
    """O(L^2 N) explicit selective convolution (see the module docstring)."""
    b, L, Dn = x.shape
    N = A.shape[1]
    S = np.cumsum(dt, axis=1)
    y = np.zeros((b, L, Dn))
    hf = np.zeros((b, Dn, N))
    for bi in range(b):
        for d in range(Dn):
            for t in range(L):
                w = np.exp(np.outer(S[bi, t, d] - S[bi, :t + 1, d], A[d]))          # [t+1, N]
                h_t = (w * (dt[bi, :t + 1, d] * x[bi, :t + 1, d])[:, None] * B[bi, :t + 1]).sum(0)
                if h0 is not None:
                    h_t = h_t + np.exp(A[d] * S[bi, t, d]) * h0[bi, d]
                yv = float(C[bi, t] @ h_t) + D[d] * x[bi, t, d]
                if z is not None:
                    yv *= silu(z[bi, t, d])
                y[bi, t, d] = yv
                if t == L - 1:
                    hf[bi, d] = h_t
    return y, hf


def brute_complex(x, dt, A, B, C, D, z=None, h0=None):
    """Complex-state explicit convolution in complex128 arithmetic."""
    b, L, Dn = x.shape
    N = A.shape[1]
    Ac = A[..., 0] + 1j * A[..., 1]
    Bc = B[..., 0] + 1j * B[..., 1]
    Cc = C[..., 0] + 1j * C[..., 1]
    H0 = None if h0 is None else h0[..., 0] + 1j * h0[..., 1]
    S = np.cumsum(dt, axis=1)
    y = np.zeros((b, L, Dn))
    hf = np.zeros((b, Dn, N, 2))
    for bi in range(b):
        for d in range(Dn):
            for t in range(L):
                w = np.exp(np.outer(S[bi, t, d] - S[bi, :t + 1, d], Ac[d]))
                h_t = (w * (dt[bi, :t + 1, d] * x[bi, :t + 1, d])[:, None] * Bc[bi, :t + 1]).sum(0)
                if H0 is not None:
                    h_t = h_t + np.exp(Ac[d] * S[bi, t, d]) * H0[bi, d]
                yv = float(np.real(Cc[bi, t] @ h_t)) + D[d] * x[bi, t, d]
                if z is not None:
                    yv *= silu(z[bi, t, d])
                y[bi, t, d] = yv
                if t == L - 1:
                    hf[bi, d, :, 0] = h_t.real
                    hf[bi, d, :, 1] = h_t.imag
    return y, hf


def _rel(a, b):
    a = np.asarray(a); b = np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _bitwise(a, b):
    return np.array_equal(np.asarray(a).view(np.uint64), np.asarray(b).view(np.uint64))


# ----------------------------------------------------------------------------- pins

def pin_brute_force(O, tol=1e-12):
    for seed, kw in [(1, {}), (2, dict(gated=False, with_h0=False)), (3, dict(b=1, L=64, Dn=2, N=4))]:
        inp = tiny_real(seed, **kw)
        y, hf = O.scan(**inp)
        yb, hb = brute_real(**inp)
        assert _rel(y, yb) <= tol, f"brute force y mismatch {_rel(y, yb)} (seed {seed})"
        assert _rel(hf, hb) <= tol, f"brute force h_final mismatch {_rel(hf, hb)} (seed {seed})"


def pin_convolution(O, tol=1e-12):
    r = np.random.default_rng(5)
    L, Dn, N = 48, 3, 4
    dtc = 0.37
    Bc, Cc = r.normal(0, 1, N), r.normal(0, 1, N)
    A = -np.exp(r.normal(0, 0.5, (Dn, N)))
    D = r.normal(1, 0.1, Dn)
    x = r.normal(0, 1, (1, L, Dn))
    y, _ = O.scan(x, np.full((1, L, Dn), dtc), A, np.tile(Bc, (1, L, 1)), np.tile(Cc, (1, L, 1)), D)
    for d in range(Dn):
        k = np.arange(L)[:, None]
        K = (Cc * np.exp(k * dtc * A[d]) * dtc * Bc).sum(1)
        ref = np.convolve(x[0, :, d], K)[:L] + D[d] * x[0, :, d]
        assert _rel(y[0, :, d], ref) <= tol, f"time-invariant case is not the convolution (d={d})"


def pin_geometric_series(O, tol=1e-12):
    L, a, dtc, b_, c_, d_, xv = 40, -0.8, 0.25, 1.3, -0.7, 0.9, 0.6
    y, hf = O.scan(np.full((1, L, 1), xv), np.full((1, L, 1), dtc), np.array([[a]]),
                   np.full((1, L, 1), b_), np.full((1, L, 1), c_), np.array([d_]))
    rr = np.exp(dtc * a)
    t = np.arange(L)
    ref = c_ * dtc * b_ * xv * (1 - rr ** (t + 1)) / (1 - rr) + d_ * xv
    assert _rel(y[0, :, 0], ref) <= tol, "geometric-series closed form"
    assert _rel(hf[0, 0, 0], dtc * b_ * xv * (1 - rr ** L) / (1 - rr)) <= tol, "closed-form final state"


def pin_dt_zero(O):
    inp = tiny_real(7, with_h0=False)
    inp["dt"] = np.zeros_like(inp["dt"])
    y, hf = O.scan(**inp)
    assert np.all(hf == 0.0), "dt = 0 must keep a zero state at exactly zero"
    ref = inp["D"] * inp["x"] * silu(inp["z"])
    assert _rel(y, ref) <= 1e-15, "dt = 0: y must be D*x*silu(z)"
    inp = tiny_real(8)
    inp["dt"] = np.zeros_like(inp["dt"])
    y, hf = O.scan(**inp)
    assert _bitwise(hf, inp["h0"]), "dt = 0 must keep h0 unchanged"
    ref = (np.einsum("bln,bdn->bld", inp["C"], inp["h0"]) + inp["D"] * inp["x"]) * silu(inp["z"])
    assert _rel(y, ref) <= 1e-13, "dt = 0: y must be (C.h0 + D*x)*silu(z)"


def pin_linearity(O, tol=1e-12):
    i1, i2 = tiny_real(11, gated=False, with_h0=False), tiny_real(12, gated=False, with_h0=False)
    al, be = 0.7, -1.9
    base = {k: i1[k] for k in ("dt", "A", "B", "C", "D")}
    y1, h1 = O.scan(i1["x"], **base)
    y2, h2 = O.scan(i2["x"], **base)
    y3, h3 = O.scan(al * i1["x"] + be * i2["x"], **base)
    assert _rel(y3, al * y1 + be * y2) <= tol, "linearity in x (y)"
    assert _rel(h3, al * h1 + be * h2) <= tol, "linearity in x (h)"


def _slice_t(inp, t0, t1):
    out = dict(inp)
    for k in ("x", "dt", "z", "B", "C"):
        if out.get(k) is not None:
            out[k] = np.ascontiguousarray(inp[k][:, t0:t1])
    return out


def pin_split_resume(O, complex_state=False):
    inp = tiny_complex(13) if complex_state else tiny_real(13, L=30)
    fn = O.scan_complex if complex_state else O.scan
    L = inp["x"].shape[1]
    y, hf = fn(**inp)
    for L1 in (1, 11, L - 1):
        a = _slice_t(inp, 0, L1)
        ya, ha = fn(**a)
        bpart = _slice_t(inp, L1, L)
        bpart["h0"] = ha
        yb, hb = fn(**bpart)
        assert _bitwise(np.concatenate([ya, yb], 1), y), f"split at {L1}: y differs"
        assert _bitwise(hb, hf), f"split at {L1}: h_final differs"


def pin_step_equals_scan(O, complex_state=False):
    inp = tiny_complex(17) if complex_state else tiny_real(17, L=16)
    if complex_state:
        inp["z"] = np.random.default_rng(3).normal(0, 1, inp["x"].shape)
    fn, st = (O.scan_complex, O.step_complex) if complex_state else (O.scan, O.step)
    y, hf = fn(**inp)
    h = inp["h0"][None].copy()
    b, L, Dn = inp["x"].shape
    for t in range(L):
        yt, h = st(h, inp["x"][None, :, t], inp["dt"][None, :, t], inp["A"][None],
                   inp["B"][None, :, t], inp["C"][None, :, t], inp["D"][None],
                   None if inp["z"] is None else inp["z"][None, :, t])
        assert _bitwise(yt[0], y[:, t]), f"decode step {t} differs from prefill"
    assert _bitwise(h[0], hf), "state after L decode steps differs from prefill h_final"


def pin_layers_are_independent(O, complex_state=False):
    """A step over several layers equals one single-layer step per layer, each with
    that layer's own A and D (single-layer steps are pinned to prefill above)."""
    r = np.random.default_rng(37)
    Ln, S, Dn, N = 3, 2, 4, 4
    ext = (2,) if complex_state else ()
    st = O.step_complex if complex_state else O.step
    h = r.normal(0, 1, (Ln, S, Dn, N) + ext)
    x, z = r.normal(0, 1, (Ln, S, Dn)), r.normal(0, 1, (Ln, S, Dn))
    dt = np.log1p(np.exp(r.normal(-1, 0.5, (Ln, S, Dn))))
    if complex_state:
        A = np.stack([-np.exp(r.normal(0, 0.5, (Ln, Dn, N))), r.uniform(-3, 3, (Ln, Dn, N))], -1)
    else:
        A = -np.exp(r.normal(0, 0.5, (Ln, Dn, N)))
    B, C = r.normal(0, 1, (Ln, S, N) + ext), r.normal(0, 1, (Ln, S, N) + ext)
    D = r.normal(1, 0.1, (Ln, Dn))
    y, h2 = st(h, x, dt, A, B, C, D, z)
    for l in range(Ln):
        sl = slice(l, l + 1)
        yl, hl = st(h[sl], x[sl], dt[sl], A[sl], B[sl], C[sl], D[sl], z[sl])
        assert _bitwise(yl, y[sl]) and _bitwise(hl, h2[sl]), f"layer {l} is not independent"


def pin_isolation(O):
    inp = tiny_real(19)
    y, hf = O.scan(**inp)
    bad = dict(inp)
    bad["x"] = inp["x"].copy()
    bad["x"][0, 5, 1] = np.nan
    y2, h2 = O.scan(**bad)
    other = [d for d in range(inp["x"].shape[2]) if d != 1]
    assert _bitwise(y2[:, :, other], y[:, :, other]), "NaN leaked into other channels (y)"
    assert _bitwise(y2[1], y[1]), "NaN leaked into the other batch row"
    assert _bitwise(h2[:, other], hf[:, other]), "NaN leaked into other channels (h)"
    assert np.all(np.isnan(y2[0, 5:, 1])) and np.all(np.isfinite(y2[0, :5, 1])), "NaN not confined in time"


def pin_state_bytes(O):
    with open(os.path.join(GOLDEN, "state_memory.json")) as f:
        g = json.load(f)
    nbytes = O.state_bytes(g["layers"], g["channels"], g["state_size"], g["bytes_per_value"])
    assert nbytes == 28 * 4096 * 16 * 2 == 3670016
    assert abs(nbytes / 1e6 - g["printed_total_MB"]) <= g["printed_rounding_MB"], "3.7 MB figure"
    # Independent of the sequence length: the oracle's final state has the same shape.
    shapes = set()
    for L in (1, 8, 64):
        _, hf = O.scan(**tiny_real(23, L=L))
        shapes.add(hf.shape)
    assert len(shapes) == 1, "h_final shape depends on L"


def pin_complex_reduces_to_real(O):
    inp = tiny_real(29, L=20)
    y, hf = O.scan(**inp)
    c = dict(inp)
    c["A"] = np.stack([inp["A"], np.zeros_like(inp["A"])], -1)
    c["B"] = np.stack([inp["B"], np.zeros_like(inp["B"])], -1)
    c["C"] = np.stack([inp["C"], np.zeros_like(inp["C"])], -1)
    c["h0"] = np.stack([inp["h0"], np.zeros_like(inp["h0"])], -1)
    yc, hc = O.scan_complex(**c)
    assert _bitwise(yc, y), "theta = 0 complex scan differs from the real scan (y)"
    assert _bitwise(hc[..., 0], hf) and np.all(hc[..., 1] == 0.0), "theta = 0: state differs"


def pin_rotation(O, tol=1e-12):
    L, N = 64, 4
    theta = np.array([0.3, -1.1, 2.5, np.pi / 7])
    A = np.stack([np.zeros((1, N)), theta[None]], -1)
    x = np.zeros((1, L, 1)); x[0, 0, 0] = 1.0
    B = np.zeros((1, L, N, 2)); B[..., 0] = 1.0
    for n in range(N):
        C = np.zeros((1, L, N, 2)); C[:, :, n, 0] = 1.0
        y, _ = O.scan_complex(x, np.ones((1, L, 1)), A, B, C, np.zeros(1))
        assert _rel(y[0, :, 0], np.cos(theta[n] * np.arange(L))) <= tol, f"rotation, state {n}"
        Cs = np.zeros((1, L, N, 2)); Cs[:, :, n, 1] = -1.0   # Re(-i h) = Im h = sin
        ys, _ = O.scan_complex(x, np.ones((1, L, 1)), A, B, Cs, np.zeros(1))
        assert _rel(ys[0, :, 0], np.sin(theta[n] * np.arange(L))) <= tol, f"rotation sense, state {n}"


def pin_brute_force_complex(O, tol=1e-12):
    for seed, kw in [(31, {}), (32, dict(gated=True, with_h0=False))]:
        inp = tiny_complex(seed, **kw)
        y, hf = O.scan_complex(**inp)
        yb, hb = brute_complex(**inp)
        assert _rel(y, yb) <= tol, f"complex brute force y mismatch {_rel(y, yb)}"
        assert _rel(hf, hb) <= tol, f"complex brute force h_final mismatch {_rel(hf, hb)}"


# ---------------------------------------------------------------- input stage
def pin_conv_matches_numpy(O, tol=1e-12):
    # With a large bias the silu is the identity to far below fp64 resolution
    # (silu(v) = v (1 - e^-v + ...), e^-55 ~ 1e-24), so the convolution itself shows.
    r = np.random.default_rng(41)
    for K in (1, 2, 3, 4):
        b, L, Dn = 2, 13, 3
        x = r.normal(0, 1, (b, L, Dn))
        w = r.normal(0, 1, (Dn, K))
        cb = 60.0 + r.normal(0, 1, Dn)
        u, _ = O.conv_silu(x, w, cb)
        for bb in range(b):
            for d in range(Dn):
                ref = np.convolve(x[bb, :, d], w[d, ::-1])[:L] + cb[d]
                assert _rel(u[bb, :, d], ref) <= tol, f"conv vs np.convolve, K={K}, b={bb}, d={d}"


def pin_conv_impulse(O):
    # A unit impulse at step t0 of one channel: output t0 + j is silu(w[K-1-j]) for
    # j < K and silu(0) = 0 everywhere else (no bias); other channels stay 0.
    K, L, Dn, t0 = 4, 11, 3, 5
    w = np.array([[0.5, -1.5, 2.0, 3.0], [1.0, 1.0, 1.0, 1.0], [0.25, 0.75, -0.5, 1.25]])
    x = np.zeros((1, L, Dn)); x[0, t0, 2] = 1.0
    u, _ = O.conv_silu(x, w)
    ref = np.zeros((1, L, Dn))
    for j in range(K):
        ref[0, t0 + j, 2] = silu(w[2, K - 1 - j])
    assert np.array_equal(u, ref), "conv impulse response"


def pin_conv_state_carry(O):
    # Running a sequence in two calls with the conv state carried must equal one call
    # over the concatenation, also when the second part is shorter than K-1.
    r = np.random.default_rng(43)
    for K, L1, L2 in [(4, 7, 9), (4, 5, 2), (3, 6, 1), (2, 4, 5), (4, 1, 0)]:
        b, Dn = 2, 3
        x = r.normal(0, 1, (b, L1 + L2, Dn))
        w = r.normal(0, 1, (Dn, K)); cb = r.normal(0, 1, Dn)
        s0 = r.normal(0, 1, (b, K - 1, Dn))
        u, so = O.conv_silu(x, w, cb, s0)
        u1, so1 = O.conv_silu(x[:, :L1], w, cb, s0)
        u2, so2 = O.conv_silu(x[:, L1:], w, cb, so1)
        assert np.array_equal(np.concatenate([u1, u2], axis=1), u), f"conv split, K={K}"
        full = np.concatenate([s0, x], axis=1)
        assert np.array_equal(so2, full[:, full.shape[1] - (K - 1):]), f"conv state, K={K}"
        assert np.array_equal(so, so2), f"conv state of one call vs two, K={K}"


def pin_softplus(O):
    v = np.linspace(-30.0, 30.0, 241)
    assert _rel(O.softplus(v[None]), np.logaddexp(0.0, v)[None]) <= 1e-15, "softplus vs logaddexp"
    assert _rel(O.softplus(v[None]) - O.softplus(-v[None]), v[None]) <= 1e-14, "softplus(v) - softplus(-v) = v"
    assert abs(O.softplus(np.zeros((1, 1)))[0, 0] - np.log(2.0)) <= 1e-16, "softplus(0) = log 2"
    big = O.softplus(np.array([[800.0, -800.0, -40.0]]))
    assert big[0, 0] == 800.0 and 0.0 <= big[0, 1] < 1e-300, "softplus far from 0"
    assert abs(big[0, 2] - np.exp(-40.0)) <= 1e-15 * np.exp(-40.0), "softplus keeps tiny values"
    bias = np.array([-2.0, 0.5, 3.0, 7.0])
    out = O.softplus(np.zeros((3, 2, 4)), bias)
    assert _rel(out, np.broadcast_to(np.logaddexp(0.0, bias), (3, 2, 4))) <= 1e-15, "dt bias per channel"


def _inv_softplus(dt):
    return np.log(np.expm1(dt))


def pin_fused_identity_filter(O, tol=1e-12):
    # Filter (0, .., 0, 1) with no bias passes x through the convolution; the step
    # softplus^-1(dt) comes back as dt. The fused scan then equals the plain scan of
    # silu(x) with that dt, whatever the carried conv state holds.
    for seed, K in [(51, 4), (52, 2)]:
        inp = tiny_real(seed)
        b, L, Dn = inp["x"].shape
        w = np.zeros((Dn, K)); w[:, K - 1] = 1.0
        s0 = np.random.default_rng(seed).normal(0, 1, (b, K - 1, Dn))
        y, hf, _ = O.scan_fused(inp["x"], _inv_softplus(inp["dt"]), inp["A"], inp["B"], inp["C"],
                                inp["D"], inp["z"], inp["h0"], conv_w=w, conv_state0=s0)
        yr, hr = O.scan(silu(inp["x"]), inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                        inp["z"], inp["h0"])
        assert _rel(y, yr) <= tol and _rel(hf, hr) <= tol, f"fused identity filter, K={K}"


def pin_fused_step_equals_scan(O, tol=1e-12):
    # L fused decode steps (conv state and SSM state carried, two layers with their
    # own weights) against one fused prefill per layer.
    r = np.random.default_rng(61)
    Ln, S, Dn, N, K, L = 2, 2, 3, 4, 4, 9
    xin = r.normal(0, 1, (Ln, S, L, Dn)); dtr = r.normal(-1, 0.5, (Ln, S, L, Dn))
    z = r.normal(0, 1, (Ln, S, L, Dn))
    B = r.normal(0, 1, (Ln, S, L, N)); C = r.normal(0, 1, (Ln, S, L, N))
    A = -np.exp(r.normal(0, 0.5, (Ln, Dn, N))); D = r.normal(1, 0.1, (Ln, Dn))
    w = r.normal(0, 1, (Ln, Dn, K)); cb = r.normal(0, 0.5, (Ln, Dn)); db = r.normal(0, 0.5, (Ln, Dn))
    cs = r.normal(0, 1, (Ln, S, K - 1, Dn)); h = r.normal(0, 1, (Ln, S, Dn, N))
    ys = []
    hs, css = h, cs
    for t in range(L):
        yt, hs, css = O.step_fused(hs, css, xin[:, :, t], dtr[:, :, t], A, B[:, :, t], C[:, :, t], D,
                                   z[:, :, t], conv_w=w, conv_b=cb, dt_bias=db)
        ys.append(yt)
    ys = np.stack(ys, axis=2)
    for l in range(Ln):
        y, hf, so = O.scan_fused(xin[l], dtr[l], A[l], B[l], C[l], D[l], z[l], h[l], conv_w=w[l],
                                 conv_b=cb[l], conv_state0=cs[l], dt_bias=db[l])
        assert _rel(ys[l], y) <= tol and _rel(hs[l], hf) <= tol, f"fused decode vs prefill, layer {l}"
        assert np.array_equal(css[l], so), f"fused decode conv state, layer {l}"


# ---------------------------------------------------------------- backward
def _loss(O, inp, dy, dhf):
    y, hf = O.scan(**inp)
    return float(np.sum(dy * y) + (np.sum(dhf * hf) if dhf is not None else 0.0))


def pin_backward_finite_differences(O, tol=1e-7):
    # Every element of every input is perturbed by +-eps (relative to its size) and
    # the loss difference quotient compared with the gradient: truncation is
    # O(eps^2) ~ 1e-12 and rounding ~1e-16 / eps ~ 1e-10, far inside tol.
    for seed, kw, with_dhf in [(71, {}, True), (72, dict(gated=False, with_h0=False), False)]:
        inp = tiny_real(seed, b=2, L=5, Dn=2, N=3, **kw)
        r = np.random.default_rng(seed + 1)
        dy = r.normal(0, 1, inp["x"].shape)
        dhf = r.normal(0, 1, (2, 2, 3)) if with_dhf else None
        g = O.scan_bwd(**inp, dy=dy, dh_final=dhf)
        names = {"x": "dx", "dt": "ddt", "z": "dz", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "h0": "dh0"}
        for name, gname in names.items():
            if inp[name] is None:
                continue
            base = inp[name]
            fd = np.empty(base.shape)
            for idx in np.ndindex(base.shape):
                eps = 1e-6 * max(1.0, abs(base[idx]))
                hi = dict(inp); hi[name] = base.copy(); hi[name][idx] += eps
                lo = dict(inp); lo[name] = base.copy(); lo[name][idx] -= eps
                fd[idx] = (_loss(O, hi, dy, dhf) - _loss(O, lo, dy, dhf)) / (2 * eps)
            scale = max(1.0, float(np.max(np.abs(fd))))
            err = float(np.max(np.abs(fd - g[gname]))) / scale
            assert err <= tol, f"backward {gname} vs finite differences: {err:.2e} (seed {seed})"
        if inp["z"] is None:
            assert g["dz"] is None


def pin_fused_backward_finite_differences(O, tol=1e-7):
    # The backward through the input stage: every element of the raw input, the raw dt,
    # the filter, its bias, the carried conv state and the dt bias is perturbed by
    # +-eps and the difference quotient of the fused scan's loss compared with
    # scan_fused_bwd's gradient (and the scan's own inputs A, B, C, D, z, h0 once more,
    # through the input stage). K = 3 with every optional input, K = 1 without bias or
    # state, and K = 0 (no convolution: u = x_in).
    def loss(inp, dy, dhf):
        if inp["conv_w"] is None:
            y, hf = O.scan(inp["x_in"], O.softplus(inp["dt_raw"], inp["dt_bias"]), inp["A"],
                           inp["B"], inp["C"], inp["D"], inp["z"], inp["h0"])
        else:
            y, hf, _ = O.scan_fused(**inp)
        return float(np.sum(dy * y) + (np.sum(dhf * hf) if dhf is not None else 0.0))

    for seed, K, full in [(81, 3, True), (82, 1, False), (83, 0, True)]:
        base = tiny_real(seed, b=2, L=5, Dn=2, N=3, with_h0=full)
        r = np.random.default_rng(seed + 1)
        b, L, Dn = base["x"].shape
        inp = dict(x_in=base.pop("x"), dt_raw=_inv_softplus(base.pop("dt")) - 0.3, **base,
                   conv_w=r.normal(0, 0.7, (Dn, K)) if K else None,
                   conv_b=r.normal(0, 0.5, Dn) if (K and full) else None,
                   conv_state0=r.normal(0, 1, (b, K - 1, Dn)) if (K > 1 and full) else None,
                   dt_bias=r.normal(0, 0.2, Dn) if full else None)
        dy = r.normal(0, 1, (b, L, Dn))
        dhf = r.normal(0, 1, (b, Dn, 3)) if full else None
        g = O.scan_fused_bwd(**inp, dy=dy, dh_final=dhf)
        names = {"x_in": "dx_in", "dt_raw": "ddt_raw", "conv_w": "dconv_w", "conv_b": "dconv_b",
                 "conv_state0": "dconv_state0", "dt_bias": "ddt_bias", "A": "dA", "B": "dB",
                 "C": "dC", "D": "dD", "z": "dz", "h0": "dh0"}
        for name, gname in names.items():
            if inp[name] is None:
                continue
            v = inp[name]
            fd = np.empty(v.shape)
            for idx in np.ndindex(v.shape):
                eps = 1e-6 * max(1.0, abs(v[idx]))
                hi = dict(inp); hi[name] = v.copy(); hi[name][idx] += eps
                lo = dict(inp); lo[name] = v.copy(); lo[name][idx] -= eps
                fd[idx] = (loss(hi, dy, dhf) - loss(lo, dy, dhf)) / (2 * eps)
            scale = max(1.0, float(np.max(np.abs(fd))))
            err = float(np.max(np.abs(fd - g[gname]))) / scale
            assert err <= tol, f"fused backward {gname} vs finite differences: {err:.2e} (K={K})"


# ----------------------------------------------------------------------------- trapezoid

def brute_trap(x, dt, A, B, C, D, z=None, h0=None, x_prev=None, B_prev=None, lam=None):
    """The exponential-trapezoidal state written out: with S_t the running sum of dt
    (S_-1 = 0), p_s = B_s x_s, p_-1 the input before step 0 and lam_s the weight of
    step s's current input (1/2 when lam is None),
        h_t = exp(A S_t) h0 + sum_{s<=t} dt_s (lam_s exp(A (S_t - S_s)) p_s
                                               + (1 - lam_s) exp(A (S_t - S_{s-1})) p_{s-1})."""
    b, L, Dn = x.shape
    N = A.shape[1]
    lam = np.full((b, L, Dn), 0.5) if lam is None else lam
    S = np.concatenate([np.zeros((b, 1, Dn)), np.cumsum(dt, axis=1)], axis=1)   # S[:, t+1] = S_t
    y = np.zeros((b, L, Dn)); hf = np.zeros((b, Dn, N))
    for bi in range(b):
        for d in range(Dn):
            p = np.zeros((L + 1, N))                                        # p[s+1] = p_s
            if x_prev is not None:
                p[0] = B_prev[bi] * x_prev[bi, d]
            p[1:] = B[bi] * x[bi, :, d][:, None]
            for t in range(L):
                h = np.zeros(N) if h0 is None else np.exp(A[d] * S[bi, t + 1, d]) * h0[bi, d]
                for s_ in range(t + 1):
                    lv = lam[bi, s_, d]
                    h = h + dt[bi, s_, d] * (
                        lv * np.exp(A[d] * (S[bi, t + 1, d] - S[bi, s_ + 1, d])) * p[s_ + 1]
                        + (1.0 - lv) * np.exp(A[d] * (S[bi, t + 1, d] - S[bi, s_, d])) * p[s_])
                yv = float(C[bi, t] @ h) + D[d] * x[bi, t, d]
                if z is not None:
                    yv *= silu(z[bi, t, d])
                y[bi, t, d] = yv
                if t == L - 1:
                    hf[bi, d] = h
    return y, hf


def pin_trap_brute_force(O, tol=1e-12):
    # the default weight (1/2, the trapezoid rule) and random per-step weights in [0, 1]
    for seed, with_prev, with_lam in [(71, True, False), (72, False, False), (76, True, True),
                                      (77, False, True)]:
        inp = tiny_real(seed, L=16)
        r = np.random.default_rng(seed + 100)
        b, L, Dn = inp["x"].shape
        xp = r.normal(0, 1, (b, Dn)) if with_prev else None
        Bp = r.normal(0, 1, (b, inp["A"].shape[1])) if with_prev else None
        lam = r.uniform(0.0, 1.0, (b, L, Dn)) if with_lam else None
        y, hf = O.scan_trap(**inp, x_prev=xp, B_prev=Bp, lam=lam)
        yb, hb = brute_trap(**inp, x_prev=xp, B_prev=Bp, lam=lam)
        assert _rel(y, yb) <= tol and _rel(hf, hb) <= tol, \
            f"trapezoid vs brute force (prev={with_prev}, lam={with_lam})"
        if not with_lam:  # an explicit weight of 1/2 is the default
            y2, h2 = O.scan_trap(**inp, x_prev=xp, B_prev=Bp, lam=np.full((b, L, Dn), 0.5))
            assert _bitwise(y2, y) and _bitwise(h2, hf), "lam = 1/2 differs from the default"


def pin_trap_lambda_one_is_euler(O, tol=1e-13):
    # Weight 1 on the current input is Euler's step: the plain scan (and its decode
    # step), whatever the previous input holds.
    inp = tiny_real(78, L=24)
    r = np.random.default_rng(178)
    b, L, Dn = inp["x"].shape
    N = inp["A"].shape[1]
    ones = np.ones((b, L, Dn))
    y, hf = O.scan_trap(**inp, x_prev=r.normal(0, 1, (b, Dn)), B_prev=r.normal(0, 1, (b, N)), lam=ones)
    ye, he = O.scan(**inp)
    assert _rel(y, ye) <= tol and _rel(hf, he) <= tol, "lam = 1 is not the Euler scan"
    Ln, S = 2, 3
    h = r.normal(0, 1, (Ln, S, Dn, N))
    x = r.normal(0, 1, (Ln, S, Dn)); dt = np.log1p(np.exp(r.normal(-1, 0.5, (Ln, S, Dn))))
    B = r.normal(0, 1, (Ln, S, N)); C = r.normal(0, 1, (Ln, S, N)); z = r.normal(0, 1, (Ln, S, Dn))
    A = -np.exp(r.normal(0, 0.5, (Ln, Dn, N))); D = r.normal(1, 0.1, (Ln, Dn))
    yt, ht = O.step_trap(h, r.normal(0, 1, (Ln, S, Dn)), r.normal(0, 1, (Ln, S, N)), x, dt, A, B, C, D, z,
                         lam=np.ones((Ln, S, Dn)))
    ys, hs = O.step(h, x, dt, A, B, C, D, z)
    assert _rel(yt, ys) <= tol and _rel(ht, hs) <= tol, "decode with lam = 1 is not the Euler step"


def pin_trap_a_zero_is_trapezoid_rule(O, tol=1e-12):
    # With A = 0 nothing decays: the state is h0 plus the trapezoid-rule integral of
    # the samples p_s = B_s x_s over the time grid (0, dt_0, dt_0 + dt_1, ..), p_-1 at 0.
    r = np.random.default_rng(73)
    b, L, Dn, N = 2, 11, 3, 4
    x = r.normal(0, 1, (b, L, Dn)); dt = r.uniform(0.05, 0.9, (b, L, Dn))
    B = r.normal(0, 1, (b, L, N)); C = r.normal(0, 1, (b, L, N))
    xp = r.normal(0, 1, (b, Dn)); Bp = r.normal(0, 1, (b, N)); h0 = r.normal(0, 1, (b, Dn, N))
    y, hf = O.scan_trap(x, dt, np.zeros((Dn, N)), B, C, np.zeros(Dn), None, h0, x_prev=xp, B_prev=Bp)
    for bi in range(b):
        for d in range(Dn):
            grid = np.concatenate([[0.0], np.cumsum(dt[bi, :, d])])
            samples = np.concatenate([(Bp[bi] * xp[bi, d])[None], B[bi] * x[bi, :, d][:, None]])  # [L+1, N]
            for t in range(L):
                h = h0[bi, d] + np.trapezoid(samples[:t + 2], grid[:t + 2], axis=0)
                assert abs(y[bi, t, d] - float(C[bi, t] @ h)) <= tol * max(1.0, np.abs(h).max()), "A = 0: y"
            assert _rel(hf[bi, d], h) <= tol, "A = 0: trapezoid rule"


def pin_trap_second_order(O):
    # h' = -a h + b cos(w s) from h(0) = h0, sampled at s = k T / M: the discrete state
    # after M steps against the closed form
    #   h(T) = e^{-aT} h0 + b (a cos wT + w sin wT - a e^{-aT}) / (a^2 + w^2).
    # The trapezoid rule is second order: the error falls ~4x per halved step; the
    # Euler scan's (first order) ~2x.
    a, bb, w, T, h0 = 1.3, 0.7, 2.1, 3.0, 0.4
    exact = np.exp(-a * T) * h0 + bb * (a * np.cos(w * T) + w * np.sin(w * T) - a * np.exp(-a * T)) / (a * a + w * w)
    # With the weight 1 (Euler's step inside the same rule) it is first order again.
    errs, errs_euler, errs_one = [], [], []
    for M in (40, 80, 160):
        dt = np.full((1, M, 1), T / M)
        s = np.arange(1, M + 1) * (T / M)
        x = np.cos(w * s).reshape(1, M, 1)
        B = np.full((1, M, 1), bb); C = np.ones((1, M, 1))
        A = np.full((1, 1), -a); D = np.zeros(1); H0 = np.full((1, 1, 1), h0)
        prev = dict(x_prev=np.ones((1, 1)), B_prev=np.full((1, 1), bb))
        _, hf = O.scan_trap(x, dt, A, B, C, D, None, H0, **prev)
        _, h1 = O.scan_trap(x, dt, A, B, C, D, None, H0, **prev, lam=np.ones((1, M, 1)))
        _, he = O.scan(x, dt, A, B, C, D, None, H0)
        errs.append(abs(hf[0, 0, 0] - exact)); errs_euler.append(abs(he[0, 0, 0] - exact))
        errs_one.append(abs(h1[0, 0, 0] - exact))
    for e1, e2 in zip(errs, errs[1:]):
        assert 3.6 <= e1 / e2 <= 4.4, f"trapezoid convergence ratio {e1 / e2:.3f}"
    for e1, e2 in zip(errs_euler, errs_euler[1:]):
        assert 1.7 <= e1 / e2 <= 2.3, f"Euler convergence ratio {e1 / e2:.3f}"
    for e1, e2 in zip(errs_one, errs_one[1:]):
        assert 1.7 <= e1 / e2 <= 2.3, f"lam = 1 convergence ratio {e1 / e2:.3f}"


def pin_trap_split_resume(O):
    inp = tiny_real(74, L=30)
    r = np.random.default_rng(174)
    b, L, Dn = inp["x"].shape
    N = inp["A"].shape[1]
    xp, Bp = r.normal(0, 1, (b, Dn)), r.normal(0, 1, (b, N))
    lam = r.uniform(0.0, 1.0, (b, L, Dn))
    y, hf = O.scan_trap(**inp, x_prev=xp, B_prev=Bp, lam=lam)
    k = 13
    part = lambda v, sl: None if v is None else v[:, sl]
    y1, h1 = O.scan_trap(part(inp["x"], slice(0, k)), part(inp["dt"], slice(0, k)), inp["A"],
                         part(inp["B"], slice(0, k)), part(inp["C"], slice(0, k)), inp["D"],
                         part(inp["z"], slice(0, k)), inp["h0"], x_prev=xp, B_prev=Bp,
                         lam=part(lam, slice(0, k)))
    y2, h2 = O.scan_trap(part(inp["x"], slice(k, L)), part(inp["dt"], slice(k, L)), inp["A"],
                         part(inp["B"], slice(k, L)), part(inp["C"], slice(k, L)), inp["D"],
                         part(inp["z"], slice(k, L)), h1, x_prev=inp["x"][:, k - 1],
                         B_prev=inp["B"][:, k - 1], lam=part(lam, slice(k, L)))
    assert _bitwise(np.concatenate([y1, y2], axis=1), y) and _bitwise(h2, hf), "trapezoid split/resume"


def pin_trap_step_equals_scan(O):
    # L decode steps, each given the previous token's x and B, against one prefill per
    # (layer, sequence); two layers with their own A and D.
    r = np.random.default_rng(75)
    Ln, S, Dn, N, L = 2, 3, 3, 4, 8
    x = r.normal(0, 1, (Ln, S, L, Dn)); dt = np.log1p(np.exp(r.normal(-1, 0.5, (Ln, S, L, Dn))))
    z = r.normal(0, 1, (Ln, S, L, Dn))
    B = r.normal(0, 1, (Ln, S, L, N)); C = r.normal(0, 1, (Ln, S, L, N))
    A = -np.exp(r.normal(0, 0.5, (Ln, Dn, N))); D = r.normal(1, 0.1, (Ln, Dn))
    h = r.normal(0, 1, (Ln, S, Dn, N))
    xp0, Bp0 = r.normal(0, 1, (Ln, S, Dn)), r.normal(0, 1, (Ln, S, N))
    lam = r.uniform(0.0, 1.0, (Ln, S, L, Dn))
    hs, ys = h, []
    for t in range(L):
        xp = xp0 if t == 0 else x[:, :, t - 1]
        Bp = Bp0 if t == 0 else B[:, :, t - 1]
        yt, hs = O.step_trap(hs, xp, Bp, x[:, :, t], dt[:, :, t], A, B[:, :, t], C[:, :, t], D, z[:, :, t],
                             lam=lam[:, :, t])
        ys.append(yt)
    ys = np.stack(ys, axis=2)
    for l in range(Ln):
        yl, hl = O.scan_trap(x[l], dt[l], A[l], B[l], C[l], D[l], z[l], h[l], x_prev=xp0[l], B_prev=Bp0[l],
                             lam=lam[l])
        assert _bitwise(ys[l], yl) and _bitwise(hs[l], hl), f"trapezoid decode vs prefill, layer {l}"


# ----------------------------------------------------------------------------- MIMO

def tiny_mimo(seed, b=2, L=20, Dn=3, N=4, R=3, gated=True, with_h0=True):
    r = np.random.default_rng(seed)
    inp = tiny_real(seed, b=b, L=L, Dn=Dn, N=N, gated=False, with_h0=with_h0)
    inp["x"] = r.normal(0, 1, (b, L, Dn, R))
    inp["B"] = r.normal(0, 1, (b, L, N, R))
    inp["C"] = r.normal(0, 1, (b, L, N, R))
    inp["z"] = r.normal(0, 1, (b, L, Dn, R)) if gated else None
    return inp


def brute_mimo(x, dt, A, B, C, D, z=None, h0=None):
    """The MIMO state written out with S_t the running sum of dt:
        h_t = exp(A S_t) h0 + sum_{s<=t} exp(A (S_t - S_s)) dt_s B_s x_s   (B_s: N x R),
        y_t = C_t^T h_t + D x_t, then the gate per output."""
    b, L, Dn, R = x.shape
    N = A.shape[1]
    S = np.cumsum(dt, axis=1)
    y = np.zeros((b, L, Dn, R)); hf = np.zeros((b, Dn, N))
    for bi in range(b):
        for d in range(Dn):
            for t in range(L):
                h = np.zeros(N) if h0 is None else np.exp(A[d] * S[bi, t, d]) * h0[bi, d]
                for s_ in range(t + 1):
                    h = h + np.exp(A[d] * (S[bi, t, d] - S[bi, s_, d])) * dt[bi, s_, d] * (B[bi, s_] @ x[bi, s_, d])
                yv = C[bi, t].T @ h + D[d] * x[bi, t, d]
                if z is not None:
                    yv = yv * silu(z[bi, t, d])
                y[bi, t, d] = yv
                if t == L - 1:
                    hf[bi, d] = h
    return y, hf


def pin_mimo_rank_one_is_siso(O):
    inp = tiny_mimo(81, R=1)
    y, hf = O.scan_mimo(**inp)
    ys, hs = O.scan(inp["x"][..., 0], inp["dt"], inp["A"], inp["B"][..., 0], inp["C"][..., 0],
                    inp["D"], inp["z"][..., 0], inp["h0"])
    assert _bitwise(y[..., 0], ys) and _bitwise(hf, hs), "MIMO rank 1 vs the scan"


def pin_mimo_superposition(O, tol=1e-12):
    # No skip, gate or initial state: the state is linear in the input, so output r is
    # the sum over inputs r' of the scan that reads only input r' (through column r' of
    # B) and reads out through column r of C.
    inp = tiny_mimo(82, R=3, gated=False, with_h0=False)
    x, dt, A, B, C = inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"]
    b, L, Dn, R = x.shape
    zero = np.zeros(Dn)
    y, hf = O.scan_mimo(x, dt, A, B, C, zero)
    for r in range(R):
        acc = np.zeros((b, L, Dn)); hacc = np.zeros(hf.shape)
        for rp in range(R):
            ys, hs = O.scan(x[..., rp], dt, A, B[..., rp], C[..., r], zero)
            acc += ys; hacc += hs
        assert _rel(y[..., r], acc) <= tol, f"MIMO superposition, output {r}"
        assert _rel(hf, hacc) <= tol, "MIMO superposition, final state"


def pin_mimo_brute_force(O, tol=1e-12):
    for seed, R, gated in [(83, 4, True), (84, 2, False)]:
        inp = tiny_mimo(seed, L=14, R=R, gated=gated)
        y, hf = O.scan_mimo(**inp)
        yb, hb = brute_mimo(**inp)
        assert _rel(y, yb) <= tol and _rel(hf, hb) <= tol, f"MIMO vs brute force (R={R})"


def pin_mimo_split_resume(O):
    inp = tiny_mimo(85, L=27, R=4)
    y, hf = O.scan_mimo(**inp)
    k = 11
    part = lambda v, sl: None if v is None else v[:, sl]
    args = lambda sl: (part(inp["x"], sl), part(inp["dt"], sl), inp["A"], part(inp["B"], sl),
                       part(inp["C"], sl), inp["D"], part(inp["z"], sl))
    y1, h1 = O.scan_mimo(*args(slice(0, k)), inp["h0"])
    y2, h2 = O.scan_mimo(*args(slice(k, None)), h1)
    assert _bitwise(np.concatenate([y1, y2], axis=1), y) and _bitwise(h2, hf), "MIMO split/resume"


def pin_mimo_step_equals_scan(O):
    r = np.random.default_rng(86)
    Ln, S, Dn, N, R, L = 2, 3, 3, 4, 4, 7
    x = r.normal(0, 1, (Ln, S, L, Dn, R)); z = r.normal(0, 1, (Ln, S, L, Dn, R))
    dt = np.log1p(np.exp(r.normal(-1, 0.5, (Ln, S, L, Dn))))
    B = r.normal(0, 1, (Ln, S, L, N, R)); C = r.normal(0, 1, (Ln, S, L, N, R))
    A = -np.exp(r.normal(0, 0.5, (Ln, Dn, N))); D = r.normal(1, 0.1, (Ln, Dn))
    h = r.normal(0, 1, (Ln, S, Dn, N))
    hs, ys = h, []
    for t in range(L):
        yt, hs = O.step_mimo(hs, x[:, :, t], dt[:, :, t], A, B[:, :, t], C[:, :, t], D, z[:, :, t])
        ys.append(yt)
    ys = np.stack(ys, axis=2)
    for l in range(Ln):
        yl, hl = O.scan_mimo(x[l], dt[l], A[l], B[l], C[l], D[l], z[l], h[l])
        assert _bitwise(ys[l], yl) and _bitwise(hs[l], hl), f"MIMO decode vs prefill, layer {l}"


ALL_PINS = [
    pin_brute_force, pin_convolution, pin_geometric_series, pin_dt_zero, pin_linearity,
    pin_split_resume, pin_step_equals_scan, pin_isolation, pin_state_bytes,
    pin_complex_reduces_to_real, pin_rotation, pin_brute_force_complex,
    lambda O: pin_split_resume(O, complex_state=True),
    lambda O: pin_step_equals_scan(O, complex_state=True),
    pin_layers_are_independent,
    lambda O: pin_layers_are_independent(O, complex_state=True),
    pin_conv_matches_numpy, pin_conv_impulse, pin_conv_state_carry, pin_softplus,
    pin_fused_identity_filter, pin_fused_step_equals_scan, pin_backward_finite_differences,
    pin_fused_backward_finite_differences,
    pin_trap_brute_force, pin_trap_lambda_one_is_euler, pin_trap_a_zero_is_trapezoid_rule,
    pin_trap_second_order,
    pin_trap_split_resume, pin_trap_step_equals_scan,
    pin_mimo_rank_one_is_siso, pin_mimo_superposition, pin_mimo_brute_force,
    pin_mimo_split_resume, pin_mimo_step_equals_scan,
]
