"""The exponential-trapezoidal scan (ssm_scan_fwd_trap) and decode step (ssm_step_trap)
on the GPU against the fp64 oracle's scan_trap / step_trap, plus invariants.

Prefill cases span several chunks and 64-lane waves with ragged tails, every state
size, with and without the input before step 0 (x_prev, B_prev), gate and h0, each
with no weight (1/2), weight 1 (Euler's step) and random weights in [0, 1]. Weight 1
equals the Euler prefill's values exactly; an explicit weight 1/2 equals no weight bit
for bit. Decode is checked bit for bit against its replay kernel and against the
oracle. Resuming a sequence from (h_final, last x, last B) equals one call; L decode
steps equal one prefill; the 256k prefill at full size on 1024 sampled channels.
"""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_49_amd as ssm
from tests.gpu_util import TOL, bitwise_equal, gather_channels, rel_err, say, threaded_channels, to_dev
from workloads import (WORKLOADS, DecodeShape, ScanShape, make_decode_params, make_decode_step,
                       make_h0, make_prev_input, make_scan_inputs, make_trap_weight,
                       sample_channels)

pytestmark = pytest.mark.gpu

# (batch, L, d_inner, d_state, io, gated, with_h0, with_prev, chunk_len)
CASES = [
    (2, 300, 200, 16, "bf16", True, True, True, 64),     # 5 chunks, ragged last chunk
    (2, 300, 200, 16, "f32", False, True, True, 37),     # 9 chunks of odd length
    (1, 1000, 130, 8, "bf16", True, False, True, 0),     # library's own plan
    (2, 257, 70, 4, "f32", True, True, False, 50),       # no input before step 0
    (1, 203, 65, 2, "f32", True, True, True, 50),
    (3, 129, 64, 1, "f32", False, False, True, 16),
    (3, 131, 40, 1, "bf16", True, True, True, 16),       # bf16, N = 1, odd rows of B
    (1, 1, 1, 1, "f32", True, True, True, 0),            # one step, one channel
    (1, 4501, 33, 16, "f32", True, True, True, 64),      # 71 chunks
    (2, 777, 96, 16, "bf16", False, True, True, 5),      # chunks shorter than a register block
]


def _ids(c):
    b, L, Dn, N, io, g, h0, pv, T = c
    return (f"b{b}_L{L}_D{Dn}_N{N}_{io}_{'gated' if g else 'nogate'}_{'h0' if h0 else 'zero'}_"
            f"{'prev' if pv else 'noprev'}_T{T}")


LAMS = ("none", "one", "random")


def _draw(case, seed=0, lam="none"):
    b, L, Dn, N, io, gated, with_h0, with_prev, T = case
    shape = ScanShape("trap", b, L, Dn, N, io, gated=gated, seed=300 + seed)
    inp = make_scan_inputs(shape, "cpu")
    inp["h0"] = make_h0(b, Dn, N, seed=17 + seed) if with_h0 else None
    prev = make_prev_input(b, Dn, N, io, seed=31 + seed) if with_prev else {"x_prev": None, "B_prev": None}
    inp.update(prev)
    inp["lam"] = None if lam == "none" else make_trap_weight((b, L, Dn), io, kind=lam, seed=41 + seed)
    return shape, inp


def _gpu(d, chunk_len):
    g = to_dev(d)
    return ssm.ssm_scan_fwd_trap(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["z"], g["h0"],
                                 g["x_prev"], g["B_prev"], lam=g["lam"], chunk_len=chunk_len)


def _oracle(d):
    return oracle.scan_trap(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], d["h0"],
                            x_prev=d["x_prev"], B_prev=d["B_prev"], lam=d["lam"])


@pytest.mark.parametrize("lam", LAMS)
@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_trap_prefill_matches_oracle(case, lam):
    shape, d = _draw(case, lam=lam)
    say("trapezoid prefill", _ids(case), "lam", lam)
    y, hf = _gpu(d, case[-1])
    torch.cuda.synchronize()
    yr, hr = _oracle(d)
    tol = TOL[shape.io]
    assert rel_err(y, yr) <= tol, f"y error {rel_err(y, yr)}"
    assert rel_err(hf, hr) <= tol, f"h_final error {rel_err(hf, hr)}"


def test_trap_single_step_cancelling_output():
    # One step of one channel with 16 states (fp32, gated, h0, input before step 0), for
    # every weight. The single output is a sum of 17 terms of size ~1 that can cancel to
    # ~1e-4, so the plain criterion (error over max |y_ref| of a one-element tensor) would
    # measure fp32 rounding of the terms against their cancelled sum. The written
    # criterion for tensors of fewer than 64 outputs takes the size of the terms instead:
    # scale = max over outputs of (sum_n |C_n h_n| + |D x|) |silu(z)|, in fp64 from the
    # oracle's state (h_final is the state after the one step).
    for seed in range(6):
        for lam in LAMS:
            shape, d = _draw((1, 1, 1, 16, "f32", True, True, True, 0), seed=10 + seed, lam=lam)
            say("trapezoid single step", seed, lam)
            y, hf = _gpu(d, 0)
            torch.cuda.synchronize()
            yr, hr = _oracle(d)
            f = {k: oracle.to_f64(v) for k, v in d.items() if v is not None}
            zv = f["z"][0, 0, 0]
            terms = (np.abs(f["C"][0, 0] * hr[0, 0]).sum() + abs(f["D"][0] * f["x"][0, 0, 0])) \
                * abs(zv / (1.0 + np.exp(-zv)))
            err = float(np.abs(oracle.to_f64(y) - yr).max())
            assert err <= TOL["f32"] * terms, f"y error {err:.3e} vs term scale {terms:.3e} (seed {seed}, {lam})"
            assert rel_err(hf, hr) <= TOL["f32"], f"h_final (seed {seed}, {lam})"


def test_trap_weight_one_is_euler_and_half_is_default():
    # Weight 1 makes both taps Euler's: the trapezoid kernels then give the Euler
    # prefill's values exactly (same chunks; the older tap adds 0 * B_prev x_prev).
    # An explicit weight 1/2 performs the default's operations: bit for bit.
    for case in [(2, 300, 200, 16, "bf16", True, True, True, 64), (1, 1000, 130, 8, "f32", False, True, True, 100)]:
        shape, d = _draw(case, seed=5, lam="one")
        g = to_dev(d)
        T = case[-1]
        say("trapezoid weight 1 vs Euler", _ids(case))
        y1, h1 = _gpu(d, T)
        ye, he = ssm.ssm_scan_fwd_ex(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["z"], g["h0"],
                                     chunk_len=T)
        g["lam"] = make_trap_weight(g["x"].shape, shape.io, "cuda", kind="half")
        yh, hh = ssm.ssm_scan_fwd_trap(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["z"], g["h0"],
                                       g["x_prev"], g["B_prev"], lam=g["lam"], chunk_len=T)
        yn, hn = ssm.ssm_scan_fwd_trap(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["z"], g["h0"],
                                       g["x_prev"], g["B_prev"], chunk_len=T)
        torch.cuda.synchronize()
        assert torch.equal(y1, ye) and torch.equal(h1, he), "weight 1 differs from the Euler prefill"
        assert bitwise_equal(yh, yn) and bitwise_equal(hh, hn), "weight 1/2 differs from no weight"


def test_trap_chunking_determinism_and_empty():
    case = (2, 600, 96, 16, "f32", True, True, True, 0)
    shape, d = _draw(case, seed=1, lam="random")
    say("trapezoid chunk independence")
    y0, h0 = _gpu(d, 0)
    y1, h1 = _gpu(d, 0)
    torch.cuda.synchronize()
    assert bitwise_equal(y0, y1) and bitwise_equal(h0, h1), "not deterministic"
    for T in (600, 64, 41, 8):
        y, hf = _gpu(d, T)
        torch.cuda.synchronize()
        assert rel_err(y, oracle.to_f64(y0)) <= TOL["f32"], f"chunk {T}"
        assert rel_err(hf, oracle.to_f64(h0)) <= TOL["f32"], f"chunk {T}"
    # L = 0: h_final = h0 and nothing else is read
    g = to_dev(d)
    e = lambda t: t[:, :0].contiguous()
    y, hf = ssm.ssm_scan_fwd_trap(e(g["x"]), e(g["dt"]), g["A"], e(g["B"]), e(g["C"]), g["D"],
                                  e(g["z"]), g["h0"], g["x_prev"], g["B_prev"], lam=e(g["lam"]))
    torch.cuda.synchronize()
    assert y.numel() == 0 and bitwise_equal(hf, g["h0"])


def test_trap_split_resume_matches_whole():
    # Two calls, the second from (h_final, x and B of the first part's last step),
    # against one call over the whole sequence.
    case = (2, 700, 96, 16, "f32", True, True, True, 64)
    shape, d = _draw(case, seed=2, lam="random")
    g = to_dev(d)
    say("trapezoid split/resume")
    y, hf = _gpu(d, 64)
    k = 333
    p = lambda t, sl: None if t is None else t[:, sl].contiguous()
    y1, h1 = ssm.ssm_scan_fwd_trap(p(g["x"], slice(0, k)), p(g["dt"], slice(0, k)), g["A"],
                                   p(g["B"], slice(0, k)), p(g["C"], slice(0, k)), g["D"],
                                   p(g["z"], slice(0, k)), g["h0"], g["x_prev"], g["B_prev"],
                                   lam=p(g["lam"], slice(0, k)), chunk_len=64)
    y2, h2 = ssm.ssm_scan_fwd_trap(p(g["x"], slice(k, None)), p(g["dt"], slice(k, None)), g["A"],
                                   p(g["B"], slice(k, None)), p(g["C"], slice(k, None)), g["D"],
                                   p(g["z"], slice(k, None)), h1, g["x"][:, k - 1].contiguous(),
                                   g["B"][:, k - 1].contiguous(), lam=p(g["lam"], slice(k, None)),
                                   chunk_len=64)
    torch.cuda.synchronize()
    yy = torch.cat([y1, y2], dim=1)
    assert rel_err(yy, oracle.to_f64(y)) <= TOL["f32"] and rel_err(h2, oracle.to_f64(hf)) <= TOL["f32"]


def test_trap_slow_decay_and_frozen_state():
    # Decay horizons that are never reached within a chunk (whole-chunk windows).
    shape, d = _draw((1, 3000, 130, 16, "f32", True, True, True, 500), seed=3, lam="random")
    d["A"] = d["A"] * 1e-3
    d["A"][5] = 0.0
    say("trapezoid slow decay")
    y, hf = _gpu(d, 500)
    torch.cuda.synchronize()
    yr, hr = _oracle(d)
    assert rel_err(y, yr) <= TOL["f32"] and rel_err(hf, hr) <= TOL["f32"]


# ---------------------------------------------------------------- decode
# (n_layers, n_seq, d_inner, d_state, io, gated)
DECODE_CASES = [
    (3, 5, 130, 16, "bf16", True),
    (2, 4, 64, 16, "f32", False),
    (2, 3, 77, 8, "f32", True),
    (1, 7, 33, 4, "bf16", True),
    (2, 2, 40, 2, "f32", True),
    (2, 3, 20, 1, "bf16", True),
    (1, 2, 600, 16, "bf16", True),   # three blocks of 256 channels, the last ragged
]
STEPS = 5


def _dids(c):
    Ln, S, Dn, N, io, g = c
    return f"L{Ln}_S{S}_D{Dn}_N{N}_{io}_{'gated' if g else 'nogate'}"


@pytest.mark.parametrize("lam", ("none", "random"))
@pytest.mark.parametrize("case", DECODE_CASES, ids=_dids)
def test_trap_step_bitwise_replay_and_oracle(case, lam):
    Ln, S, Dn, N, io, gated = case
    shape = DecodeShape("trap", Ln, S, Dn, N, STEPS, io, gated=gated, seed=470)
    par = make_decode_params(shape, "cpu")
    h0 = torch.randn((Ln, S, Dn, N), generator=torch.Generator().manual_seed(8))
    h_fast, h_rep, h_ref = h0.cuda(), h0.cuda(), h0.double().numpy()
    A, D = par["A"].cuda(), par["D"].cuda()
    prev = None
    for k in range(STEPS):
        inp = make_decode_step(shape, k, "cpu")
        g = to_dev(inp)
        xp = None if prev is None else prev["x"]
        Bp = None if prev is None else prev["B"]
        gxp = None if xp is None else xp.cuda()
        gBp = None if Bp is None else Bp.cuda()
        lw = None if lam == "none" else make_trap_weight((Ln, S, Dn), io, kind=lam, seed=60 + k)
        glw = None if lw is None else lw.cuda()
        say("trapezoid decode", _dids(case), lam, "step", k)
        y1 = ssm.ssm_step_trap(h_fast, gxp, gBp, g["x"], g["dt"], A, g["B"], g["C"], D, g["z"], lam_t=glw)
        y2 = ssm.ssm_step_trap_replay(h_rep, gxp, gBp, g["x"], g["dt"], A, g["B"], g["C"], D, g["z"],
                                      lam_t=glw)
        torch.cuda.synchronize()
        assert bitwise_equal(y1, y2), f"y differs from replay at step {k}"
        assert bitwise_equal(h_fast, h_rep), f"state differs from replay at step {k}"
        yr, h_ref = oracle.step_trap(h_ref, xp, Bp, inp["x"], inp["dt"], par["A"], inp["B"], inp["C"],
                                     par["D"], inp["z"], lam=lw)
        assert rel_err(y1, yr) <= TOL[io], f"y vs oracle {rel_err(y1, yr)} at step {k}"
        assert rel_err(h_fast, h_ref) <= TOL[io], f"h vs oracle at step {k}"
        prev = inp


def test_trap_prefill_equals_decode():
    # L decode steps (one layer, n_seq = batch) against one prefill of the same tokens.
    b, L, Dn, N = 3, 40, 96, 16
    shape, d = _draw((b, L, Dn, N, "f32", True, True, True, 16), seed=4, lam="random")
    say("trapezoid prefill vs decode")
    y, hf = _gpu(d, 16)
    g = to_dev(d)
    h = g["h0"].view(1, b, Dn, N).contiguous()
    row = lambda v, t: v[:, t].unsqueeze(0).contiguous()
    ys = []
    for t in range(L):
        xp = g["x_prev"].unsqueeze(0).contiguous() if t == 0 else row(g["x"], t - 1)
        Bp = g["B_prev"].unsqueeze(0).contiguous() if t == 0 else row(g["B"], t - 1)
        ys.append(ssm.ssm_step_trap(h, xp, Bp, row(g["x"], t), row(g["dt"], t), g["A"].unsqueeze(0),
                                    row(g["B"], t), row(g["C"], t), g["D"].unsqueeze(0),
                                    row(g["z"], t), lam_t=row(g["lam"], t))[0])
    torch.cuda.synchronize()
    assert rel_err(torch.stack(ys, dim=1), oracle.to_f64(y)) <= TOL["f32"]
    assert rel_err(h[0], oracle.to_f64(hf)) <= TOL["f32"]


@pytest.mark.parametrize("lam", ("none", "random"))
def test_trap_full_size_long_context_sampled(lam):
    # The 256k prefill (batch 1, L 262144, 8192 channels, N 16, bf16) in the library's
    # own chunk plan, as the benchmark times it; 1024 sampled channels (8 of each 64-lane
    # wave's channels on average, every wave reached) vs the oracle on 16 host threads.
    shape = WORKLOADS["long_context_256k"]
    say("trapezoid full size: inputs", lam)
    d = make_scan_inputs(shape, "cuda")
    pv = make_prev_input(shape.batch, shape.d_inner, shape.d_state, shape.io, "cuda")
    lw = None if lam == "none" else make_trap_weight((1, shape.L, shape.d_inner), shape.io, "cuda", kind=lam)
    say("trapezoid full size: running", lam)
    y, hf = ssm.ssm_scan_fwd_trap(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], None,
                                  pv["x_prev"], pv["B_prev"], lam=lw)
    torch.cuda.synchronize()
    idx = sample_channels(shape.d_inner, 1024, seed=15)
    gc = lambda t: gather_channels(t, idx)
    say("trapezoid full size: oracle on", len(idx), "channels")
    X, DT, Z, A, Dv = gc(d["x"]), gc(d["dt"]), gc(d["z"]), d["A"].cpu()[idx], d["D"].cpu()[idx]
    B, C, XP, BP = d["B"].cpu(), d["C"].cpu(), gather_channels(pv["x_prev"], idx, axis=1), pv["B_prev"].cpu()
    LW = None if lw is None else gc(lw)
    yr, hr = threaded_channels(
        lambda sl: oracle.scan_trap(X[:, :, sl], DT[:, :, sl], A[sl], B, C, Dv[sl], Z[:, :, sl], None,
                                    x_prev=XP[:, sl], B_prev=BP, lam=None if LW is None else LW[:, :, sl]),
        len(idx))
    assert rel_err(gc(y), yr) <= TOL["bf16"], f"y error {rel_err(gc(y), yr)}"
    assert rel_err(hf.index_select(1, idx.cuda()).cpu(), hr) <= TOL["bf16"]
    assert torch.isfinite(y.float()).all()
