"""The fused MambaBlock input stage (causal depthwise conv + silu on x, softplus on
dt) on the GPU, against the fp64 oracle's scan_fused / step_fused.

Prefill: y and h_final within the tolerance of the plain scan, the carried conv
state bit for bit (it is a copy of inputs). Decode: bit for bit against the replay
kernel, within tolerance of the oracle over several steps, the conv state bit for
bit. Plus the properties that hold at any size: chunking does not change the result,
a sequence split in two with both states carried equals one call, prefill equals
decode, a NaN stays in its channel, and softplus itself is accurate to a few ulp.
"""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_49_amd as ssm
from tests.gpu_util import TOL, bitwise_equal, gather_channels, rel_err, say, to_dev
from workloads import (WORKLOADS, DecodeShape, ScanShape, make_decode_dt_raw,
                       make_decode_input_stage, make_decode_params, make_decode_step, make_h0,
                       make_input_stage, make_scan_inputs, sample_channels)

pytestmark = pytest.mark.gpu

# (batch, L, d_inner, d_state, io, gated, K, chunk_len, with_h0, with_state)
CASES = [
    (2, 300, 130, 16, "bf16", True, 4, 64, True, True),    # several chunks, ragged L and channels
    (1, 257, 64, 16, "f32", True, 4, 32, True, True),
    (2, 100, 33, 8, "f32", False, 3, 16, False, True),
    (1, 150, 40, 4, "bf16", True, 2, 0, True, False),      # library's own chunk plan, zero padding
    (1, 70, 20, 1, "f32", True, 1, 16, True, False),       # one tap: no carried state
    (2, 64, 48, 16, "bf16", True, 0, 16, True, False),     # softplus only, x as is
    (1, 2, 16, 16, "f32", True, 4, 1, True, True),         # L < K-1: the state out mixes old rows
    (3, 1000, 70, 16, "f32", True, 4, 128, True, True),
    (3, 131, 40, 1, "bf16", True, 4, 32, True, True),     # bf16, N = 1, odd L
]


def _ids(c):
    b, L, Dn, N, io, g, K, T, h0, st = c
    return f"b{b}_L{L}_D{Dn}_N{N}_{io}_{'gated' if g else 'nogate'}_K{K}_T{T}{'_h0' if h0 else ''}{'_s0' if st else ''}"


def _draw(case, seed=400):
    b, L, Dn, N, io, gated, K, T, with_h0, with_state = case
    shape = ScanShape("fused", b, L, Dn, N, io, gated=gated, seed=seed)
    d = make_scan_inputs(shape, "cpu")
    s = make_input_stage(shape, K, "cpu", with_state=with_state)
    h0 = make_h0(b, Dn, N) if with_h0 else None
    return shape, d, s, h0


def _oracle(d, s, h0, K):
    if K == 0:   # softplus only: the plain scan of x with the oracle's softplus step
        y, hf = oracle.scan(d["x"], oracle.softplus(s["dt_raw"], s["dt_bias"]), d["A"], d["B"],
                            d["C"], d["D"], d["z"], h0)
        return y, hf, None
    return oracle.scan_fused(d["x"], s["dt_raw"], d["A"], d["B"], d["C"], d["D"], d["z"], h0,
                             conv_w=s["conv_w"], conv_b=s["conv_b"], conv_state0=s["conv_state0"],
                             dt_bias=s["dt_bias"])


def _run(d, s, h0, K, chunk_len, **kw):
    g = to_dev(d)
    gs = to_dev(s)
    return ssm.ssm_scan_fwd_fused(g["x"], gs["dt_raw"], g["A"], g["B"], g["C"], g["D"], g["z"],
                                  None if h0 is None else h0.cuda(), conv_w=gs["conv_w"],
                                  conv_b=gs["conv_b"], conv_state0=gs["conv_state0"],
                                  dt_bias=gs["dt_bias"], chunk_len=chunk_len, **kw)


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_fused_prefill_matches_oracle(case):
    shape, d, s, h0 = _draw(case)
    K, T = case[6], case[7]
    say("fused prefill", _ids(case))
    y, hf, so = _run(d, s, h0, K, T)
    torch.cuda.synchronize()
    yr, hr, sr = _oracle(d, s, h0, K)
    tol = TOL[shape.io]
    assert rel_err(y, yr) <= tol, f"y error {rel_err(y, yr)}"
    assert rel_err(hf, hr) <= tol, f"h_final error {rel_err(hf, hr)}"
    if K > 1:
        assert np.array_equal(oracle.to_f64(so), sr), "conv state out"
    else:
        assert so is None


def test_fused_chunking_and_split_resume():
    # chunk plans agree; two calls with (h_final, conv state) carried equal one call
    case = (2, 480, 96, 16, "f32", True, 4, 0, True, True)
    shape, d, s, h0 = _draw(case, seed=410)
    say("fused chunking")
    outs = [_run(d, s, h0, 4, T) for T in (0, 480, 37, 64)]
    torch.cuda.synchronize()
    for y, hf, so in outs[1:]:
        assert rel_err(y, outs[0][0].cpu()) <= TOL["f32"] and rel_err(hf, outs[0][1].cpu()) <= TOL["f32"]
        assert bitwise_equal(so, outs[0][2])
    L1 = 203
    cut = lambda t, a, b: None if t is None else t[:, a:b].contiguous()
    d1 = {k: (cut(v, 0, L1) if k in ("x", "z", "B", "C", "dt") else v) for k, v in d.items()}
    d2 = {k: (cut(v, L1, 480) if k in ("x", "z", "B", "C", "dt") else v) for k, v in d.items()}
    s1 = dict(s, dt_raw=cut(s["dt_raw"], 0, L1))
    say("fused split part 1")
    y1, hf1, so1 = _run(d1, s1, h0, 4, 64)
    s2 = dict(s, dt_raw=cut(s["dt_raw"], L1, 480), conv_state0=so1.cpu())
    say("fused split part 2")
    y2, hf2, so2 = _run(d2, s2, hf1.cpu(), 4, 64)
    torch.cuda.synchronize()
    y_all, hf_all, so_all = outs[0]
    assert rel_err(torch.cat([y1, y2], 1), y_all.cpu()) <= TOL["f32"]
    assert rel_err(hf2, hf_all.cpu()) <= TOL["f32"]
    assert bitwise_equal(so2, so_all)


def test_fused_empty_sequence_passes_states_through():
    shape = ScanShape("empty", 2, 0, 40, 16, "bf16", seed=420)
    d = to_dev(make_scan_inputs(shape, "cpu"))
    s = to_dev(make_input_stage(shape, 4, "cpu"))
    h0 = make_h0(2, 40, 16).cuda()
    say("fused L = 0")
    y, hf, so = ssm.ssm_scan_fwd_fused(d["x"], s["dt_raw"], d["A"], d["B"], d["C"], d["D"], d["z"],
                                       h0, conv_w=s["conv_w"], conv_b=s["conv_b"],
                                       conv_state0=s["conv_state0"], dt_bias=s["dt_bias"])
    torch.cuda.synchronize()
    assert y.numel() == 0 and bitwise_equal(hf, h0) and bitwise_equal(so, s["conv_state0"])
    y, hf, so = ssm.ssm_scan_fwd_fused(d["x"], s["dt_raw"], d["A"], d["B"], d["C"], d["D"], d["z"],
                                       None, conv_w=s["conv_w"])
    torch.cuda.synchronize()
    assert not hf.any() and not so.float().any()


def test_fused_nan_stays_in_its_channel_and_window():
    # A NaN input of channel 5 at step 100 reaches that channel's outputs from step 100
    # on (through u_100..u_103 and the state) and no other channel.
    case = (1, 256, 64, 16, "f32", True, 4, 32, True, True)
    shape, d, s, h0 = _draw(case, seed=430)
    say("fused NaN isolation, clean")
    y0, hf0, so0 = _run(d, s, h0, 4, 32)
    x = d["x"].clone()
    x[0, 100, 5] = float("nan")
    say("fused NaN isolation, poisoned")
    y1, hf1, so1 = _run(dict(d, x=x), s, h0, 4, 32)
    torch.cuda.synchronize()
    other = [c for c in range(64) if c != 5]
    assert bitwise_equal(y1[:, :, other], y0[:, :, other])
    assert bitwise_equal(y1[:, :100, 5], y0[:, :100, 5])
    assert torch.isnan(y1[0, 100:104, 5]).all()
    assert bitwise_equal(so1, so0)


def test_fused_softplus_accuracy():
    # With no convolution, x = B = C = 1, D = 0, A = -1, N = 1, L = 1 and no gate, the
    # output is exactly the kernel's dt (every product and fma on the way is exact), so
    # y shows softplus itself. Bound: 8 ulp, plus the rounding of the exponent
    # argument -|v| log2(e) (half an ulp of a number near 1.44 |v|, i.e. a relative
    # error up to |v| 2^-24 ln 2 log2(e) = |v| 2^-24 in e^-|v|), or 1e-37 absolute
    # below the normal range.
    v = torch.cat([torch.linspace(-100.0, 100.0, 4001), torch.tensor([0.0, -0.0, 1e-8, -1e-8, 20.0, 88.0, -88.0])])
    Dn = v.numel()
    one = lambda *s: torch.ones(*s, device="cuda")
    dt_raw = v.view(1, 1, Dn).cuda()
    say("softplus accuracy")
    y, _, _ = ssm.ssm_scan_fwd_fused(one(1, 1, Dn), dt_raw, -one(Dn, 1), one(1, 1, 1), one(1, 1, 1),
                                     torch.zeros(Dn, device="cuda"), None, None)
    torch.cuda.synchronize()
    ref = oracle.softplus(v.double().numpy())
    got = oracle.to_f64(y).reshape(-1)
    err = np.abs(got - ref)
    bound = np.abs(ref) * (8 * 2.0 ** -23 + np.abs(v.double().numpy()) * 2.0 ** -24)
    ok = (err <= bound) | (err <= 1e-37)
    assert ok.all(), f"softplus off at {v[~torch.from_numpy(ok)][:8].tolist()}"
    special = ssm.ssm_scan_fwd_fused(one(1, 1, 3), torch.tensor([[[float("inf"), -float("inf"), float("nan")]]], device="cuda"),
                                     -one(3, 1), one(1, 1, 1), one(1, 1, 1), torch.zeros(3, device="cuda"))[0]
    torch.cuda.synchronize()
    assert special[0, 0, 0] == float("inf") and special[0, 0, 1] == 0.0 and torch.isnan(special[0, 0, 2])


# ---------------------------------------------------------------- decode
# (n_layers, n_seq, d_inner, d_state, io, gated, K)
DECODE_CASES = [
    (3, 5, 130, 16, "bf16", True, 4),
    (2, 4, 64, 16, "f32", False, 4),
    (2, 3, 77, 8, "f32", True, 3),
    (1, 7, 33, 4, "bf16", True, 2),
    (2, 2, 40, 2, "f32", True, 1),
    (2, 2, 40, 16, "bf16", True, 0),
    (1, 2, 600, 16, "bf16", True, 4),   # three blocks of 256 channels, the last ragged
]
STEPS = 6


def _dids(c):
    Ln, S, Dn, N, io, g, K = c
    return f"L{Ln}_S{S}_D{Dn}_N{N}_{io}_{'gated' if g else 'nogate'}_K{K}"


@pytest.mark.parametrize("case", DECODE_CASES, ids=_dids)
def test_fused_step_bitwise_replay_and_oracle(case):
    Ln, S, Dn, N, io, gated, K = case
    shape = DecodeShape("fused", Ln, S, Dn, N, STEPS, io, gated=gated, seed=440)
    par = make_decode_params(shape, "cpu")
    ist = make_decode_input_stage(shape, K, "cpu")
    h0 = torch.randn((Ln, S, Dn, N), generator=torch.Generator().manual_seed(6))
    h_fast, h_rep, h_ref = h0.cuda(), h0.cuda(), h0.double().numpy()
    cs0 = ist["conv_state"]
    cs_fast = None if cs0 is None else cs0.cuda()
    cs_rep = None if cs0 is None else cs0.cuda()
    cs_ref = oracle.to_f64(cs0) if cs0 is not None else np.zeros((Ln, S, max(K - 1, 0), Dn))
    A, D = par["A"].cuda(), par["D"].cuda()
    gi = to_dev({k: v for k, v in ist.items() if k != "conv_state"})
    for k in range(STEPS):
        inp = make_decode_step(shape, k, "cpu")
        dtr = make_decode_dt_raw(shape, k, "cpu")
        g = to_dev(inp)
        say("fused decode", _dids(case), "step", k)
        kw = dict(conv_w=gi["conv_w"], conv_b=gi["conv_b"], dt_bias=gi["dt_bias"])
        y1 = ssm.ssm_step_fused(h_fast, cs_fast, g["x"], dtr.cuda(), A, g["B"], g["C"], D, g["z"], **kw)
        y2 = ssm.ssm_step_fused_replay(h_rep, cs_rep, g["x"], dtr.cuda(), A, g["B"], g["C"], D, g["z"], **kw)
        torch.cuda.synchronize()
        assert bitwise_equal(y1, y2), f"y differs from replay at step {k}"
        assert bitwise_equal(h_fast, h_rep), f"state differs from replay at step {k}"
        if cs_fast is not None:
            assert bitwise_equal(cs_fast, cs_rep), f"conv state differs from replay at step {k}"
        if K:
            yr, h_ref, cs_ref = oracle.step_fused(h_ref, cs_ref, inp["x"], dtr, par["A"], inp["B"],
                                                  inp["C"], par["D"], inp["z"], conv_w=ist["conv_w"],
                                                  conv_b=ist["conv_b"], dt_bias=ist["dt_bias"])
        else:
            dts = np.stack([oracle.softplus(dtr[l], ist["dt_bias"][l]) for l in range(Ln)])
            yr, h_ref = oracle.step(h_ref, inp["x"], dts, par["A"], inp["B"], inp["C"], par["D"],
                                    inp["z"])
        assert rel_err(y1, yr) <= TOL[io], f"y vs oracle {rel_err(y1, yr)} at step {k}"
        assert rel_err(h_fast, h_ref) <= TOL[io], f"h vs oracle at step {k}"
        if K > 1:
            assert np.array_equal(oracle.to_f64(cs_fast), cs_ref), f"conv state vs oracle at step {k}"


def test_fused_prefill_equals_decode():
    # L decode steps (one layer, n_seq = batch) against one prefill of the same tokens.
    b, L, Dn, N, K = 3, 40, 96, 16, 4
    shape = ScanShape("pd", b, L, Dn, N, "f32", seed=450)
    d = make_scan_inputs(shape, "cpu")
    s = make_input_stage(shape, K, "cpu")
    h0 = make_h0(b, Dn, N)
    say("fused prefill vs decode: prefill")
    y, hf, so = _run(d, s, h0, K, 16)
    h = h0.view(1, b, Dn, N).cuda().contiguous()
    cs = s["conv_state0"].view(1, b, K - 1, Dn).cuda().contiguous()
    g = to_dev(d)
    gs = to_dev(s)
    ys = []
    for t in range(L):
        row = lambda v: v[:, t].unsqueeze(0).contiguous()
        ys.append(ssm.ssm_step_fused(h, cs, row(g["x"]), row(gs["dt_raw"]), g["A"].unsqueeze(0),
                                     row(g["B"]), row(g["C"]), g["D"].unsqueeze(0), row(g["z"]),
                                     conv_w=gs["conv_w"].unsqueeze(0), conv_b=gs["conv_b"].unsqueeze(0),
                                     dt_bias=gs["dt_bias"].unsqueeze(0))[0])
    say("fused prefill vs decode: compare")
    torch.cuda.synchronize()
    yd = torch.stack(ys, dim=1)
    assert rel_err(yd, oracle.to_f64(y)) <= TOL["f32"]
    assert rel_err(h[0], oracle.to_f64(hf)) <= TOL["f32"]
    assert bitwise_equal(cs[0], so)


@pytest.mark.parametrize("name,k", [("jamba_layer_prefill", 128), ("long_context_256k", 24)])
def test_fused_full_size_sampled(name, k):
    # The Jamba-shaped layer (batch 2, L 4096) and the 256k prefill (batch 1, L 262144),
    # 8192 channels, N 16, bf16, through the fused entry point in the library's own chunk
    # plan (the configuration the benchmark times); sampled channels vs the oracle.
    shape = WORKLOADS[name]
    say("fused full size:", name, "generating inputs")
    d = make_scan_inputs(shape, "cuda")
    s = make_input_stage(shape, 4, "cuda")
    say("fused full size: running")
    y, hf, so = ssm.ssm_scan_fwd_fused(d["x"], s["dt_raw"], d["A"], d["B"], d["C"], d["D"], d["z"],
                                       conv_w=s["conv_w"], conv_b=s["conv_b"],
                                       conv_state0=s["conv_state0"], dt_bias=s["dt_bias"])
    torch.cuda.synchronize()
    idx = sample_channels(shape.d_inner, k, seed=9)
    g = lambda t: gather_channels(t, idx)
    say("fused full size: oracle on", len(idx), "channels")
    yr, hr, sr = oracle.scan_fused(g(d["x"]), g(s["dt_raw"]), d["A"].cpu()[idx], d["B"].cpu(),
                                   d["C"].cpu(), d["D"].cpu()[idx], g(d["z"]),
                                   conv_w=s["conv_w"].cpu()[idx], conv_b=s["conv_b"].cpu()[idx],
                                   conv_state0=g(s["conv_state0"]), dt_bias=s["dt_bias"].cpu()[idx])
    assert rel_err(g(y), yr) <= TOL["bf16"], f"y error {rel_err(g(y), yr)}"
    assert rel_err(hf.index_select(1, idx.cuda()).cpu(), hr) <= TOL["bf16"]
    assert np.array_equal(oracle.to_f64(g(so)), sr)
    assert torch.isfinite(y.float()).all()
