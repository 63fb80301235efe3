"""Complex-state prefill (ssm_scan_fwd_c64) on the GPU against the fp64 oracle."""
import math

import pytest
import torch

import oracle
import selective_state_space_49_amd as ssm
from tests.gpu_util import TOL, rel_err, say, to_dev
from workloads import ScanShape, make_h0, make_scan_inputs

pytestmark = pytest.mark.gpu

# (batch, L, d_inner, d_state, io, gated, with_h0, chunk_len)
CASES = [
    (1, 64, 16, 4, "f32", False, False, 0),
    (2, 300, 100, 16, "bf16", False, True, 64),
    (2, 300, 100, 16, "f32", True, True, 37),
    (1, 500, 70, 8, "f32", False, False, 0),
    (2, 129, 65, 2, "bf16", True, True, 16),
    (1, 77, 3, 1, "f32", False, True, 8),
    (1, 4300, 16, 4, "f32", False, True, 64),   # 68 chunks: two carry tiles
    (2, 1500, 300, 16, "bf16", True, True, 0),  # library's plan; 64-channel blocks, the last ragged
    (1, 203, 130, 16, "f32", False, True, 50),  # ragged blocks of 4-step rows
]


def _ids(c):
    b, L, Dn, N, io, g, h0, T = c
    return f"b{b}_L{L}_D{Dn}_N{N}_{io}_{'gated' if g else 'nogate'}_{'h0' if h0 else 'zero'}_T{T}"


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_complex_prefill_matches_oracle(case):
    b, L, Dn, N, io, gated, with_h0, T = case
    shape = ScanShape("c", b, L, Dn, N, io, complex_state=True, gated=gated, seed=500)
    inp = make_scan_inputs(shape, "cpu")
    h0 = make_h0(b, Dn, N, complex_state=True, seed=3) if with_h0 else None
    d = to_dev(inp)
    say("complex prefill", _ids(case))
    y, hf = ssm.ssm_scan_fwd_c64(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"],
                                 None if h0 is None else h0.cuda(), chunk_len=T)
    torch.cuda.synchronize()
    yr, hr = oracle.scan_complex(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                                 inp["z"], h0)
    assert rel_err(y, yr) <= TOL[io], f"y error {rel_err(y, yr)}"
    assert rel_err(hf, hr) <= TOL[io], f"h_final error {rel_err(hf, hr)}"


def test_zero_angle_matches_real_kernel():
    shape = ScanShape("r", 2, 300, 100, 16, "f32", seed=77)
    inp = make_scan_inputs(shape, "cpu")
    d = to_dev(inp)
    say("theta=0 vs real")
    yr, hr = ssm.ssm_scan_fwd_ex(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], chunk_len=64)
    A2 = torch.stack([d["A"], torch.zeros_like(d["A"])], -1).contiguous()
    B2 = torch.stack([d["B"], torch.zeros_like(d["B"])], -1).contiguous()
    C2 = torch.stack([d["C"], torch.zeros_like(d["C"])], -1).contiguous()
    yc, hc = ssm.ssm_scan_fwd_c64(d["x"], d["dt"], A2, B2, C2, d["D"], d["z"], chunk_len=64)
    torch.cuda.synchronize()
    assert rel_err(yc, yr.cpu().double().numpy()) <= 1e-6
    assert rel_err(hc[..., 0], hr.cpu().double().numpy()) <= 1e-6
    assert float(hc[..., 1].abs().max()) == 0.0


def test_pure_rotation_impulse_response():
    # No decay, dt = 1, unit impulse, B = 1: y_t = Re(h_t[n]) = cos(theta_n t).
    L, N = 200, 4
    theta = torch.tensor([0.3, -1.1, 2.5, math.pi / 7])
    A = torch.stack([torch.zeros(N), theta], -1).view(1, N, 2).cuda()
    x = torch.zeros((1, L, 1)); x[0, 0, 0] = 1.0
    B = torch.zeros((1, L, N, 2)); B[..., 0] = 1.0
    for n in range(N):
        C = torch.zeros((1, L, N, 2)); C[:, :, n, 0] = 1.0
        say("rotation", n)
        y, _ = ssm.ssm_scan_fwd_c64(x.cuda(), torch.ones((1, L, 1), device="cuda"), A, B.cuda(),
                                    C.cuda(), torch.zeros(1, device="cuda"), chunk_len=64)
        ref = torch.cos(theta[n].double() * torch.arange(L, dtype=torch.float64))
        assert rel_err(y, ref.view(1, L, 1).numpy()) <= 1e-4


@pytest.mark.parametrize("variant", ["slow_decay", "frozen_states", "fast_decay"])
def test_complex_decay_horizon_edge_cases(variant):
    shape = ScanShape("hc", 1, 2000, 70, 16, "f32", complex_state=True, gated=False, seed=63)
    inp = make_scan_inputs(shape, "cpu")
    if variant == "slow_decay":
        inp["A"][..., 0] = inp["A"][..., 0] * 1e-3
    elif variant == "frozen_states":
        inp["A"][5, :, 0] = 0.0                          # a pure rotation channel
        inp["A"][66, 2, 0] = 0.0
    elif variant == "fast_decay":
        inp["dt"] = inp["dt"] * 20.0
    h0 = make_h0(1, 70, 16, complex_state=True, seed=64)
    d = to_dev(inp)
    say("complex horizon", variant)
    y, hf = ssm.ssm_scan_fwd_c64(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], h0.cuda(),
                                 chunk_len=300)
    torch.cuda.synchronize()
    yr, hr = oracle.scan_complex(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                                 inp["z"], h0)
    assert rel_err(y, yr) <= TOL["f32"], f"y error {rel_err(y, yr)}"
    assert rel_err(hf, hr) <= TOL["f32"], f"h_final error {rel_err(hf, hr)}"
