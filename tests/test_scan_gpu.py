"""Prefill (ssm_scan_fwd) on the GPU against the fp64 oracle, plus invariants.

Sizes are small enough for the oracle to finish in seconds but span several chunks,
several 64-lane waves and ragged tails (d_inner not a multiple of 64, L not a
multiple of the chunk length or of the 4-step register blocks, more than 64 chunks
so the carry scan walks several chunk tiles).
"""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_49_amd as ssm
from tests.gpu_util import TOL, bitwise_equal, rel_err, say, to_dev
from workloads import ScanShape, make_h0, make_scan_inputs, WORKLOADS

pytestmark = pytest.mark.gpu

# (batch, L, d_inner, d_state, io, gated, with_h0, chunk_len)
CASES = [
    (1, 64, 16, 4, "f32", True, False, 0),        # the tiny fp32 workload's shape
    (2, 300, 200, 16, "bf16", True, True, 64),    # 5 chunks, ragged last chunk
    (2, 300, 200, 16, "f32", False, True, 37),    # 9 chunks of odd length
    (1, 1000, 130, 8, "bf16", True, False, 0),    # library's own plan
    (2, 257, 70, 4, "f32", True, True, 50),
    (1, 203, 65, 2, "f32", True, True, 50),
    (3, 129, 64, 1, "f32", False, False, 16),
    (3, 129, 64, 16, "f32", True, True, 1000),    # one chunk
    (1, 1, 1, 1, "f32", True, True, 0),           # one step, one channel
    (1, 4501, 33, 16, "f32", True, True, 64),     # 71 chunks: two tiles of the carry scan
    (2, 777, 96, 16, "bf16", False, True, 5),     # chunks shorter than a register block
    (3, 129, 64, 1, "bf16", True, True, 16),      # bf16, N = 1, odd L: rows of B, C start at odd elements
]


def _ids(c):
    b, L, Dn, N, io, g, h0, T = c
    return f"b{b}_L{L}_D{Dn}_N{N}_{io}_{'gated' if g else 'nogate'}_{'h0' if h0 else 'zero'}_T{T}"


def _run(case, seed=0):
    b, L, Dn, N, io, gated, with_h0, T = case
    shape = ScanShape("case", b, L, Dn, N, io, gated=gated, seed=100 + seed)
    inp = make_scan_inputs(shape, "cpu")
    h0 = make_h0(b, Dn, N, seed=7 + seed) if with_h0 else None
    return shape, inp, h0


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_prefill_matches_oracle(case):
    shape, inp, h0 = _run(case)
    T = case[-1]
    say("prefill", _ids(case))
    d = to_dev(inp)
    y, hf = ssm.ssm_scan_fwd_ex(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"],
                                None if h0 is None else h0.cuda(), chunk_len=T)
    torch.cuda.synchronize()
    yr, hr = oracle.scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], h0)
    tol = TOL[shape.io]
    assert rel_err(y, yr) <= tol, f"y error {rel_err(y, yr)}"
    assert rel_err(hf, hr) <= tol, f"h_final error {rel_err(hf, hr)}"


def test_tiny_workload_uses_its_own_seeded_inputs():
    shape = WORKLOADS["tiny_f32"]
    inp = make_scan_inputs(shape, "cpu")
    say("tiny workload")
    d = to_dev(inp)
    y, hf = ssm.ssm_scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"])
    yr, hr = oracle.scan(**inp)
    assert rel_err(y, yr) <= TOL["f32"] and rel_err(hf, hr) <= TOL["f32"]


def test_chunk_length_does_not_change_results():
    case = (2, 600, 130, 16, "f32", True, True, 0)
    shape, inp, h0 = _run(case, seed=3)
    d = to_dev(inp)
    outs = []
    for T in (0, 7, 64, 600):
        say("chunk sweep", T)
        outs.append(ssm.ssm_scan_fwd_ex(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"],
                                        h0.cuda(), chunk_len=T))
    yr, hr = oracle.scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], h0)
    for y, hf in outs:
        assert rel_err(y, yr) <= TOL["f32"] and rel_err(hf, hr) <= TOL["f32"]


def test_deterministic_and_every_output_written():
    case = (2, 500, 100, 16, "bf16", True, True, 64)
    shape, inp, h0 = _run(case, seed=4)
    d = to_dev(inp)
    say("determinism")
    res = []
    for fill in (float("nan"), 0.0):
        y = torch.full_like(d["x"], fill)
        hf = torch.full((2, 100, 16), fill, device="cuda")
        ws = torch.full((ssm.ssm_scan_fwd_workspace_ex(2, 500, 100, 16, 64),), 255,
                        dtype=torch.uint8, device="cuda")
        ssm.ssm_scan_fwd_ex(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], h0.cuda(),
                            chunk_len=64, y=y, h_final=hf, workspace=ws)
        res.append((y, hf))
    assert torch.isfinite(res[0][0].float()).all() and torch.isfinite(res[0][1]).all()
    assert bitwise_equal(res[0][0], res[1][0]) and bitwise_equal(res[0][1], res[1][1])


def test_zero_length_and_empty_batch():
    h0 = make_h0(2, 40, 8).cuda()
    x = torch.empty((2, 0, 40), dtype=torch.float32, device="cuda")
    A = -torch.ones((40, 8), device="cuda")
    B = torch.empty((2, 0, 8), device="cuda")
    D = torch.ones(40, device="cuda")
    say("L=0")
    y, hf = ssm.ssm_scan_fwd(x, x, A, B, B, D, None, h0)
    torch.cuda.synchronize()
    assert bitwise_equal(hf, h0)
    y, hf = ssm.ssm_scan_fwd(x, x, A, B, B, D, None, None)
    torch.cuda.synchronize()
    assert torch.all(hf == 0)
    xe = torch.empty((0, 10, 40), device="cuda")
    y, hf = ssm.ssm_scan_fwd(xe, xe, A, torch.empty((0, 10, 8), device="cuda"),
                             torch.empty((0, 10, 8), device="cuda"), D)
    assert y.shape == (0, 10, 40) and hf.shape == (0, 40, 8)


def test_dt_zero_keeps_state_exactly():
    case = (2, 300, 70, 16, "f32", True, True, 64)
    shape, inp, h0 = _run(case, seed=5)
    inp["dt"] = torch.zeros_like(inp["dt"])
    d = to_dev(inp)
    say("dt=0")
    y, hf = ssm.ssm_scan_fwd_ex(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], h0.cuda(),
                                chunk_len=64)
    torch.cuda.synchronize()
    assert bitwise_equal(hf, h0.cuda()), "dt = 0 must leave the state bit for bit unchanged"
    yr, _ = oracle.scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], h0)
    assert rel_err(y, yr) <= TOL["f32"]


def test_nan_stays_in_its_channel():
    case = (2, 400, 130, 16, "f32", True, True, 64)
    shape, inp, h0 = _run(case, seed=6)
    d = to_dev(inp)
    say("nan isolation")
    y0, h_0 = ssm.ssm_scan_fwd_ex(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"],
                                  h0.cuda(), chunk_len=64)
    x = d["x"].clone()
    x[1, 100, 77] = float("nan")
    y1, h_1 = ssm.ssm_scan_fwd_ex(x, d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], h0.cuda(),
                                  chunk_len=64)
    torch.cuda.synchronize()
    mask = torch.ones(130, dtype=torch.bool)
    mask[77] = False
    assert bitwise_equal(y1[:, :, mask].contiguous(), y0[:, :, mask].contiguous())
    assert bitwise_equal(y1[0].contiguous(), y0[0].contiguous())
    assert bitwise_equal(h_1[:, mask].contiguous(), h_0[:, mask].contiguous())
    assert torch.isnan(y1[1, 100:, 77]).all() and torch.isfinite(y1[1, :100, 77]).all()


def test_split_and_resume_matches_whole():
    case = (2, 700, 96, 16, "f32", True, True, 64)
    shape, inp, h0 = _run(case, seed=8)
    d = to_dev(inp)
    say("split/resume")
    y, hf = ssm.ssm_scan_fwd_ex(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], h0.cuda(),
                                chunk_len=64)
    L1 = 333
    sl = lambda t, a, b: t[:, a:b].contiguous()
    ya, ha = ssm.ssm_scan_fwd_ex(sl(d["x"], 0, L1), sl(d["dt"], 0, L1), d["A"], sl(d["B"], 0, L1),
                                 sl(d["C"], 0, L1), d["D"], sl(d["z"], 0, L1), h0.cuda(), chunk_len=64)
    yb, hb = ssm.ssm_scan_fwd_ex(sl(d["x"], L1, 700), sl(d["dt"], L1, 700), d["A"],
                                 sl(d["B"], L1, 700), sl(d["C"], L1, 700), d["D"],
                                 sl(d["z"], L1, 700), ha, chunk_len=64)
    yr, hr = oracle.scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], h0)
    assert rel_err(torch.cat([ya, yb], 1), yr) <= TOL["f32"]
    assert rel_err(hb, hr) <= TOL["f32"] and rel_err(hf, hr) <= TOL["f32"]


def test_prefill_equals_decode_steps():
    case = (2, 50, 72, 16, "bf16", True, True, 16)
    shape, inp, h0 = _run(case, seed=9)
    d = to_dev(inp)
    say("prefill vs decode")
    y, hf = ssm.ssm_scan_fwd_ex(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], h0.cuda(),
                                chunk_len=16)
    h = h0.cuda().unsqueeze(0).contiguous()
    ys = []
    for t in range(50):
        col = lambda v: v[:, t].unsqueeze(0).contiguous()
        ys.append(ssm.ssm_step(h, col(d["x"]), col(d["dt"]), d["A"].unsqueeze(0).contiguous(),
                               col(d["B"]), col(d["C"]), d["D"].unsqueeze(0).contiguous(),
                               col(d["z"]))[0])
    yd = torch.stack(ys, 1)
    yr, hr = oracle.scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], h0)
    assert rel_err(y, yr) <= TOL["bf16"] and rel_err(yd, yr) <= TOL["bf16"]
    assert rel_err(h[0], hr) <= TOL["bf16"] and rel_err(hf, hr) <= TOL["bf16"]


def test_state_size_does_not_depend_on_length():
    for L in (1, 64, 4096):
        x = torch.zeros((1, L, 64), device="cuda")
        B = torch.zeros((1, L, 16), device="cuda")
        _, hf = ssm.ssm_scan_fwd(x, x, -torch.ones((64, 16), device="cuda"), B, B,
                                 torch.ones(64, device="cuda"))
        assert hf.shape == (1, 64, 16)


@pytest.mark.parametrize("variant", ["slow_decay", "frozen_states", "fast_decay", "dt_zero_block"])
def test_decay_horizon_edge_cases(variant):
    # The chunk summaries walk back only to the point where every state of a wave has
    # decayed below 2^-H (H = 28 + the bit length of the chunk length); these inputs make
    # that point come early, late or never.
    shape = ScanShape("h", 1, 3000, 130, 16, "f32", seed=61)
    inp = make_scan_inputs(shape, "cpu")
    if variant == "slow_decay":
        inp["A"] = inp["A"] * 1e-3                      # never within one chunk
    elif variant == "frozen_states":
        inp["A"][5] = 0.0                                # one channel never decays
        inp["A"][70, 3] = 0.0                            # one state of another wave
    elif variant == "fast_decay":
        inp["dt"] = inp["dt"] * 20.0                     # horizon within a few steps
    elif variant == "dt_zero_block":
        inp["dt"][:, 400:1400] = 0.0                     # no decay across a whole chunk
    h0 = make_h0(1, 130, 16, seed=62)
    d = to_dev(inp)
    say("horizon", variant)
    y, hf = ssm.ssm_scan_fwd_ex(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], h0.cuda(),
                                chunk_len=500)
    torch.cuda.synchronize()
    yr, hr = oracle.scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], h0)
    assert rel_err(y, yr) <= TOL["f32"], f"y error {rel_err(y, yr)}"
    assert rel_err(hf, hr) <= TOL["f32"], f"h_final error {rel_err(hf, hr)}"


def test_prefill_in_captured_graph_matches_eager():
    # A multi-chunk prefill (summaries, carry, rescan) with its workspace and outputs
    # allocated beforehand, captured in a graph and replayed several times with eager
    # prefills and synchronisation between replays: every replay equals the eager call
    # bit for bit (the library enqueues kernels only: no allocation, no memset nodes).
    shape = ScanShape("graph", 2, 700, 130, 16, "bf16", gated=True, seed=77)
    g = to_dev(make_scan_inputs(shape, "cpu"))
    h0 = make_h0(2, 130, 16).cuda()
    T = 64  # 11 chunks
    args = (g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["z"], h0)
    y_e, h_e = ssm.ssm_scan_fwd_ex(*args, chunk_len=T)
    torch.cuda.synchronize()
    ws = torch.empty(ssm.ssm_scan_fwd_workspace_ex(2, 700, 130, 16, T), dtype=torch.uint8, device="cuda")
    y_g, h_g = torch.empty_like(y_e), torch.empty_like(h_e)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            ssm.ssm_scan_fwd_ex(*args, chunk_len=T, y=y_g, h_final=h_g, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        say("prefill graph replay", rep)
        y_g.zero_()
        h_g.zero_()
        ws.fill_(0xAB)  # stale workspace contents must not matter
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert bitwise_equal(y_g, y_e) and bitwise_equal(h_g, h_e), f"replay {rep} differs"
        ssm.ssm_scan_fwd_ex(*args, chunk_len=T)   # eager work between replays
        torch.cuda.synchronize()


def test_chunk_plan_uses_the_device_cu_count():
    # The planner queries the current device's compute units once and plans 5 rescan
    # waves per SIMD (4 SIMDs per CU) for the plain prefill: on MI355X (256 CUs) the 256k
    # workload's 128 channel waves per chunk make 40 chunks, as before the query existed.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    say("chunk plan on", cus, "CUs")
    T = ssm.ssm_scan_fwd_chunk_len(1, 262144, 8192, 16)
    n = -(-262144 // T)
    assert n == -(-5 * 4 * cus // 128), (cus, n)
    if cus == 256:
        assert n == 40
