"""Decode (ssm_step, ssm_step_c64) on the GPU: bit for bit against the reference-order
replay kernels, and within tolerance of the fp64 oracle over several steps."""
import pytest
import torch

import oracle
import selective_state_space_49_amd as ssm
from tests.gpu_util import TOL, bitwise_equal, rel_err, say
from workloads import DecodeShape, make_decode_params, make_decode_step

pytestmark = pytest.mark.gpu

# (n_layers, n_seq, d_inner, d_state, io, gated, complex)
CASES = [
    (3, 5, 130, 16, "bf16", True, False),
    (2, 4, 64, 16, "f32", False, False),
    (2, 3, 77, 8, "f32", True, False),
    (1, 7, 33, 4, "bf16", True, False),
    (2, 2, 40, 2, "f32", True, False),
    (2, 2, 40, 1, "bf16", False, False),
    (3, 5, 130, 16, "bf16", False, True),
    (2, 3, 50, 16, "f32", True, True),
    (2, 2, 31, 4, "f32", False, True),
    (1, 3, 20, 2, "bf16", True, True),
    (1, 3, 20, 1, "f32", False, True),
]
STEPS = 6


def _ids(c):
    Ln, S, Dn, N, io, g, cx = c
    return f"L{Ln}_S{S}_D{Dn}_N{N}_{io}_{'gated' if g else 'nogate'}{'_complex' if cx else ''}"


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_step_bitwise_replay_and_oracle(case):
    Ln, S, Dn, N, io, gated, cx = case
    shape = DecodeShape("case", Ln, S, Dn, N, STEPS, io, gated=gated, complex_state=cx, seed=300)
    par = make_decode_params(shape, "cpu")
    ext = (2,) if cx else ()
    h0 = torch.randn((Ln, S, Dn, N) + ext, generator=torch.Generator().manual_seed(5))
    h_fast = h0.cuda()
    h_rep = h0.cuda()
    h_ref = h0.double().numpy()
    A, D = par["A"].cuda(), par["D"].cuda()
    fast = ssm.ssm_step_c64 if cx else ssm.ssm_step
    rep = ssm.ssm_step_c64_replay if cx else ssm.ssm_step_replay
    ostep = oracle.step_complex if cx else oracle.step
    for k in range(STEPS):
        inp = make_decode_step(shape, k, "cpu")
        d = {n: (None if v is None else v.cuda()) for n, v in inp.items()}
        say("decode", _ids(case), "step", k)
        y1 = fast(h_fast, d["x"], d["dt"], A, d["B"], d["C"], D, d["z"])
        y2 = rep(h_rep, d["x"], d["dt"], A, d["B"], d["C"], D, d["z"])
        torch.cuda.synchronize()
        assert bitwise_equal(y1, y2), f"y differs from replay at step {k}"
        assert bitwise_equal(h_fast, h_rep), f"state differs from replay at step {k}"
        yr, h_ref = ostep(h_ref, inp["x"], inp["dt"], par["A"], inp["B"], inp["C"], par["D"], inp["z"])
        assert rel_err(y1, yr) <= TOL[io], f"y vs oracle {rel_err(y1, yr)} at step {k}"
        assert rel_err(h_fast, h_ref) <= TOL[io], f"h vs oracle at step {k}"


def test_step_is_deterministic_and_in_place():
    shape = DecodeShape("det", 2, 8, 256, 16, 1, "bf16", seed=9)
    par = make_decode_params(shape, "cuda")
    inp = make_decode_step(shape, 0, "cuda")
    h0 = torch.randn((2, 8, 256, 16), device="cuda")
    outs = []
    for _ in range(2):
        h = h0.clone()
        ptr = h.data_ptr()
        say("decode determinism")
        y = ssm.ssm_step(h, inp["x"], inp["dt"], par["A"], inp["B"], inp["C"], par["D"], inp["z"])
        assert h.data_ptr() == ptr
        outs.append((y, h))
    torch.cuda.synchronize()
    assert bitwise_equal(outs[0][0], outs[1][0]) and bitwise_equal(outs[0][1], outs[1][1])
    assert not bitwise_equal(outs[0][1], h0)


def test_state_survives_a_host_round_trip():
    # The state is the whole checkpoint: copy it out, free it, restore, continue.
    shape = DecodeShape("ckpt", 2, 4, 96, 16, 4, "bf16", seed=12)
    par = make_decode_params(shape, "cuda")
    steps = [make_decode_step(shape, k, "cuda") for k in range(4)]
    h_a = torch.zeros((2, 4, 96, 16), device="cuda")
    h_b = torch.zeros((2, 4, 96, 16), device="cuda")
    ya, yb = [], []
    for k, s in enumerate(steps):
        say("checkpoint step", k)
        ya.append(ssm.ssm_step(h_a, s["x"], s["dt"], par["A"], s["B"], s["C"], par["D"], s["z"]))
        if k == 2:
            host = h_b.cpu()
            del h_b
            torch.cuda.synchronize()
            h_b = host.cuda()
        yb.append(ssm.ssm_step(h_b, s["x"], s["dt"], par["A"], s["B"], s["C"], par["D"], s["z"]))
    torch.cuda.synchronize()
    assert all(bitwise_equal(a, b) for a, b in zip(ya, yb)) and bitwise_equal(h_a, h_b)


def test_decode_in_captured_graph_matches_eager():
    # A captured graph of per-layer ssm_step calls, replayed several times with eager
    # work and synchronisation between replays: every replay must equal the eager run
    # bit for bit (the calls enqueue kernels only; no memset nodes).
    shape = DecodeShape("graph", 3, 4, 192, 16, 1, "bf16", seed=31)
    par = make_decode_params(shape, "cuda")
    tok = make_decode_step(shape, 0, "cuda")
    h0 = torch.randn((3, 4, 192, 16), device="cuda")
    layers = lambda h, y: [ssm.ssm_step(h[l:l + 1], tok["x"][l:l + 1], tok["dt"][l:l + 1],
                                        par["A"][l:l + 1], tok["B"][l:l + 1], tok["C"][l:l + 1],
                                        par["D"][l:l + 1], tok["z"][l:l + 1], y_t=y[l:l + 1])
                           for l in range(3)]
    h_e, y_e = h0.clone(), torch.empty_like(tok["x"])
    layers(h_e, y_e)
    torch.cuda.synchronize()
    h_g, y_g = h0.clone(), torch.empty_like(tok["x"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            layers(h_g, y_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        say("graph replay", rep)
        h_g.copy_(h0)
        y_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert bitwise_equal(y_g, y_e) and bitwise_equal(h_g, h_e), f"replay {rep} differs"
        layers(h0.clone(), torch.empty_like(y_e))   # eager work between replays
        torch.cuda.synchronize()
