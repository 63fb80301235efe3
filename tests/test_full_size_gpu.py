"""The four large workloads at full size, in the launch configuration the benchmark
times (the library's own chunk plan), checked on sampled channels.

Channels are independent, so the oracle run on a subset of channels over the full
sequence is exact for those channels. Inputs are drawn on the GPU with a seeded
generator; the sampled channels are copied to the host for the oracle.
"""
import pytest
import torch

import oracle
import selective_state_space_49_amd as ssm
from tests.gpu_util import TOL, bitwise_equal, gather_channels, rel_err, say
from workloads import (WORKLOADS, make_decode_params, make_decode_step, make_scan_inputs,
                       sample_channels)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,k", [("jamba_layer_prefill", 256), ("long_context_256k", 24),
                                    ("complex_rotation", 48)])
def test_full_size_prefill_sampled(name, k):
    shape = WORKLOADS[name]
    say("full-size prefill", name, "generating inputs")
    d = make_scan_inputs(shape, "cuda")
    torch.cuda.synchronize()
    fn = ssm.ssm_scan_fwd_c64 if shape.complex_state else ssm.ssm_scan_fwd
    say("full-size prefill", name, "running")
    y, hf = fn(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"])
    torch.cuda.synchronize()
    idx = sample_channels(shape.d_inner, k, seed=5)
    g = lambda t: gather_channels(t, idx)
    ora = oracle.scan_complex if shape.complex_state else oracle.scan
    say("full-size prefill", name, "oracle on", len(idx), "channels")
    yr, hr = ora(g(d["x"]), g(d["dt"]), d["A"].cpu()[idx], d["B"].cpu(), d["C"].cpu(),
                 d["D"].cpu()[idx], g(d["z"]))
    tol = TOL[shape.io]
    assert rel_err(g(y), yr) <= tol, f"y error {rel_err(g(y), yr)}"
    assert rel_err(hf.index_select(1, idx.cuda()).cpu(), hr) <= tol
    assert torch.isfinite(y.float()).all()


def test_full_size_batched_decode_512_steps():
    shape = WORKLOADS["batched_decode"]
    Ln, S, Dn, N = shape.n_layers, shape.n_seq, shape.d_inner, shape.d_state
    par = make_decode_params(shape, "cuda")
    h = torch.zeros((Ln, S, Dn, N), device="cuda")
    h_rep = torch.zeros_like(h)
    # 4096 sampled (layer, sequence, channel) triples, followed through every step
    g = torch.Generator().manual_seed(21)
    flat = torch.randperm(Ln * S * Dn, generator=g)[:4096]
    li, si, di = flat // (S * Dn), (flat // Dn) % S, flat % Dn
    D_s = par["D"].cpu()[li, di].view(1, 1, -1)
    A_s = par["A"].cpu()[li, di].view(1, 4096, N)
    h_ref = torch.zeros((1, 1, 4096, N), dtype=torch.float64).numpy()
    lic, sic, dic = li.cuda(), si.cuda(), di.cuda()
    compare_at = {0, 255, 511}
    for k in range(shape.steps):
        inp = make_decode_step(shape, k, "cuda")
        if k % 64 == 0:
            say("decode full size, step", k)
        y = ssm.ssm_step(h, inp["x"], inp["dt"], par["A"], inp["B"], inp["C"], par["D"], inp["z"])
        y_rep = ssm.ssm_step_replay(h_rep, inp["x"], inp["dt"], par["A"], inp["B"], inp["C"],
                                    par["D"], inp["z"])
        if k in compare_at:
            torch.cuda.synchronize()
            assert bitwise_equal(y, y_rep), f"y differs from replay at step {k}"
            assert bitwise_equal(h, h_rep), f"state differs from replay at step {k}"
        # the oracle follows the sampled triples as 4096 one-channel "layers"
        xs = inp["x"][lic, sic, dic].cpu().view(1, 1, -1)
        ds = inp["dt"][lic, sic, dic].cpu().view(1, 1, -1)
        zs = inp["z"][lic, sic, dic].cpu().view(1, 1, -1)
        Bs = inp["B"][lic, sic].cpu()                            # [4096, N]
        Cs = inp["C"][lic, sic].cpu()
        yr, h_ref = oracle.step(h_ref.reshape(4096, 1, 1, N), xs.view(4096, 1, 1), ds.view(4096, 1, 1),
                                A_s.view(4096, 1, N), Bs.view(4096, 1, N), Cs.view(4096, 1, N),
                                D_s.view(4096, 1), zs.view(4096, 1, 1))
        assert rel_err(y[lic, sic, dic].cpu(), yr.reshape(-1)) <= TOL["bf16"], f"step {k}"
    torch.cuda.synchronize()
    assert rel_err(h[lic, sic, dic].cpu(), h_ref.reshape(4096, N)) <= TOL["bf16"]
