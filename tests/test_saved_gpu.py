"""Training with stored states on the GPU: ssm_scan_fwd_save (the forward that also
stores the state entering every 8th step) and ssm_scan_bwd_saved (the backward that
reads those states instead of recomputing them by a forward walk).

- The forward's y and h_final equal ssm_scan_fwd_ex's bit for bit for the same chunk
  length, and every stored row equals the oracle's state after 8 r steps (the oracle's
  scan of the first 8 r steps) to the forward's tolerance.
- The backward's gradients match the fp64 oracle's scan_bwd to the backward's tolerance
  on the plain backward's cases (chunks of every length, ragged ends, every state size,
  padding waves, bf16 with N = 1 and odd rows of B and C).
- selective_scan(save_states=True) returns exactly what the two direct calls return.
- Full size: every stored row of the 256k training forward on a channel sample against
  the oracle's sequential states (fp32 tolerance, row by row), and the 256k prefill's
  backward from stored states on a channel sample, as the plain backward's full-size test
  does it.
"""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_49_amd as ssm
from tests.gpu_util import TOL, bitwise_equal, gather_channels, rel_err, say, to_dev
from tests.test_bwd_gpu import CASES as BWD_CASES, GRADS, _compare, _draw, _ids as _bwd_ids, _oracle, \
    _oracle_threaded
from workloads import WORKLOADS, ScanShape, make_h0, make_scan_inputs, sample_channels

pytestmark = pytest.mark.gpu
EVERY = ssm.STATE_EVERY


def _rows(states, b, Dn, N):
    """Stored states as [rows, b, Dn, N]."""
    if N % 4 == 0:
        return states.permute(0, 1, 3, 2, 4).reshape(states.shape[0], b, Dn, N)
    return states


# (batch, L, d_inner, d_state, io, gated, with_h0, chunk_len)
FWD_CASES = [
    (2, 300, 200, 16, "bf16", True, True, 64),    # 5 chunks, ragged last chunk
    (2, 300, 130, 16, "f32", False, True, 37),    # chunk length rounded down to 32
    (1, 1000, 130, 8, "bf16", True, False, 0),    # the library's own plan
    (2, 257, 70, 4, "f32", True, True, 48),
    (1, 203, 65, 2, "f32", True, True, 16),
    (3, 129, 64, 1, "bf16", True, True, 16),      # bf16, N = 1, odd L
    (3, 129, 64, 16, "f32", True, True, 1000),    # one chunk
    (1, 5, 16, 16, "f32", True, True, 0),         # shorter than one stored row's span
    (1, 1, 1, 1, "f32", True, True, 0),           # one step
]


def _fwd_ids(c):
    b, L, Dn, N, io, g, h0, T = c
    return f"b{b}_L{L}_D{Dn}_N{N}_{io}_{'gated' if g else 'nogate'}_{'h0' if h0 else 'zero'}_T{T}"


@pytest.mark.parametrize("case", FWD_CASES, ids=_fwd_ids)
def test_forward_save_matches_ex_and_stores_the_oracle_states(case):
    b, L, Dn, N, io, gated, with_h0, T = case
    shape = ScanShape("save", b, L, Dn, N, io, gated=gated, seed=300)
    inp = make_scan_inputs(shape, "cpu")
    h0 = make_h0(b, Dn, N, seed=301) if with_h0 else None
    d = to_dev(inp)
    h0d = None if h0 is None else h0.cuda()
    say("forward with stored states", _fwd_ids(case))
    y, hf, st = ssm.ssm_scan_fwd_save(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], h0d,
                                      chunk_len=T)
    torch.cuda.synchronize()
    tol = TOL[io]
    if T > 0 and T % EVERY == 0:  # the same chunks as ssm_scan_fwd_ex: the same bits
        y2, hf2 = ssm.ssm_scan_fwd_ex(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], h0d,
                                      chunk_len=T)
        torch.cuda.synchronize()
        assert bitwise_equal(y, y2) and bitwise_equal(hf, hf2)
    yr, hr = oracle.scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], h0)
    assert rel_err(y, yr) <= tol and rel_err(hf, hr) <= tol
    rows = _rows(st, b, Dn, N).cpu()
    n = rows.shape[0]
    assert n == (L + EVERY - 1) // EVERY
    for r in sorted({0, 1, n // 2, n - 1} & set(range(n))):
        t = r * EVERY
        if t == 0:
            ref = torch.zeros((b, Dn, N), dtype=torch.float64) if h0 is None else h0.double()
        else:
            _, ref = oracle.scan(inp["x"][:, :t], inp["dt"][:, :t], inp["A"], inp["B"][:, :t],
                                 inp["C"][:, :t], inp["D"], None if inp["z"] is None else inp["z"][:, :t], h0)
        assert rel_err(rows[r], ref) <= tol, f"stored state {r} (step {t}): error {rel_err(rows[r], ref):.3e}"


def _saved(d, chunk_len, **kw):
    g = to_dev(d)
    _, _, st = ssm.ssm_scan_fwd_save(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["z"], g["h0"],
                                     chunk_len=chunk_len)
    return ssm.ssm_scan_bwd_saved(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["z"], states=st,
                                  dy=g["dy"], dh_final=g["dh_final"], chunk_len=chunk_len, **kw)


@pytest.mark.parametrize("case", BWD_CASES, ids=_bwd_ids)
def test_backward_from_stored_states_matches_oracle(case):
    shape, d = _draw(case)
    say("backward from stored states", _bwd_ids(case))
    got = _saved(d, case[6])
    torch.cuda.synchronize()
    _compare(got, _oracle(d), TOL[shape.io])


def test_stored_states_do_not_depend_on_either_chunk_plan():
    # The rows are global (row r: the state entering step 8 r), so the backward may cut
    # its chunks differently from the forward that stored them.
    case = (2, 500, 130, 16, "bf16", True, 0, True, True)
    shape, d = _draw(case, seed=315)
    g = to_dev(d)
    say("stored states across chunk plans")
    _, _, st = ssm.ssm_scan_fwd_save(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["z"], g["h0"],
                                     chunk_len=24)
    ref = _oracle(d)
    for T in (0, 64, 1000):
        got = ssm.ssm_scan_bwd_saved(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["z"], states=st,
                                     dy=g["dy"], dh_final=g["dh_final"], chunk_len=T)
        torch.cuda.synchronize()
        _compare(got, ref, TOL[shape.io])


def test_backward_from_stored_states_edges():
    # L = 0: no states are needed (dA = dD = 0, dh0 = dh_final); states are required for
    # L > 0; the backward's chunk length is rounded down to a multiple of 8.
    shape = ScanShape("saved0", 2, 0, 40, 16, "f32", seed=310)
    d = to_dev(make_scan_inputs(shape, "cpu"))
    dh = torch.randn((2, 40, 16), generator=torch.Generator().manual_seed(311)).cuda()
    say("backward from stored states: L = 0")
    got = ssm.ssm_scan_bwd_saved(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"],
                                 states=torch.empty((0, 2, 4, 40, 4), device="cuda"),
                                 dy=torch.empty((2, 0, 40), device="cuda"), dh_final=dh)
    torch.cuda.synchronize()
    assert not got["dA"].any() and not got["dD"].any() and bitwise_equal(got["dh0"], dh)
    case = (1, 100, 40, 16, "f32", True, 0, True, True)
    shape, d = _draw(case, seed=312)
    g = to_dev(d)
    with pytest.raises(ssm.SsmError):
        ssm.ssm_scan_bwd_saved(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["z"], states=None,
                               dy=g["dy"])
    assert ssm.ssm_scan_bwd_saved_workspace(1, 100, 40, 16, 20) == ssm.ssm_scan_bwd_saved_workspace(1, 100, 40, 16, 16)
    assert ssm.ssm_scan_bwd_saved_workspace(1, 1000, 40, 16, 64) < ssm.ssm_scan_bwd_workspace(1, 1000, 40, 16, 64)


@pytest.mark.parametrize("io,gated,with_h0", [("f32", True, True), ("bf16", True, False)])
def test_selective_scan_with_stored_states(io, gated, with_h0):
    # The autograd function with save_states: the forward is ssm_scan_fwd_save's, and the
    # gradients are ssm_scan_bwd_saved's from its states, bit for bit.
    b, L, Dn, N, T = 2, 150, 70, 16, 32
    shape = ScanShape("autograd_saved", b, L, Dn, N, io, gated=gated, seed=320)
    d = make_scan_inputs(shape, "cpu")
    d["h0"] = make_h0(b, Dn, N) if with_h0 else None
    g = to_dev(d)
    gen = torch.Generator().manual_seed(321)
    gy = torch.randn((b, L, Dn), generator=gen).to(g["x"].dtype).cuda()
    gh = torch.randn((b, Dn, N), generator=gen).cuda()
    names = ("x", "dt", "A", "B", "C", "D", "z", "h0")
    leaves = {k: (None if g[k] is None else g[k].clone().requires_grad_()) for k in names}
    say("selective_scan with stored states", io, gated, with_h0)
    y, hf = ssm.selective_scan(*[leaves[k] for k in names], chunk_len=T, save_states=True)
    ((y.float() * gy.float()).sum() + (hf * gh).sum()).backward()
    y_ref, hf_ref, st = ssm.ssm_scan_fwd_save(*[g[k] for k in names], chunk_len=T)
    ref = ssm.ssm_scan_bwd_saved(*[g[k] for k in names[:7]], states=st, dy=gy, dh_final=gh, chunk_len=T)
    torch.cuda.synchronize()
    assert bitwise_equal(y.detach(), y_ref) and bitwise_equal(hf.detach(), hf_ref)
    for k in names:
        if leaves[k] is None:
            continue
        grad, want = leaves[k].grad, ref["d" + k]
        assert bitwise_equal(grad, want.to(grad.dtype)), f"d{k} differs from ssm_scan_bwd_saved"


def test_forward_save_full_size_every_stored_row_sampled():
    # The 256k prefill in the library's own plan: every one of the 32768 stored rows, on a
    # channel sample, against the oracle's state entering that step. The oracle walks the
    # sequence in 8-step pieces, each resumed from the last one's final state (its
    # split/resume is exact), so its states are those of one sequential walk. States are
    # fp32 and the inputs exact bf16 values: the fp32 tolerance applies, row by row.
    shape = WORKLOADS["long_context_256k"]
    N, Dn, L = shape.d_state, shape.d_inner, shape.L
    say("stored states 256k, every row: inputs")
    d = make_scan_inputs(shape, "cuda")
    idx = sample_channels(Dn, 32, seed=29)
    say("stored states 256k, every row: forward")
    _, _, st = ssm.ssm_scan_fwd_save(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"])
    torch.cuda.synchronize()
    rows = _rows(st, shape.batch, Dn, N).index_select(2, idx.cuda()).cpu()
    del st
    n = rows.shape[0]
    assert n == (L + EVERY - 1) // EVERY
    gc = lambda t: oracle.to_f64(gather_channels(t, idx))
    x, dt, z = gc(d["x"]), gc(d["dt"]), gc(d["z"])
    B, C = oracle.to_f64(d["B"].cpu()), oracle.to_f64(d["C"].cpu())
    A, D = oracle.to_f64(d["A"].cpu()[idx]), oracle.to_f64(d["D"].cpu()[idx])
    say("stored states 256k, every row: oracle on", len(idx), "channels")
    ref = np.zeros((n, shape.batch, len(idx), N))
    h = ref[0].copy()
    for r in range(1, n):
        a, b = (r - 1) * EVERY, r * EVERY
        _, h = oracle.scan(x[:, a:b], dt[:, a:b], A, B[:, a:b], C[:, a:b], D, z[:, a:b], h)
        ref[r] = h
    got = oracle.to_f64(rows)
    err = np.max(np.abs(got - ref), axis=(1, 2, 3)) / np.maximum(np.max(np.abs(ref), axis=(1, 2, 3)), 1e-30)
    bad = np.nonzero(err > TOL["f32"])[0]
    assert len(bad) == 0, f"{len(bad)} stored rows off, first {bad[:5]}, worst {err.max():.3e}"


def test_backward_from_stored_states_full_size_long_context_sampled():
    # The 256k prefill (batch 1, L 262144, 8192 channels, N 16, bf16) in the library's own
    # plans: the training forward stores 17 GB of states, the backward reads them. dy on
    # a channel sample, as in the plain backward's full-size test.
    shape = WORKLOADS["long_context_256k"]
    say("backward from stored states 256k: inputs")
    d = make_scan_inputs(shape, "cuda")
    idx = sample_channels(shape.d_inner, 256, seed=17)
    g = torch.Generator(device="cuda").manual_seed(83)
    dy = torch.zeros(d["x"].shape, dtype=d["x"].dtype, device="cuda")
    dy[:, :, idx.cuda()] = torch.randn((shape.batch, shape.L, len(idx)), generator=g,
                                       device="cuda").to(dy.dtype)
    say("backward from stored states 256k: forward")
    _, _, st = ssm.ssm_scan_fwd_save(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"])
    say("backward from stored states 256k: backward")
    got = ssm.ssm_scan_bwd_saved(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], states=st, dy=dy)
    torch.cuda.synchronize()
    del st
    rest = torch.ones(shape.d_inner, dtype=torch.bool)
    rest[idx] = False
    for k in ("dx", "ddt", "dz"):
        assert not got[k][:, :, rest.cuda()].any(), f"{k} nonzero outside the sample"
    gc = lambda t: gather_channels(t, idx)
    sub = {"x": gc(d["x"]), "dt": gc(d["dt"]), "z": gc(d["z"]), "dy": gc(dy), "A": d["A"].cpu()[idx],
           "B": d["B"].cpu(), "C": d["C"].cpu(), "D": d["D"].cpu()[idx], "h0": None, "dh_final": None}
    say("backward from stored states 256k: oracle on", len(idx), "channels")
    ref = _oracle_threaded(sub)
    tol = TOL["bf16"]
    for k in ("dx", "ddt", "dz"):
        e = rel_err(gc(got[k]), ref[k])
        assert e <= tol, f"{k}: error {e:.3e}"
    for k, v in (("dA", got["dA"].cpu()[idx]), ("dD", got["dD"].cpu()[idx]), ("dB", got["dB"]),
                 ("dC", got["dC"])):
        e = rel_err(v, ref[k])
        assert e <= tol, f"{k}: error {e:.3e}"
