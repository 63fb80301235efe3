"""Helpers shared by the GPU tests: moving seeded inputs to the device, the error
metric, and the tolerances.

Tolerance: max |y_gpu - y_ref| <= tol * max |y_ref| over the compared tensor, with
tol = 1e-4 for fp32 inputs and 2e-2 for bf16 inputs (fp32 state). The same
criterion is applied to the final state.
"""
import sys
import threading

import numpy as np
import torch

import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(*a):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print("[case]", *a, file=sys.stderr, flush=True)


def to_dev(d: dict, device="cuda") -> dict:
    return {k: (None if v is None else v.to(device)) for k, v in d.items()}


def rel_err(got, ref) -> float:
    g = oracle.to_f64(got)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    scale = max(float(np.max(np.abs(r))) if r.size else 0.0, 1e-30)
    if g.size == 0:
        return 0.0
    return float(np.max(np.abs(g - r))) / scale


def bitwise_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    if a.dtype != b.dtype or a.shape != b.shape:
        return False
    ia = a.contiguous().view(torch.int16 if a.element_size() == 2 else torch.int32)
    ib = b.contiguous().view(torch.int16 if b.element_size() == 2 else torch.int32)
    return bool(torch.equal(ia, ib))


def gather_channels(t, idx, axis=2):
    """Channels idx (a CPU index tensor) of a device tensor, copied to the host."""
    return None if t is None else t.index_select(axis, idx.to(t.device)).cpu()


def threaded_channels(fn, n_channels, threads=16):
    """fn(sl) -> (y [.., .., k], h [.., k, ..]) on the channel slice sl of a sample,
    run from several threads (the oracle releases the GIL; channels are independent)
    and joined along the channel axes: y's axis 2 (or its last axis for rank > 1
    outputs, with channels at axis 2) and h's axis 1."""
    parts = [p for p in np.array_split(np.arange(n_channels), max(1, threads)) if len(p)]
    res = [None] * len(parts)

    def work(i, p):
        res[i] = fn(slice(int(p[0]), int(p[-1]) + 1))

    ts = [threading.Thread(target=work, args=(i, p)) for i, p in enumerate(parts)]
    for t in ts: t.start()
    for t in ts: t.join()
    return (np.concatenate([r[0] for r in res], axis=2), np.concatenate([r[1] for r in res], axis=1))
