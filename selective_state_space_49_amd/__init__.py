"""Python binding of libssmscan: the selective state-space scan on MI355X (gfx950).

This module only marshals arguments: it checks tensor shapes, dtypes and devices,
allocates outputs and workspace with torch when the caller does not pass them, and
calls the C entry points of ``include/ssm_scan.h`` by the same names, on torch's
current HIP stream. Every step of the computation runs in the library's HIP
kernels. There is no fallback: if the library is missing or the tensors are not on
the GPU, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "SsmError", "load_library", "library_path",
    "ssm_scan_fwd", "ssm_scan_fwd_ex", "ssm_scan_fwd_c64", "ssm_scan_fwd_workspace",
    "ssm_scan_fwd_workspace_ex", "ssm_scan_fwd_c64_workspace", "ssm_scan_fwd_chunk_len",
    "ssm_step", "ssm_step_replay", "ssm_step_c64", "ssm_step_c64_replay",
    "ssm_status_str", "ssm_last_error", "ssm_abi_version", "EXPORTED_SYMBOLS",
    "ssm_scan_fwd_profiled", "ssm_scan_fwd_c64_profiled",
    "ssm_scan_fwd_fused", "ssm_scan_fwd_fused_profiled", "ssm_step_fused", "ssm_step_fused_replay",
    "ssm_scan_bwd", "ssm_scan_bwd_workspace", "ssm_scan_bwd_fused", "ssm_scan_bwd_fused_workspace",
    "ssm_scan_fwd_trap", "ssm_scan_fwd_trap_profiled", "ssm_step_trap", "ssm_step_trap_replay",
    "ssm_scan_fwd_mimo", "ssm_scan_fwd_mimo_profiled", "ssm_scan_fwd_mimo_workspace",
    "ssm_step_mimo", "ssm_scan_fwd_fused_chunk_len", "ssm_scan_fwd_c64_chunk_len",
    "ssm_scan_fwd_mimo_chunk_len", "selective_scan", "selective_scan_fused",
    "ssm_scan_fwd_noalloc", "NOALLOC_SCRATCH_BYTES",
    "ssm_scan_fwd_save", "ssm_scan_fwd_save_workspace", "ssm_scan_fwd_save_states_bytes",
    "ssm_scan_bwd_saved", "ssm_scan_bwd_saved_workspace", "STATE_EVERY",
    "ssm_scan_fwd_fused_save", "ssm_scan_bwd_fused_saved", "ssm_scan_bwd_fused_saved_workspace",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# SSMSCAN_LIBRARY may point at another build of the same library (e.g. a tuning variant).
_LIB_PATH = os.environ.get("SSMSCAN_LIBRARY") or os.path.join(_HERE, "libssmscan.so")
_lib = None

SSM_F32, SSM_BF16 = 0, 1
EXPORTED_SYMBOLS = [
    "ssm_scan_fwd", "ssm_scan_fwd_ex", "ssm_scan_fwd_c64", "ssm_scan_fwd_workspace",
    "ssm_scan_fwd_workspace_ex", "ssm_scan_fwd_c64_workspace", "ssm_scan_fwd_chunk_len",
    "ssm_step", "ssm_step_replay", "ssm_step_c64", "ssm_step_c64_replay",
    "ssm_status_str", "ssm_last_error", "ssm_abi_version",
    "ssm_scan_fwd_profiled", "ssm_scan_fwd_c64_profiled",
    "ssm_scan_fwd_fused", "ssm_scan_fwd_fused_profiled", "ssm_step_fused", "ssm_step_fused_replay",
    "ssm_scan_bwd", "ssm_scan_bwd_workspace", "ssm_scan_bwd_fused", "ssm_scan_bwd_fused_workspace",
    "ssm_scan_fwd_trap", "ssm_scan_fwd_trap_profiled", "ssm_step_trap", "ssm_step_trap_replay",
    "ssm_scan_fwd_mimo", "ssm_scan_fwd_mimo_profiled", "ssm_scan_fwd_mimo_workspace",
    "ssm_step_mimo", "ssm_scan_fwd_fused_chunk_len", "ssm_scan_fwd_c64_chunk_len",
    "ssm_scan_fwd_mimo_chunk_len", "ssm_scan_fwd_noalloc",
    "ssm_scan_fwd_save", "ssm_scan_fwd_save_workspace", "ssm_scan_fwd_save_states_bytes",
    "ssm_scan_bwd_saved", "ssm_scan_bwd_saved_workspace",
    "ssm_scan_fwd_fused_save", "ssm_scan_bwd_fused_saved", "ssm_scan_bwd_fused_saved_workspace",
]
# Steps between the states ssm_scan_fwd_save stores for ssm_scan_bwd_saved.
STATE_EVERY = 8
# SSM_NOALLOC_SCRATCH_BYTES of ssm_scan.h: the scratch ssm_scan_fwd_noalloc has per GPU.
NOALLOC_SCRATCH_BYTES = 64 << 20


class SsmError(RuntimeError):
    """A non-zero ssm_status from the library, with its detail string."""

    def __init__(self, status: int, detail: str):
        super().__init__(f"ssm status {status} ({ssm_status_str(status)}): {detail}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libssmscan.so (built by selective_state_space_49_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m selective_state_space_49_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    ci = ctypes.c_int
    scan = [vp] * 10 + [i64, i64, i64, i32, ci]
    sig = {
        "ssm_scan_fwd_workspace": ([i64, i64, i64, i32], sz),
        "ssm_scan_fwd_workspace_ex": ([i64, i64, i64, i32, i64], sz),
        "ssm_scan_fwd_c64_workspace": ([i64, i64, i64, i32, i64], sz),
        "ssm_scan_fwd_chunk_len": ([i64, i64, i64, i32], i64),
        "ssm_scan_fwd_fused_chunk_len": ([i64, i64, i64, i32], i64),
        "ssm_scan_fwd_c64_chunk_len": ([i64, i64, i64, i32], i64),
        "ssm_scan_fwd_mimo_chunk_len": ([i64, i64, i64, i32, i32], i64),
        "ssm_scan_fwd": (scan + [vp, sz, vp], ci),
        "ssm_scan_fwd_ex": (scan + [i64, vp, sz, vp], ci),
        "ssm_scan_fwd_c64": (scan + [i64, vp, sz, vp], ci),
        "ssm_scan_fwd_noalloc": (scan + [i64, vp], ci),
        "ssm_scan_fwd_profiled": (scan + [i64, vp, sz, vp, vp, i32], ci),
        "ssm_scan_fwd_c64_profiled": (scan + [i64, vp, sz, vp, vp, i32], ci),
        "ssm_status_str": ([ci], ctypes.c_char_p),
        "ssm_last_error": ([], ctypes.c_char_p),
        "ssm_abi_version": ([], i32),
    }
    step = [vp] * 9 + [i64, i64, i64, i32, ci, vp]
    for name in ("ssm_step", "ssm_step_replay", "ssm_step_c64", "ssm_step_c64_replay"):
        sig[name] = (step, ci)
    fused = [vp] * 10 + [i32, vp, vp, vp, vp, vp, i64, i64, i64, i32, ci, i64, vp, sz, vp]
    sig["ssm_scan_fwd_fused"] = (fused, ci)
    sig["ssm_scan_fwd_fused_profiled"] = (fused + [vp, i32], ci)
    sig["ssm_scan_fwd_fused_save"] = ([vp] * 10 + [i32] + [vp] * 8 + [i64, i64, i64, i32, ci, i64, vp, sz, vp], ci)
    sig["ssm_scan_bwd_workspace"] = ([i64, i64, i64, i32, i64], sz)
    sig["ssm_scan_bwd"] = ([vp] * 18 + [i64, i64, i64, i32, ci, i64, vp, sz, vp], ci)
    sig["ssm_scan_bwd_saved"] = ([vp] * 18 + [i64, i64, i64, i32, ci, i64, vp, sz, vp], ci)
    sig["ssm_scan_bwd_saved_workspace"] = ([i64, i64, i64, i32, i64], sz)
    sig["ssm_scan_fwd_save"] = ([vp] * 11 + [i64, i64, i64, i32, ci, i64, vp, sz, vp], ci)
    sig["ssm_scan_fwd_save_workspace"] = ([i64, i64, i64, i32, i64], sz)
    sig["ssm_scan_fwd_save_states_bytes"] = ([i64, i64, i64, i32], sz)
    sig["ssm_scan_bwd_fused_workspace"] = ([i64, i64, i64, i32, i32, ci, i64], sz)
    sig["ssm_scan_bwd_fused"] = ([vp] * 10 + [i32] + [vp] * 16 + [i64, i64, i64, i32, ci, i64, vp, sz, vp], ci)
    sig["ssm_scan_bwd_fused_saved"] = ([vp] * 12 + [i32] + [vp] * 16 + [i64, i64, i64, i32, ci, i64, vp, sz, vp], ci)
    sig["ssm_scan_bwd_fused_saved_workspace"] = sig["ssm_scan_bwd_fused_workspace"]
    trap = [vp] * 13 + [i64, i64, i64, i32, ci, i64, vp, sz, vp]
    sig["ssm_scan_fwd_trap"] = (trap, ci)
    sig["ssm_scan_fwd_trap_profiled"] = (trap + [vp, i32], ci)
    for name in ("ssm_step_trap", "ssm_step_trap_replay"):
        sig[name] = ([vp] * 12 + [i64, i64, i64, i32, ci, vp], ci)
    sig["ssm_scan_fwd_mimo_workspace"] = ([i64, i64, i64, i32, i32, i64], sz)
    mimo = [vp] * 10 + [i64, i64, i64, i32, i32, ci, i64, vp, sz, vp]
    sig["ssm_scan_fwd_mimo"] = (mimo, ci)
    sig["ssm_scan_fwd_mimo_profiled"] = (mimo + [vp, i32], ci)
    sig["ssm_step_mimo"] = ([vp] * 9 + [i64, i64, i64, i32, i32, ci, vp], ci)
    step_fused = [vp] * 11 + [i32, vp, vp, i64, i64, i64, i32, ci, vp]
    for name in ("ssm_step_fused", "ssm_step_fused_replay"):
        sig[name] = (step_fused, ci)
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes, f.restype = args, res
    _lib = lib
    return lib


def ssm_status_str(status: int) -> str:
    return load_library().ssm_status_str(status).decode()


def ssm_last_error() -> str:
    return load_library().ssm_last_error().decode()


def ssm_abi_version() -> int:
    return int(load_library().ssm_abi_version())


def _check(status: int):
    if status != 0:
        raise SsmError(status, ssm_last_error())


def _io(*tensors) -> int:
    dts = {t.dtype for t in tensors if t is not None}
    if len(dts) != 1:
        raise TypeError(f"x, dt, z, B, C (and y) must share one dtype, got {dts}")
    dt = dts.pop()
    if dt == torch.float32:
        return SSM_F32
    if dt == torch.bfloat16:
        return SSM_BF16
    raise TypeError(f"io dtype must be float32 or bfloat16, got {dt}")


def _dev(t: Optional[torch.Tensor], name: str, shape=None, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


# ------------------------------------------------------------------ workspace queries
def ssm_scan_fwd_workspace(batch: int, L: int, d_inner: int, d_state: int) -> int:
    return int(load_library().ssm_scan_fwd_workspace(batch, L, d_inner, d_state))


def ssm_scan_fwd_workspace_ex(batch, L, d_inner, d_state, chunk_len) -> int:
    return int(load_library().ssm_scan_fwd_workspace_ex(batch, L, d_inner, d_state, chunk_len))


def ssm_scan_fwd_c64_workspace(batch, L, d_inner, d_state, chunk_len=0) -> int:
    return int(load_library().ssm_scan_fwd_c64_workspace(batch, L, d_inner, d_state, chunk_len))


def ssm_scan_fwd_chunk_len(batch, L, d_inner, d_state) -> int:
    return int(load_library().ssm_scan_fwd_chunk_len(batch, L, d_inner, d_state))


def ssm_scan_fwd_fused_chunk_len(batch, L, d_inner, d_state) -> int:
    return int(load_library().ssm_scan_fwd_fused_chunk_len(batch, L, d_inner, d_state))


def ssm_scan_fwd_c64_chunk_len(batch, L, d_inner, d_state) -> int:
    return int(load_library().ssm_scan_fwd_c64_chunk_len(batch, L, d_inner, d_state))


def ssm_scan_fwd_mimo_chunk_len(batch, L, d_inner, d_state, rank) -> int:
    return int(load_library().ssm_scan_fwd_mimo_chunk_len(batch, L, d_inner, d_state, rank))


# ------------------------------------------------------------------ prefill
def _scan(fn_name, cplx, x, dt, A, B, C, D, z, h0, chunk_len, y, h_final, workspace, want_h_final,
          events=None):
    lib = load_library()
    b, L, Dn = x.shape
    N = A.shape[1]
    ext = (2,) if cplx else ()
    f32 = torch.float32
    _dev(x, "x"); _dev(dt, "dt", (b, L, Dn)); _dev(z, "z", (b, L, Dn))
    _dev(A, "A", (Dn, N) + ext, f32); _dev(D, "D", (Dn,), f32)
    _dev(B, "B", (b, L, N) + ext); _dev(C, "C", (b, L, N) + ext)
    _dev(h0, "h0", (b, Dn, N) + ext, f32)
    io = _io(x, dt, z, B, C)
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y", (b, L, Dn), x.dtype)
    if h_final is None and want_h_final:
        h_final = torch.empty((b, Dn, N) + ext, dtype=f32, device=x.device)
    _dev(h_final, "h_final", (b, Dn, N) + ext, f32)
    if cplx:
        need = ssm_scan_fwd_c64_workspace(b, L, Dn, N, chunk_len)
    else:
        need = ssm_scan_fwd_workspace_ex(b, L, Dn, N, chunk_len)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y),
            _ptr(h_final), b, L, Dn, N, io]
    if fn_name == "ssm_scan_fwd":
        st = lib.ssm_scan_fwd(*args, _ptr(workspace), ws_bytes, _stream(x))
    elif events is not None:
        handles = (ctypes.c_void_p * 4)(*[ctypes.c_void_p(e) for e in events])
        st = getattr(lib, fn_name)(*args, chunk_len, _ptr(workspace), ws_bytes, _stream(x),
                                   handles, len(events))
    else:
        st = getattr(lib, fn_name)(*args, chunk_len, _ptr(workspace), ws_bytes, _stream(x))
    _check(st)
    return y, h_final


def ssm_scan_fwd(x, dt, A, B, C, D, z=None, h0=None, *, y=None, h_final=None, workspace=None,
                 want_h_final=True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Prefill: y [b, L, d_inner] and h_final [b, d_inner, d_state] (see ssm_scan.h)."""
    return _scan("ssm_scan_fwd", False, x, dt, A, B, C, D, z, h0, 0, y, h_final, workspace,
                 want_h_final)


def ssm_scan_fwd_ex(x, dt, A, B, C, D, z=None, h0=None, *, chunk_len=0, y=None, h_final=None,
                    workspace=None, want_h_final=True):
    """Prefill with an explicit chunk length (0 = the library's choice)."""
    return _scan("ssm_scan_fwd_ex", False, x, dt, A, B, C, D, z, h0, chunk_len, y, h_final,
                 workspace, want_h_final)


def _states_shape(b, L, Dn, N):
    """The stored states' layout (ssm_scan.h): ceil(L / 8) rows; in a row [b][N/4][Dn][4]
    for N a multiple of 4, else [b][Dn][N]."""
    rows = (L + STATE_EVERY - 1) // STATE_EVERY
    return (rows, b, N // 4, Dn, 4) if N % 4 == 0 else (rows, b, Dn, N)


def ssm_scan_fwd_save_states_bytes(batch, L, d_inner, d_state) -> int:
    return int(load_library().ssm_scan_fwd_save_states_bytes(batch, L, d_inner, d_state))


def ssm_scan_fwd_save_workspace(batch, L, d_inner, d_state, chunk_len=0) -> int:
    return int(load_library().ssm_scan_fwd_save_workspace(batch, L, d_inner, d_state, chunk_len))


def ssm_scan_fwd_save(x, dt, A, B, C, D, z=None, h0=None, *, chunk_len=0, y=None, h_final=None,
                      states=None, workspace=None):
    """The training forward: ssm_scan_fwd_ex's y and h_final, and the state entering every
    8th step (float32, shaped as _states_shape) for ssm_scan_bwd_saved."""
    lib = load_library()
    b, L, Dn = x.shape
    N = A.shape[1]
    f32 = torch.float32
    _dev(x, "x"); _dev(dt, "dt", (b, L, Dn)); _dev(z, "z", (b, L, Dn))
    _dev(A, "A", (Dn, N), f32); _dev(D, "D", (Dn,), f32)
    _dev(B, "B", (b, L, N)); _dev(C, "C", (b, L, N)); _dev(h0, "h0", (b, Dn, N), f32)
    io = _io(x, dt, z, B, C)
    dev = x.device
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y", (b, L, Dn), x.dtype)
    if h_final is None:
        h_final = torch.empty((b, Dn, N), dtype=f32, device=dev)
    _dev(h_final, "h_final", (b, Dn, N), f32)
    if states is None:
        states = torch.empty(_states_shape(b, L, Dn, N), dtype=f32, device=dev)
    _dev(states, "states", _states_shape(b, L, Dn, N), f32)
    need = ssm_scan_fwd_save_workspace(b, L, Dn, N, chunk_len)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.ssm_scan_fwd_save(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                               _ptr(h0), _ptr(y), _ptr(h_final), _ptr(states), b, L, Dn, N, io,
                               chunk_len, _ptr(workspace), ws_bytes, _stream(x))
    _check(st)
    return y, h_final, states


def ssm_scan_fwd_noalloc(x, dt, A, B, C, D, z=None, h0=None, *, chunk_len=0, y=None, h_final=None,
                         want_h_final=True):
    """Prefill with no workspace: the library's per-GPU scratch array holds the chunk
    summaries (see ssm_scan.h). The C entry point allocates nothing; y and h_final are
    allocated here with torch unless given. Calls that overlap in time on one GPU race
    on the scratch."""
    lib = load_library()
    b, L, Dn = x.shape
    N = A.shape[1]
    f32 = torch.float32
    _dev(x, "x"); _dev(dt, "dt", (b, L, Dn)); _dev(z, "z", (b, L, Dn))
    _dev(A, "A", (Dn, N), f32); _dev(D, "D", (Dn,), f32)
    _dev(B, "B", (b, L, N)); _dev(C, "C", (b, L, N)); _dev(h0, "h0", (b, Dn, N), f32)
    io = _io(x, dt, z, B, C)
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y", (b, L, Dn), x.dtype)
    if h_final is None and want_h_final:
        h_final = torch.empty((b, Dn, N), dtype=f32, device=x.device)
    _dev(h_final, "h_final", (b, Dn, N), f32)
    with torch.cuda.device(x.device):  # the scratch of the tensors' own GPU
        st = lib.ssm_scan_fwd_noalloc(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                      _ptr(h0), _ptr(y), _ptr(h_final), b, L, Dn, N, io, chunk_len,
                                      _stream(x))
    _check(st)
    return y, h_final


def ssm_scan_fwd_c64(x, dt, A, B, C, D, z=None, h0=None, *, chunk_len=0, y=None, h_final=None,
                     workspace=None, want_h_final=True):
    """Complex-state prefill: A [d_inner, d_state, 2]; B, C [b, L, d_state, 2]."""
    return _scan("ssm_scan_fwd_c64", True, x, dt, A, B, C, D, z, h0, chunk_len, y, h_final,
                 workspace, want_h_final)


def ssm_scan_fwd_profiled(x, dt, A, B, C, D, z=None, h0=None, *, events, chunk_len=0, y=None,
                          h_final=None, workspace=None, want_h_final=True, complex_state=False):
    """Prefill that records 4 HIP events (raw hipEvent_t handles as ints) at the
    kernel boundaries on the current stream; see ssm_scan.h."""
    if len(events) != 4:
        raise ValueError("need exactly 4 event handles")
    name = "ssm_scan_fwd_c64_profiled" if complex_state else "ssm_scan_fwd_profiled"
    return _scan(name, complex_state, x, dt, A, B, C, D, z, h0, chunk_len, y, h_final, workspace,
                 want_h_final, events=list(events))


def ssm_scan_fwd_c64_profiled(*a, **k):
    return ssm_scan_fwd_profiled(*a, complex_state=True, **k)


# ------------------------------------------------------------------ decode
def _step(fn_name, cplx, h, x, dt, A, B, C, D, z, y):
    lib = load_library()
    Ln, S, Dn = x.shape
    N = A.shape[2]
    ext = (2,) if cplx else ()
    f32 = torch.float32
    _dev(h, "h", (Ln, S, Dn, N) + ext, f32)
    _dev(x, "x_t"); _dev(dt, "dt_t", (Ln, S, Dn)); _dev(z, "z_t", (Ln, S, Dn))
    _dev(A, "A", (Ln, Dn, N) + ext, f32); _dev(D, "D", (Ln, Dn), f32)
    _dev(B, "B_t", (Ln, S, N) + ext); _dev(C, "C_t", (Ln, S, N) + ext)
    io = _io(x, dt, z, B, C)
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y_t", (Ln, S, Dn), x.dtype)
    st = getattr(lib, fn_name)(_ptr(h), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                               _ptr(z), _ptr(y), Ln, S, Dn, N, io, _stream(x))
    _check(st)
    return y


def ssm_step(h, x_t, dt_t, A, B_t, C_t, D, z_t=None, *, y_t=None):
    """One decode token for every (layer, sequence): h updated in place, returns y_t."""
    return _step("ssm_step", False, h, x_t, dt_t, A, B_t, C_t, D, z_t, y_t)


def ssm_step_replay(h, x_t, dt_t, A, B_t, C_t, D, z_t=None, *, y_t=None):
    """The decode step in its written-down reference order, one thread per channel."""
    return _step("ssm_step_replay", False, h, x_t, dt_t, A, B_t, C_t, D, z_t, y_t)


def ssm_step_c64(h, x_t, dt_t, A, B_t, C_t, D, z_t=None, *, y_t=None):
    return _step("ssm_step_c64", True, h, x_t, dt_t, A, B_t, C_t, D, z_t, y_t)


def ssm_step_c64_replay(h, x_t, dt_t, A, B_t, C_t, D, z_t=None, *, y_t=None):
    return _step("ssm_step_c64_replay", True, h, x_t, dt_t, A, B_t, C_t, D, z_t, y_t)


# ------------------------------------------------------------------ exponential-trapezoidal
def ssm_scan_fwd_trap(x, dt, A, B, C, D, z=None, h0=None, x_prev=None, B_prev=None, *,
                      lam=None, chunk_len=0, y=None, h_final=None, workspace=None,
                      want_h_final=True, events=None):
    """Prefill with the exponential-trapezoidal discretisation (see ssm_scan.h):
    h_t = a_t h_{t-1} + dt_t((1 - lam_t) a_t B_{t-1} x_{t-1} + lam_t B_t x_t). lam
    [b, L, d_inner] (io dtype) weighs each step's current input (None: 1/2, the
    trapezoid rule; 1 is Euler's step). x_prev [b, d_inner] and B_prev [b, d_state]
    (io dtype, both or neither) are the input before step 0. events: None, or 4 raw
    hipEvent_t handles for the profiled entry point. Returns (y, h_final)."""
    lib = load_library()
    b, L, Dn = x.shape
    N = A.shape[1]
    f32 = torch.float32
    _dev(x, "x"); _dev(dt, "dt", (b, L, Dn)); _dev(z, "z", (b, L, Dn))
    _dev(A, "A", (Dn, N), f32); _dev(D, "D", (Dn,), f32)
    _dev(B, "B", (b, L, N)); _dev(C, "C", (b, L, N)); _dev(h0, "h0", (b, Dn, N), f32)
    _dev(x_prev, "x_prev", (b, Dn)); _dev(B_prev, "B_prev", (b, N)); _dev(lam, "lam", (b, L, Dn))
    io = _io(x, dt, z, B, C, x_prev, B_prev, lam)
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y", (b, L, Dn), x.dtype)
    if h_final is None and want_h_final:
        h_final = torch.empty((b, Dn, N), dtype=f32, device=x.device)
    _dev(h_final, "h_final", (b, Dn, N), f32)
    need = ssm_scan_fwd_workspace_ex(b, L, Dn, N, chunk_len)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(x_prev),
            _ptr(B_prev), _ptr(lam), _ptr(y), _ptr(h_final), b, L, Dn, N, io, chunk_len,
            _ptr(workspace), ws_bytes, _stream(x)]
    if events is not None:
        if len(events) != 4:
            raise ValueError("need exactly 4 event handles")
        handles = (ctypes.c_void_p * 4)(*[ctypes.c_void_p(e) for e in events])
        st = lib.ssm_scan_fwd_trap_profiled(*args, handles, 4)
    else:
        st = lib.ssm_scan_fwd_trap(*args)
    _check(st)
    return y, h_final


def _step_trap(fn_name, h, x_prev, B_prev, x, dt, A, B, C, D, z, y, lam):
    lib = load_library()
    Ln, S, Dn = x.shape
    N = A.shape[2]
    f32 = torch.float32
    _dev(h, "h", (Ln, S, Dn, N), f32)
    _dev(x, "x_t"); _dev(dt, "dt_t", (Ln, S, Dn)); _dev(z, "z_t", (Ln, S, Dn))
    _dev(A, "A", (Ln, Dn, N), f32); _dev(D, "D", (Ln, Dn), f32)
    _dev(B, "B_t", (Ln, S, N)); _dev(C, "C_t", (Ln, S, N))
    _dev(x_prev, "x_prev", (Ln, S, Dn)); _dev(B_prev, "B_prev", (Ln, S, N))
    _dev(lam, "lam_t", (Ln, S, Dn))
    io = _io(x, dt, z, B, C, x_prev, B_prev, lam)
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y_t", (Ln, S, Dn), x.dtype)
    st = getattr(lib, fn_name)(_ptr(h), _ptr(x_prev), _ptr(B_prev), _ptr(x), _ptr(dt), _ptr(lam),
                               _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(y), Ln, S, Dn, N,
                               io, _stream(x))
    _check(st)
    return y


def ssm_step_trap(h, x_prev, B_prev, x_t, dt_t, A, B_t, C_t, D, z_t=None, *, lam_t=None,
                  y_t=None):
    """One exponential-trapezoidal decode token: h updated in place, returns y_t.
    x_prev and B_prev are the previous token's x_t and B_t (None and None at the start);
    lam_t [n_layers, n_seq, d_inner] the token's weight (None: 1/2)."""
    return _step_trap("ssm_step_trap", h, x_prev, B_prev, x_t, dt_t, A, B_t, C_t, D, z_t, y_t,
                      lam_t)


def ssm_step_trap_replay(h, x_prev, B_prev, x_t, dt_t, A, B_t, C_t, D, z_t=None, *, lam_t=None,
                         y_t=None):
    """Reference-order replay of ssm_step_trap, one thread per channel."""
    return _step_trap("ssm_step_trap_replay", h, x_prev, B_prev, x_t, dt_t, A, B_t, C_t, D, z_t,
                      y_t, lam_t)


# ------------------------------------------------------------------ fused input stage
def _input_stage(conv_w, conv_b, dt_bias, lead, Dn, conv_k):
    f32 = torch.float32
    _dev(conv_w, "conv_w", lead + (Dn, conv_k), f32)
    _dev(conv_b, "conv_b", lead + (Dn,), f32)
    _dev(dt_bias, "dt_bias", lead + (Dn,), f32)


def ssm_scan_fwd_fused(x_in, dt_raw, A, B, C, D, z=None, h0=None, *, conv_w=None, conv_b=None,
                       conv_state0=None, dt_bias=None, chunk_len=0, y=None, h_final=None,
                       conv_state_out=None, workspace=None, want_h_final=True,
                       want_conv_state=True, events=None, states=None, u_out=None, dt_out=None):
    """Prefill with the MambaBlock input stage fused into the load: the scan runs on
    u = silu(causal depthwise conv(x_in)) and dt = softplus(dt_raw + dt_bias).
    conv_w [d_inner, K] (None: no convolution); conv_b, dt_bias [d_inner] or None;
    conv_state0 [b, K-1, d_inner] or None (zeros). Returns (y, h_final, conv_state_out).
    states, u_out, dt_out (see ssm_scan_fwd_fused_save): ssm_scan_fwd_fused_save stores
    them there."""
    lib = load_library()
    b, L, Dn = x_in.shape
    N = A.shape[1]
    f32 = torch.float32
    K = 0 if conv_w is None else conv_w.shape[-1]
    _dev(x_in, "x_in"); _dev(dt_raw, "dt_raw", (b, L, Dn)); _dev(z, "z", (b, L, Dn))
    _dev(A, "A", (Dn, N), f32); _dev(D, "D", (Dn,), f32)
    _dev(B, "B", (b, L, N)); _dev(C, "C", (b, L, N)); _dev(h0, "h0", (b, Dn, N), f32)
    _input_stage(conv_w, conv_b, dt_bias, (), Dn, K)
    io = _io(x_in, dt_raw, z, B, C)
    if K > 1:
        _dev(conv_state0, "conv_state0", (b, K - 1, Dn), x_in.dtype)
        if conv_state_out is None and want_conv_state:
            conv_state_out = torch.empty((b, K - 1, Dn), dtype=x_in.dtype, device=x_in.device)
        _dev(conv_state_out, "conv_state_out", (b, K - 1, Dn), x_in.dtype)
    else:
        conv_state0 = conv_state_out = None
    if y is None:
        y = torch.empty_like(x_in)
    _dev(y, "y", (b, L, Dn), x_in.dtype)
    if h_final is None and want_h_final:
        h_final = torch.empty((b, Dn, N), dtype=f32, device=x_in.device)
    _dev(h_final, "h_final", (b, Dn, N), f32)
    save = states is not None
    if save:
        _dev(states, "states", _states_shape(b, L, Dn, N), f32)
        _dev(u_out, "u_out", (b, L, Dn), x_in.dtype)
        _dev(dt_out, "dt_out", (b, L, Dn), x_in.dtype)
        if u_out is None or dt_out is None:
            raise ValueError("the fused training forward stores u and dt too: give u_out and dt_out")
    need = (ssm_scan_fwd_save_workspace if save else ssm_scan_fwd_workspace_ex)(b, L, Dn, N, chunk_len)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x_in.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    head = [_ptr(x_in), _ptr(dt_raw), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
            _ptr(conv_w), _ptr(conv_b), K, _ptr(conv_state0), _ptr(conv_state_out),
            _ptr(dt_bias), _ptr(y), _ptr(h_final)]
    tail = [b, L, Dn, N, io, chunk_len, _ptr(workspace), ws_bytes, _stream(x_in)]
    args = head + tail
    if save:
        if events is not None:
            raise ValueError("the fused training forward is not profiled")
        st = lib.ssm_scan_fwd_fused_save(*head, _ptr(states), _ptr(u_out), _ptr(dt_out), *tail)
        _check(st)
        return y, h_final, conv_state_out
    if events is not None:
        if len(events) != 4:
            raise ValueError("need exactly 4 event handles")
        handles = (ctypes.c_void_p * 4)(*[ctypes.c_void_p(e) for e in events])
        st = lib.ssm_scan_fwd_fused_profiled(*args, handles, 4)
    else:
        st = lib.ssm_scan_fwd_fused(*args)
    _check(st)
    return y, h_final, conv_state_out


def ssm_scan_fwd_fused_profiled(*a, events, **k):
    """ssm_scan_fwd_fused recording 4 HIP events at the kernel boundaries."""
    return ssm_scan_fwd_fused(*a, events=events, **k)


def ssm_scan_fwd_fused_save(x_in, dt_raw, A, B, C, D, z=None, h0=None, *, states=None, u_out=None,
                            dt_out=None, **k):
    """The fused training forward: ssm_scan_fwd_fused's results, the scan's state entering
    every 8th step (float32, shaped as _states_shape) and its inputs u and dt (x_in's
    dtype and shape) for ssm_scan_bwd_fused_saved.
    Returns (y, h_final, conv_state_out, states, u, dt)."""
    b, L, Dn = x_in.shape
    if states is None:
        states = torch.empty(_states_shape(b, L, Dn, A.shape[1]), dtype=torch.float32, device=x_in.device)
    if u_out is None:
        u_out = torch.empty_like(x_in)
    if dt_out is None:
        dt_out = torch.empty_like(x_in)
    y, hf, cs = ssm_scan_fwd_fused(x_in, dt_raw, A, B, C, D, z, h0, states=states, u_out=u_out,
                                   dt_out=dt_out, **k)
    return y, hf, cs, states, u_out, dt_out


def _step_fused(fn_name, h, conv_state, x, dt, A, B, C, D, z, conv_w, conv_b, dt_bias, y):
    lib = load_library()
    Ln, S, Dn = x.shape
    N = A.shape[2]
    f32 = torch.float32
    K = 0 if conv_w is None else conv_w.shape[-1]
    _dev(h, "h", (Ln, S, Dn, N), f32)
    _dev(x, "x_t"); _dev(dt, "dt_t", (Ln, S, Dn)); _dev(z, "z_t", (Ln, S, Dn))
    _dev(A, "A", (Ln, Dn, N), f32); _dev(D, "D", (Ln, Dn), f32)
    _dev(B, "B_t", (Ln, S, N)); _dev(C, "C_t", (Ln, S, N))
    _input_stage(conv_w, conv_b, dt_bias, (Ln,), Dn, K)
    if K > 1:
        if conv_state is None:
            raise ValueError("conv_state [n_layers, n_seq, K-1, d_inner] is required")
        _dev(conv_state, "conv_state", (Ln, S, K - 1, Dn), x.dtype)
    else:
        conv_state = None
    io = _io(x, dt, z, B, C)
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y_t", (Ln, S, Dn), x.dtype)
    st = getattr(lib, fn_name)(_ptr(h), _ptr(conv_state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                               _ptr(C), _ptr(D), _ptr(z), _ptr(conv_w), _ptr(conv_b), K,
                               _ptr(dt_bias), _ptr(y), Ln, S, Dn, N, io, _stream(x))
    _check(st)
    return y


def ssm_step_fused(h, conv_state, x_t, dt_t, A, B_t, C_t, D, z_t=None, *, conv_w=None,
                   conv_b=None, dt_bias=None, y_t=None):
    """One decode token through the input stage and the recurrence; h and conv_state
    [n_layers, n_seq, K-1, d_inner] are updated in place. Returns y_t."""
    return _step_fused("ssm_step_fused", h, conv_state, x_t, dt_t, A, B_t, C_t, D, z_t, conv_w,
                       conv_b, dt_bias, y_t)


def ssm_step_fused_replay(h, conv_state, x_t, dt_t, A, B_t, C_t, D, z_t=None, *, conv_w=None,
                          conv_b=None, dt_bias=None, y_t=None):
    """ssm_step_fused in its written-down order, one thread per channel."""
    return _step_fused("ssm_step_fused_replay", h, conv_state, x_t, dt_t, A, B_t, C_t, D, z_t,
                       conv_w, conv_b, dt_bias, y_t)


# ------------------------------------------------------------------ backward
def ssm_scan_bwd_workspace(batch, L, d_inner, d_state, chunk_len=0) -> int:
    return int(load_library().ssm_scan_bwd_workspace(batch, L, d_inner, d_state, chunk_len))


def ssm_scan_bwd(x, dt, A, B, C, D, z=None, h0=None, *, dy, dh_final=None, chunk_len=0,
                 want_dz=True, want_dh0=True, workspace=None, out=None):
    """Gradients of sum(dy * y) + sum(dh_final * h_final) of the real-state prefill.
    Returns a dict: dx, ddt, dz (io dtype, dz None when ungated or not wanted), dA, dB, dC,
    dD, dh0 (float32; dh0 None when not wanted). out: an optional dict of preallocated
    outputs with those names."""
    return _bwd("ssm_scan_bwd", x, dt, A, B, C, D, z, h0, None, dy, dh_final, chunk_len, want_dz,
                want_dh0, workspace, out)


def ssm_scan_bwd_saved_workspace(batch, L, d_inner, d_state, chunk_len=0) -> int:
    return int(load_library().ssm_scan_bwd_saved_workspace(batch, L, d_inner, d_state, chunk_len))


def ssm_scan_bwd_saved(x, dt, A, B, C, D, z=None, *, states, dy, dh_final=None, chunk_len=0,
                       want_dz=True, want_dh0=True, workspace=None, out=None):
    """ssm_scan_bwd with the states ssm_scan_fwd_save stored (see ssm_scan.h); the same
    dict of gradients."""
    return _bwd("ssm_scan_bwd_saved", x, dt, A, B, C, D, z, None, states, dy, dh_final, chunk_len,
                want_dz, want_dh0, workspace, out)


def _bwd(fn_name, x, dt, A, B, C, D, z, h0, states, dy, dh_final, chunk_len, want_dz, want_dh0,
         workspace, out):
    lib = load_library()
    b, L, Dn = x.shape
    N = A.shape[1]
    f32 = torch.float32
    _dev(x, "x"); _dev(dt, "dt", (b, L, Dn)); _dev(z, "z", (b, L, Dn)); _dev(dy, "dy", (b, L, Dn))
    _dev(A, "A", (Dn, N), f32); _dev(D, "D", (Dn,), f32)
    _dev(B, "B", (b, L, N)); _dev(C, "C", (b, L, N))
    _dev(h0, "h0", (b, Dn, N), f32); _dev(dh_final, "dh_final", (b, Dn, N), f32)
    saved = fn_name == "ssm_scan_bwd_saved"
    if saved:
        _dev(states, "states", _states_shape(b, L, Dn, N), f32)
    io = _io(x, dt, z, B, C, dy)
    out = dict(out or {})
    dev = x.device
    shapes = {"dx": ((b, L, Dn), x.dtype), "ddt": ((b, L, Dn), x.dtype),
              "dA": ((Dn, N), f32), "dB": ((b, L, N), f32), "dC": ((b, L, N), f32),
              "dD": ((Dn,), f32)}
    if z is not None and want_dz:
        shapes["dz"] = ((b, L, Dn), x.dtype)
    if want_dh0:
        shapes["dh0"] = ((b, Dn, N), f32)
    for k, (shp, dtp) in shapes.items():
        if out.get(k) is None:
            out[k] = torch.empty(shp, dtype=dtp, device=dev)
        _dev(out[k], k, shp, dtp)
    out.setdefault("dz", None)
    out.setdefault("dh0", None)
    need = (ssm_scan_bwd_saved_workspace if saved else ssm_scan_bwd_workspace)(b, L, Dn, N, chunk_len)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = getattr(lib, fn_name)(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(states if saved else h0),
        _ptr(dy), _ptr(dh_final), _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dz"]), _ptr(out["dA"]),
        _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dh0"]), b, L, Dn, N, io,
        chunk_len, _ptr(workspace), ws_bytes, _stream(x))
    _check(st)
    return out


def ssm_scan_bwd_fused_workspace(batch, L, d_inner, d_state, conv_k, io, chunk_len=0) -> int:
    return int(load_library().ssm_scan_bwd_fused_workspace(batch, L, d_inner, d_state, conv_k, io,
                                                           chunk_len))


def ssm_scan_bwd_fused_saved_workspace(batch, L, d_inner, d_state, conv_k, io, chunk_len=0) -> int:
    return int(load_library().ssm_scan_bwd_fused_saved_workspace(batch, L, d_inner, d_state, conv_k,
                                                                 io, chunk_len))


def ssm_scan_bwd_fused_saved(x_in, dt_raw, A, B, C, D, z=None, *, states, u, dt, **k):
    """ssm_scan_bwd_fused from the states, u and dt that ssm_scan_fwd_fused_save stored
    (see ssm_scan.h); the same dict of gradients."""
    return ssm_scan_bwd_fused(x_in, dt_raw, A, B, C, D, z, None, states=states, u=u, dt=dt, **k)


def ssm_scan_bwd_fused(x_in, dt_raw, A, B, C, D, z=None, h0=None, *, conv_w=None, conv_b=None,
                       conv_state0=None, dt_bias=None, dy, dh_final=None, chunk_len=0,
                       want_dz=True, want_dh0=True, want_dconv_state0=True, workspace=None,
                       states=None, u=None, dt=None):
    """Gradients of ssm_scan_fwd_fused's prefill (see ssm_scan.h). Returns a dict:
    dx_in, ddt_raw, dz (io dtype; dz None when ungated or not wanted), dA, dB, dC, dD,
    dh0, dconv_w, dconv_b, ddt_bias (float32; None when the input is absent or not
    wanted), dconv_state0 (io dtype, for conv_k >= 2). states, u, dt: from what the
    fused training forward stored (ssm_scan_bwd_fused_saved; h0 is then not given)."""
    lib = load_library()
    saved = states is not None
    b, L, Dn = x_in.shape
    N = A.shape[1]
    f32 = torch.float32
    K = 0 if conv_w is None else conv_w.shape[-1]
    _dev(x_in, "x_in"); _dev(dt_raw, "dt_raw", (b, L, Dn)); _dev(z, "z", (b, L, Dn))
    _dev(dy, "dy", (b, L, Dn))
    _dev(A, "A", (Dn, N), f32); _dev(D, "D", (Dn,), f32)
    _dev(B, "B", (b, L, N)); _dev(C, "C", (b, L, N)); _dev(h0, "h0", (b, Dn, N), f32)
    _dev(dh_final, "dh_final", (b, Dn, N), f32)
    _input_stage(conv_w, conv_b, dt_bias, (), Dn, K)
    io = _io(x_in, dt_raw, z, B, C, dy)
    if K > 1:
        _dev(conv_state0, "conv_state0", (b, K - 1, Dn), x_in.dtype)
    else:
        conv_state0 = None
    dev = x_in.device
    new = lambda shp, dtp: torch.empty(shp, dtype=dtp, device=dev)
    out = {"dx_in": new((b, L, Dn), x_in.dtype), "ddt_raw": new((b, L, Dn), x_in.dtype),
           "dz": new((b, L, Dn), x_in.dtype) if (z is not None and want_dz) else None,
           "dA": new((Dn, N), f32), "dB": new((b, L, N), f32), "dC": new((b, L, N), f32),
           "dD": new((Dn,), f32), "dh0": new((b, Dn, N), f32) if want_dh0 else None,
           "dconv_w": new((Dn, K), f32) if K else None,
           "dconv_b": new((Dn,), f32) if (K and conv_b is not None) else None,
           "ddt_bias": new((Dn,), f32) if dt_bias is not None else None,
           "dconv_state0": new((b, K - 1, Dn), x_in.dtype) if (K > 1 and want_dconv_state0) else None}
    if saved:
        if h0 is not None:
            raise ValueError("h0 is in the stored states")
        if u is None or dt is None:
            raise ValueError("the backward from stored states takes the forward's u and dt too")
        _dev(states, "states", _states_shape(b, L, Dn, N), f32)
        _dev(u, "u", (b, L, Dn), x_in.dtype)
        _dev(dt, "dt", (b, L, Dn), x_in.dtype)
    need = (ssm_scan_bwd_fused_saved_workspace if saved else ssm_scan_bwd_fused_workspace)(
        b, L, Dn, N, K, io, chunk_len)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lead = [_ptr(x_in), _ptr(dt_raw), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z)]
    lead += [_ptr(states), _ptr(u), _ptr(dt)] if saved else [_ptr(h0)]
    st = getattr(lib, "ssm_scan_bwd_fused_saved" if saved else "ssm_scan_bwd_fused")(
        *lead, _ptr(conv_w), _ptr(conv_b), K, _ptr(conv_state0), _ptr(dt_bias), _ptr(dy), _ptr(dh_final),
        _ptr(out["dx_in"]), _ptr(out["ddt_raw"]), _ptr(out["dz"]), _ptr(out["dA"]), _ptr(out["dB"]),
        _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dh0"]), _ptr(out["dconv_w"]),
        _ptr(out["dconv_b"]), _ptr(out["ddt_bias"]), _ptr(out["dconv_state0"]), b, L, Dn, N, io,
        chunk_len, _ptr(workspace), ws_bytes, _stream(x_in))
    _check(st)
    return out


class _SelectiveScan(torch.autograd.Function):
    """ssm_scan_fwd_ex forwards, ssm_scan_bwd backwards (both in the library's kernels)."""

    @staticmethod
    def forward(ctx, x, dt, A, B, C, D, z, h0, chunk_len, save_states):
        if save_states:
            y, h_final, states = ssm_scan_fwd_save(x, dt, A, B, C, D, z, h0, chunk_len=chunk_len)
        else:
            y, h_final = ssm_scan_fwd_ex(x, dt, A, B, C, D, z, h0, chunk_len=chunk_len)
            states = None
        ctx.save_for_backward(x, dt, A, B, C, D, z, h0, states)
        ctx.chunk_len = chunk_len
        return y, h_final

    @staticmethod
    def backward(ctx, dy, dh_final):
        x, dt, A, B, C, D, z, h0, states = ctx.saved_tensors
        need = ctx.needs_input_grad
        if dy is None:
            dy = torch.zeros_like(x)
        kw = dict(dy=dy.to(x.dtype).contiguous(),
                  dh_final=None if dh_final is None else dh_final.float().contiguous(),
                  chunk_len=ctx.chunk_len, want_dz=z is not None and need[6],
                  want_dh0=h0 is not None and need[7])
        if states is not None:
            g = ssm_scan_bwd_saved(x, dt, A, B, C, D, z, states=states, **kw)
        else:
            g = ssm_scan_bwd(x, dt, A, B, C, D, z, h0, **kw)
        cast = lambda t, like: None if t is None else t.to(like.dtype)
        grads = (g["dx"], g["ddt"], cast(g["dA"], A), cast(g["dB"], B), cast(g["dC"], C),
                 cast(g["dD"], D), g["dz"], g["dh0"], None, None)
        return tuple(gr if (i < len(need) and need[i]) else None for i, gr in enumerate(grads))


def selective_scan(x, dt, A, B, C, D, z=None, h0=None, *, chunk_len=0, save_states=False):
    """The real-state prefill as a differentiable function: returns (y, h_final), with
    gradients for x, dt, A, B, C, D, z and h0 from ssm_scan_bwd (dB, dC, dA and dD are
    computed in float32 and returned in their inputs' dtypes). save_states: the forward
    stores the state every 8 steps (ssm_scan_fwd_save) and the backward reads them
    (ssm_scan_bwd_saved) instead of recomputing them."""
    return _SelectiveScan.apply(x, dt, A, B, C, D, z, h0, chunk_len, save_states)


class _SelectiveScanFused(torch.autograd.Function):
    """ssm_scan_fwd_fused forwards, ssm_scan_bwd_fused backwards."""

    @staticmethod
    def forward(ctx, x_in, dt_raw, A, B, C, D, z, h0, conv_w, conv_b, conv_state0, dt_bias, chunk_len,
                save_states):
        kw = dict(conv_w=conv_w, conv_b=conv_b, conv_state0=conv_state0, dt_bias=dt_bias,
                  chunk_len=chunk_len, want_conv_state=False)
        if save_states:
            y, h_final, _, states, u, dt = ssm_scan_fwd_fused_save(x_in, dt_raw, A, B, C, D, z, h0, **kw)
        else:
            y, h_final, _ = ssm_scan_fwd_fused(x_in, dt_raw, A, B, C, D, z, h0, **kw)
            states = u = dt = None
        ctx.save_for_backward(x_in, dt_raw, A, B, C, D, z, h0, conv_w, conv_b, conv_state0, dt_bias,
                              states, u, dt)
        ctx.chunk_len = chunk_len
        return y, h_final

    @staticmethod
    def backward(ctx, dy, dh_final):
        x_in, dt_raw, A, B, C, D, z, h0, conv_w, conv_b, conv_state0, dt_bias, states, u, dt = ctx.saved_tensors
        need = ctx.needs_input_grad
        if dy is None:
            dy = torch.zeros_like(x_in)
        g = ssm_scan_bwd_fused(x_in, dt_raw, A, B, C, D, z, None if states is not None else h0,
                               conv_w=conv_w, conv_b=conv_b, conv_state0=conv_state0, dt_bias=dt_bias,
                               dy=dy.to(x_in.dtype).contiguous(),
                               dh_final=None if dh_final is None else dh_final.float().contiguous(),
                               chunk_len=ctx.chunk_len, want_dz=z is not None and need[6],
                               want_dh0=h0 is not None and need[7],
                               want_dconv_state0=conv_state0 is not None and need[10], states=states,
                               u=u, dt=dt)
        cast = lambda t, like: None if (t is None or like is None) else t.to(like.dtype)
        grads = (g["dx_in"], g["ddt_raw"], cast(g["dA"], A), cast(g["dB"], B), cast(g["dC"], C),
                 cast(g["dD"], D), g["dz"], g["dh0"], cast(g["dconv_w"], conv_w),
                 cast(g["dconv_b"], conv_b), g["dconv_state0"], cast(g["ddt_bias"], dt_bias), None, None)
        return tuple(gr if need[i] else None for i, gr in enumerate(grads))


def selective_scan_fused(x_in, dt_raw, A, B, C, D, z=None, h0=None, *, conv_w=None, conv_b=None,
                         conv_state0=None, dt_bias=None, chunk_len=0, save_states=False):
    """The fused prefill (input stage + scan) as a differentiable function: returns
    (y, h_final), with gradients for every tensor input from ssm_scan_bwd_fused.
    save_states: the forward stores the scan's state every 8 steps and its inputs u and dt
    (ssm_scan_fwd_fused_save), and the backward reads them (ssm_scan_bwd_fused_saved)."""
    return _SelectiveScanFused.apply(x_in, dt_raw, A, B, C, D, z, h0, conv_w, conv_b, conv_state0,
                                     dt_bias, chunk_len, save_states)


# ------------------------------------------------------------------ MIMO projections
def ssm_scan_fwd_mimo_workspace(batch, L, d_inner, d_state, rank, chunk_len=0) -> int:
    return int(load_library().ssm_scan_fwd_mimo_workspace(batch, L, d_inner, d_state, rank,
                                                          chunk_len))


def ssm_scan_fwd_mimo(x, dt, A, B, C, D, z=None, h0=None, *, chunk_len=0, y=None, h_final=None,
                      workspace=None, want_h_final=True, events=None):
    """Prefill with MIMO projections (see ssm_scan.h): x, z [b, L, d_inner, R]; dt
    [b, L, d_inner]; B, C [b, L, d_state, R]. Returns (y [b, L, d_inner, R], h_final)."""
    lib = load_library()
    b, L, Dn, R = x.shape
    N = A.shape[1]
    f32 = torch.float32
    _dev(x, "x"); _dev(dt, "dt", (b, L, Dn)); _dev(z, "z", (b, L, Dn, R))
    _dev(A, "A", (Dn, N), f32); _dev(D, "D", (Dn,), f32)
    _dev(B, "B", (b, L, N, R)); _dev(C, "C", (b, L, N, R)); _dev(h0, "h0", (b, Dn, N), f32)
    io = _io(x, dt, z, B, C)
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y", (b, L, Dn, R), x.dtype)
    if h_final is None and want_h_final:
        h_final = torch.empty((b, Dn, N), dtype=f32, device=x.device)
    _dev(h_final, "h_final", (b, Dn, N), f32)
    need = ssm_scan_fwd_mimo_workspace(b, L, Dn, N, R, chunk_len)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y),
            _ptr(h_final), b, L, Dn, N, R, io, chunk_len, _ptr(workspace), ws_bytes, _stream(x)]
    if events is not None:
        if len(events) != 4:
            raise ValueError("need exactly 4 event handles")
        handles = (ctypes.c_void_p * 4)(*[ctypes.c_void_p(e) for e in events])
        st = lib.ssm_scan_fwd_mimo_profiled(*args, handles, 4)
    else:
        st = lib.ssm_scan_fwd_mimo(*args)
    _check(st)
    return y, h_final


def ssm_step_mimo(h, x_t, dt_t, A, B_t, C_t, D, z_t=None, *, y_t=None):
    """One MIMO decode token: h [Ln, S, d_inner, N] updated in place; x_t, z_t
    [Ln, S, d_inner, R]; dt_t [Ln, S, d_inner]; B_t, C_t [Ln, S, N, R]. Returns y_t."""
    lib = load_library()
    Ln, S, Dn, R = x_t.shape
    N = A.shape[2]
    f32 = torch.float32
    _dev(h, "h", (Ln, S, Dn, N), f32)
    _dev(x_t, "x_t"); _dev(dt_t, "dt_t", (Ln, S, Dn)); _dev(z_t, "z_t", (Ln, S, Dn, R))
    _dev(A, "A", (Ln, Dn, N), f32); _dev(D, "D", (Ln, Dn), f32)
    _dev(B_t, "B_t", (Ln, S, N, R)); _dev(C_t, "C_t", (Ln, S, N, R))
    io = _io(x_t, dt_t, z_t, B_t, C_t)
    if y_t is None:
        y_t = torch.empty_like(x_t)
    _dev(y_t, "y_t", (Ln, S, Dn, R), x_t.dtype)
    st = lib.ssm_step_mimo(_ptr(h), _ptr(x_t), _ptr(dt_t), _ptr(A), _ptr(B_t), _ptr(C_t), _ptr(D),
                           _ptr(z_t), _ptr(y_t), Ln, S, Dn, N, R, io, _stream(x_t))
    _check(st)
    return y_t
