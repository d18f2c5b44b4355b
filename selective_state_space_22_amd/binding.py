"""Thin ctypes binding of libmamba_mi355x.so (include/mamba_mi355x.h).

The functions keep the C names.  They only marshal torch tensors (device
memory, the current HIP stream) into the C ABI; every step of the scan runs
in the library's HIP kernels.  There is no fallback: if the library is
missing or the tensors are not on a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmamba_mi355x.so")

MAMBA_IO_F32 = 0
MAMBA_IO_BF16 = 1

# statuses that callers test for (the rest: see status_string)
MAMBA_OK = 0
MAMBA_ERR_TIMEOUT = 8
MAMBA_ERR_OPTION = 9

# options (enum mamba_option)
MAMBA_OPT_ENGINE = 1
MAMBA_OPT_CHUNK = 2
MAMBA_OPT_WG_WAVES = 3
MAMBA_OPT_FUSED_DT = 4
MAMBA_OPT_BWD_CHUNK = 5
MAMBA_OPT_GEMM_GENERAL = 6
MAMBA_OPT_SPIN_LIMIT = 7
MAMBA_OPT_AGG_SKIP = 8
ENGINES = {"auto": 0, "lane": 1, "wg": 2, "wp": 3}

_lib = None


class MambaError(RuntimeError):
    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__(f"{func} failed: status {status} ({status_string(status)})")


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load (once) and type the C ABI.  Raises if the shared library is absent."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with `python -m selective_state_space_22_amd.build`")
    lib = ctypes.CDLL(p)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    lib.mamba_version.argtypes = []
    lib.mamba_version.restype = I
    lib.mamba_status_string.argtypes = [I]
    lib.mamba_status_string.restype = ctypes.c_char_p
    lib.mamba_scan_fwd_workspace_size.argtypes = [I64, I64, I64, I64, I]
    lib.mamba_scan_fwd_workspace_size.restype = ctypes.c_size_t
    lib.mamba_scan_fwd.argtypes = [I64, I64, I64, I64, I, P, P, P, P, P, P, P, P, I, P, P, P, P, ctypes.c_size_t, P]
    lib.mamba_scan_fwd.restype = I
    lib.mamba_state_update.argtypes = [I64, I64, I64, I, P, P, P, P, P, P, P, P, P, I, P, P]
    lib.mamba_state_update.restype = I
    lib.mamba_scan_bwd_workspace_size.argtypes = [I64, I64, I64, I64, I]
    lib.mamba_scan_bwd_workspace_size.restype = ctypes.c_size_t
    lib.mamba_scan_bwd.argtypes = [I64, I64, I64, I64, I] + [P] * 8 + [I, P, P, P] + [P] * 9 + [P, ctypes.c_size_t, P]
    lib.mamba_scan_bwd.restype = I
    lib.mamba_selection_fwd_workspace_size.argtypes = [I64, I64, I64, I64, I64, I]
    lib.mamba_selection_fwd_workspace_size.restype = ctypes.c_size_t
    lib.mamba_selection_fwd.argtypes = [I64, I64, I64, I64, I64, I, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.mamba_selection_fwd.restype = I
    lib.mamba_ssm_fwd_workspace_size.argtypes = [I64, I64, I64, I64, I64, I]
    lib.mamba_ssm_fwd_workspace_size.restype = ctypes.c_size_t
    lib.mamba_ssm_fwd.argtypes = [I64, I64, I64, I64, I64, I, P, P, P, P, P, P, P, I, P, P, P, P, ctypes.c_size_t, P]
    lib.mamba_ssm_fwd.restype = I
    lib.mamba_scan_fwd_complex_workspace_size.argtypes = [I64, I64, I64, I64, I]
    lib.mamba_scan_fwd_complex_workspace_size.restype = ctypes.c_size_t
    lib.mamba_scan_fwd_complex.argtypes = lib.mamba_scan_fwd.argtypes
    lib.mamba_scan_fwd_complex.restype = I
    lib.mamba_state_update_complex.argtypes = lib.mamba_state_update.argtypes
    lib.mamba_state_update_complex.restype = I
    lib.mamba_block_fwd_workspace_size.argtypes = [I64, I64, I64, I64, I64, I64, I]
    lib.mamba_block_fwd_workspace_size.restype = ctypes.c_size_t
    lib.mamba_block_fwd.argtypes = [I64] * 6 + [I] + [P] * 8 + [I, P, P, P, P, ctypes.c_size_t, P]
    lib.mamba_block_fwd.restype = I
    lib.mamba_scan_fwd_noalloc.argtypes = [I64, I64, I64, I64, I, P, P, P, P, P, P, P, P, I, P, P, P, P]
    lib.mamba_scan_fwd_noalloc.restype = I
    lib.mamba_calibrate_copy.argtypes = [P, P, ctypes.c_size_t, I, P]
    lib.mamba_calibrate_copy.restype = I
    lib.mamba_set_option.argtypes = [I, I64]
    lib.mamba_set_option.restype = I
    lib.mamba_get_option.argtypes = [I]
    lib.mamba_get_option.restype = I64
    lib.mamba_stream_status.argtypes = [P]
    lib.mamba_stream_status.restype = I
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().mamba_status_string(int(status)).decode()


def mamba_version() -> int:
    return int(load_library().mamba_version())


def mamba_set_option(option: int, value: int) -> None:
    """Set a process-wide tuning option (MAMBA_OPT_*); raises on an unknown option or value."""
    st = load_library().mamba_set_option(int(option), int(value))
    if st != 0:
        raise MambaError("mamba_set_option", st)


def mamba_get_option(option: int) -> int:
    return int(load_library().mamba_get_option(int(option)))


def mamba_stream_status(device=None) -> int:
    """Synchronise the current stream of `device` and return the device's wait status
    (0, or MAMBA_ERR_TIMEOUT = 8 when a wait between sequence chunks gave up since the
    last query; the report is then cleared)."""
    import torch

    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    return int(load_library().mamba_stream_status(_stream(dev)))


def mamba_calibrate_copy(src, dst, blocks=2048):
    """Streaming copy of src into dst (same size, device tensors) with the library's
    hand-written copy kernel: the HBM reference of the memory-bound kernels."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes or not src.is_cuda or not dst.is_cuda:
        raise ValueError("src and dst must be device tensors of one size")
    st = load_library().mamba_calibrate_copy(src.data_ptr(), dst.data_ptr(), nbytes, int(blocks), _stream(src.device))
    if st != 0:
        raise MambaError("mamba_calibrate_copy", st)


def _check_status(func, device):
    st = mamba_stream_status(device)
    if st != 0:
        raise MambaError(func, st)


def _io_dtype(t):
    import torch

    if t.dtype == torch.float32:
        return MAMBA_IO_F32
    if t.dtype == torch.bfloat16:
        return MAMBA_IO_BF16
    raise TypeError(f"I/O tensors must be float32 or bfloat16, got {t.dtype}")


def _ptr(t, name, dtype=None, shape=None, device=None):
    """Device pointer of a contiguous tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr() if t.numel() > 0 else None


def _stream(device):
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def mamba_scan_fwd_workspace_size(batch: int, seqlen: int, dim: int, dstate: int, io_dtype: int) -> int:
    return int(load_library().mamba_scan_fwd_workspace_size(batch, seqlen, dim, dstate, io_dtype))


def mamba_scan_fwd(u, delta, A, B, C, delta_bias=None, Dskip=None, z=None, delta_softplus=True, h0=None,
                   out=None, last_state=None, workspace=None, return_last_state=True, check=False):
    """Forward selective scan.  u, delta, z: (batch, L, D); B, C: (batch, L, N); A: (D, N) float32.

    Returns (out, last_state); out has u's dtype, last_state is float32 (batch, D, N).
    check=True synchronises the stream and raises MambaError if a wait between
    sequence chunks gave up (mamba_stream_status); the default only enqueues."""
    import torch

    lib = load_library()
    batch, L, D = u.shape
    N = A.shape[1]
    io = _io_dtype(u)
    dev = u.device
    f32 = torch.float32
    if out is None:
        out = torch.empty_like(u)
    if last_state is None and return_last_state:
        last_state = torch.empty((batch, D, N), dtype=f32, device=dev)
    ws_bytes = mamba_scan_fwd_workspace_size(batch, L, D, N, io)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_ptr = _ptr(workspace, "workspace", device=dev)
    st = lib.mamba_scan_fwd(
        batch, L, D, N, io,
        _ptr(u, "u", u.dtype, (batch, L, D), dev), _ptr(delta, "delta", u.dtype, (batch, L, D), dev),
        _ptr(delta_bias, "delta_bias", f32, (D,), dev), _ptr(A, "A", f32, (D, N), dev),
        _ptr(B, "B", u.dtype, (batch, L, N), dev), _ptr(C, "C", u.dtype, (batch, L, N), dev),
        _ptr(Dskip, "Dskip", f32, (D,), dev), _ptr(z, "z", u.dtype, (batch, L, D), dev),
        int(bool(delta_softplus)), _ptr(h0, "h0", f32, (batch, D, N), dev),
        _ptr(out, "out", u.dtype, (batch, L, D), dev), _ptr(last_state, "last_state", f32, (batch, D, N), dev),
        ws_ptr, workspace.numel() * workspace.element_size() if workspace is not None else 0, _stream(dev))
    if st != 0:
        raise MambaError("mamba_scan_fwd", st)
    if check:
        _check_status("mamba_scan_fwd", dev)
    return out, last_state


NOALLOC_MAX_WORKSPACE = 32 << 20  # MAMBA_SCAN_FWD_NOALLOC_MAX_WORKSPACE


def mamba_scan_fwd_noalloc(u, delta, A, B, C, delta_bias=None, Dskip=None, z=None, delta_softplus=True, h0=None,
                           out=None, last_state=None, check=False):
    """mamba_scan_fwd through the entry point that allocates no device memory: its
    workspace is the library's fixed per-GPU scratch array.  Pass `out` (and
    `last_state`, or None to skip it) to allocate nothing here either; raises
    MambaError (MAMBA_ERR_WORKSPACE) when the shape needs more scratch than the
    array holds.  Calls that overlap on one GPU share that array and race."""
    import torch

    lib = load_library()
    batch, L, D = u.shape
    N = A.shape[1]
    io = _io_dtype(u)
    dev = u.device
    f32 = torch.float32
    if out is None:
        out = torch.empty_like(u)
    st = lib.mamba_scan_fwd_noalloc(
        batch, L, D, N, io,
        _ptr(u, "u", u.dtype, (batch, L, D), dev), _ptr(delta, "delta", u.dtype, (batch, L, D), dev),
        _ptr(delta_bias, "delta_bias", f32, (D,), dev), _ptr(A, "A", f32, (D, N), dev),
        _ptr(B, "B", u.dtype, (batch, L, N), dev), _ptr(C, "C", u.dtype, (batch, L, N), dev),
        _ptr(Dskip, "Dskip", f32, (D,), dev), _ptr(z, "z", u.dtype, (batch, L, D), dev),
        int(bool(delta_softplus)), _ptr(h0, "h0", f32, (batch, D, N), dev),
        _ptr(out, "out", u.dtype, (batch, L, D), dev), _ptr(last_state, "last_state", f32, (batch, D, N), dev),
        _stream(dev))
    if st != 0:
        raise MambaError("mamba_scan_fwd_noalloc", st)
    if check:
        _check_status("mamba_scan_fwd_noalloc", dev)
    return out, last_state


def mamba_scan_fwd_complex_workspace_size(batch: int, seqlen: int, dim: int, dstate: int, io_dtype: int) -> int:
    return int(load_library().mamba_scan_fwd_complex_workspace_size(batch, seqlen, dim, dstate, io_dtype))


def _re_im(t, name):
    """A complex64 tensor as its float32 (..., 2) re/im view; float32 (..., 2) tensors pass through."""
    import torch

    if t is None:
        return None
    if t.is_complex():
        if t.dtype != torch.complex64:
            raise TypeError(f"{name} must be complex64, got {t.dtype}")
        return torch.view_as_real(t.resolve_conj())
    return t


def mamba_scan_fwd_complex(u, delta, A, B, C, delta_bias=None, Dskip=None, z=None, delta_softplus=True, h0=None,
                           out=None, last_state=None, workspace=None, return_last_state=True, check=False):
    """Forward selective scan with a complex diagonal A; x, dt, B, C and out are real, y = Re(C . h).

    A: (D, N) complex64 or (D, N, 2) float32 re/im; h0 likewise (batch, D, N).  Other
    arguments as for mamba_scan_fwd.  Returns (out, last_state) with last_state
    complex64 (batch, D, N)."""
    import torch

    lib = load_library()
    batch, L, D = u.shape
    N = A.shape[1]
    A = _re_im(A, "A")
    h0 = _re_im(h0, "h0")
    io = _io_dtype(u)
    dev = u.device
    f32 = torch.float32
    if out is None:
        out = torch.empty_like(u)
    if last_state is None and return_last_state:
        last_state = torch.empty((batch, D, N, 2), dtype=f32, device=dev)
    else:
        last_state = _re_im(last_state, "last_state")
    ws_bytes = mamba_scan_fwd_complex_workspace_size(batch, L, D, N, io)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_ptr = _ptr(workspace, "workspace", device=dev)
    st = lib.mamba_scan_fwd_complex(
        batch, L, D, N, io,
        _ptr(u, "u", u.dtype, (batch, L, D), dev), _ptr(delta, "delta", u.dtype, (batch, L, D), dev),
        _ptr(delta_bias, "delta_bias", f32, (D,), dev), _ptr(A, "A", f32, (D, N, 2), dev),
        _ptr(B, "B", u.dtype, (batch, L, N), dev), _ptr(C, "C", u.dtype, (batch, L, N), dev),
        _ptr(Dskip, "Dskip", f32, (D,), dev), _ptr(z, "z", u.dtype, (batch, L, D), dev),
        int(bool(delta_softplus)), _ptr(h0, "h0", f32, (batch, D, N, 2), dev),
        _ptr(out, "out", u.dtype, (batch, L, D), dev),
        _ptr(last_state, "last_state", f32, (batch, D, N, 2), dev),
        ws_ptr, workspace.numel() * workspace.element_size() if workspace is not None else 0, _stream(dev))
    if st != 0:
        raise MambaError("mamba_scan_fwd_complex", st)
    if check:
        _check_status("mamba_scan_fwd_complex", dev)
    return out, (torch.view_as_complex(last_state) if last_state is not None else None)


def mamba_state_update(state, u, delta, A, B, C, delta_bias=None, Dskip=None, z=None, delta_softplus=True,
                       out=None):
    """One decode step in place on state (batch, D, N) float32.  u, delta, z: (batch, D); B, C: (batch, N)."""
    import torch

    lib = load_library()
    batch, D = u.shape
    N = A.shape[1]
    io = _io_dtype(u)
    dev = u.device
    f32 = torch.float32
    if out is None:
        out = torch.empty_like(u)
    st = lib.mamba_state_update(
        batch, D, N, io, _ptr(state, "state", f32, (batch, D, N), dev),
        _ptr(u, "u", u.dtype, (batch, D), dev), _ptr(delta, "delta", u.dtype, (batch, D), dev),
        _ptr(delta_bias, "delta_bias", f32, (D,), dev), _ptr(A, "A", f32, (D, N), dev),
        _ptr(B, "B", u.dtype, (batch, N), dev), _ptr(C, "C", u.dtype, (batch, N), dev),
        _ptr(Dskip, "Dskip", f32, (D,), dev), _ptr(z, "z", u.dtype, (batch, D), dev),
        int(bool(delta_softplus)), _ptr(out, "out", u.dtype, (batch, D), dev), _stream(dev))
    if st != 0:
        raise MambaError("mamba_state_update", st)
    return out


def mamba_state_update_complex(state, u, delta, A, B, C, delta_bias=None, Dskip=None, z=None, delta_softplus=True,
                               out=None):
    """One decode step with complex A, in place on state: (batch, D, N) complex64 or (batch, D, N, 2)
    float32.  A: (D, N) complex64 or (D, N, 2) float32; the rest as for mamba_state_update."""
    import torch

    lib = load_library()
    batch, D = u.shape
    N = A.shape[1]
    A = _re_im(A, "A")
    st_ri = _re_im(state, "state")
    io = _io_dtype(u)
    dev = u.device
    f32 = torch.float32
    if out is None:
        out = torch.empty_like(u)
    st = lib.mamba_state_update_complex(
        batch, D, N, io, _ptr(st_ri, "state", f32, (batch, D, N, 2), dev),
        _ptr(u, "u", u.dtype, (batch, D), dev), _ptr(delta, "delta", u.dtype, (batch, D), dev),
        _ptr(delta_bias, "delta_bias", f32, (D,), dev), _ptr(A, "A", f32, (D, N, 2), dev),
        _ptr(B, "B", u.dtype, (batch, N), dev), _ptr(C, "C", u.dtype, (batch, N), dev),
        _ptr(Dskip, "Dskip", f32, (D,), dev), _ptr(z, "z", u.dtype, (batch, D), dev),
        int(bool(delta_softplus)), _ptr(out, "out", u.dtype, (batch, D), dev), _stream(dev))
    if st != 0:
        raise MambaError("mamba_state_update_complex", st)
    return out


def mamba_scan_bwd_workspace_size(batch: int, seqlen: int, dim: int, dstate: int, io_dtype: int) -> int:
    return int(load_library().mamba_scan_bwd_workspace_size(batch, seqlen, dim, dstate, io_dtype))


def mamba_scan_bwd(u, delta, A, B, C, dout, delta_bias=None, Dskip=None, z=None, delta_softplus=True, h0=None,
                   dlast_state=None, grads=None, workspace=None, want=("dDskip", "dz", "ddelta_bias", "dh0")):
    """Backward of mamba_scan_fwd: gradients of sum(dout*out) + sum(dlast_state*last_state).

    Returns a dict with du, ddelta, dA, dB, dC and those of dDskip, dz (only
    with z), ddelta_bias, dh0 named in ``want``.  Preallocated outputs may be
    passed in ``grads`` (same keys)."""
    import torch

    lib = load_library()
    batch, L, D = u.shape
    N = A.shape[1]
    io = _io_dtype(u)
    dev = u.device
    f32 = torch.float32
    g = dict(grads or {})
    shapes = {"du": ((batch, L, D), u.dtype), "ddelta": ((batch, L, D), u.dtype), "dA": ((D, N), f32),
              "dB": ((batch, L, N), u.dtype), "dC": ((batch, L, N), u.dtype), "dDskip": ((D,), f32),
              "dz": ((batch, L, D), u.dtype), "ddelta_bias": ((D,), f32), "dh0": ((batch, D, N), f32)}
    need = ["du", "ddelta", "dA", "dB", "dC"] + [k for k in want if k != "dz" or z is not None]
    for k in need:
        if k not in g:
            shp, dt = shapes[k]
            g[k] = torch.empty(shp, dtype=dt, device=dev)
    ws_bytes = mamba_scan_bwd_workspace_size(batch, L, D, N, io)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def gp(k):
        if k not in g:
            return None
        shp, dt = shapes[k]
        return _ptr(g[k], k, dt, shp, dev)

    st = lib.mamba_scan_bwd(
        batch, L, D, N, io,
        _ptr(u, "u", u.dtype, (batch, L, D), dev), _ptr(delta, "delta", u.dtype, (batch, L, D), dev),
        _ptr(delta_bias, "delta_bias", f32, (D,), dev), _ptr(A, "A", f32, (D, N), dev),
        _ptr(B, "B", u.dtype, (batch, L, N), dev), _ptr(C, "C", u.dtype, (batch, L, N), dev),
        _ptr(Dskip, "Dskip", f32, (D,), dev), _ptr(z, "z", u.dtype, (batch, L, D), dev),
        int(bool(delta_softplus)), _ptr(h0, "h0", f32, (batch, D, N), dev),
        _ptr(dout, "dout", u.dtype, (batch, L, D), dev), _ptr(dlast_state, "dlast_state", f32, (batch, D, N), dev),
        gp("du"), gp("ddelta"), gp("dA"), gp("dB"), gp("dC"), gp("dDskip"), gp("dz"), gp("ddelta_bias"), gp("dh0"),
        _ptr(workspace, "workspace", device=dev),
        workspace.numel() * workspace.element_size() if workspace is not None else 0, _stream(dev))
    if st != 0:
        raise MambaError("mamba_scan_bwd", st)
    return {k: g[k] for k in need}


def mamba_selection_fwd_workspace_size(batch, seqlen, dim, dstate, dt_rank, io_dtype) -> int:
    return int(load_library().mamba_selection_fwd_workspace_size(batch, seqlen, dim, dstate, dt_rank, io_dtype))


def mamba_selection_fwd(x, W_x, W_dt, dstate, delta=None, B=None, C=None, workspace=None):
    """Selection projections: x (batch, L, D); W_x (R + 2N, D); W_dt (D, R).

    Returns (delta (batch, L, D), B (batch, L, N), C (batch, L, N)) in x's dtype."""
    import torch

    lib = load_library()
    batch, L, D = x.shape
    N = int(dstate)
    R = W_dt.shape[1]
    io = _io_dtype(x)
    dev = x.device
    delta = torch.empty_like(x) if delta is None else delta
    B = torch.empty((batch, L, N), dtype=x.dtype, device=dev) if B is None else B
    C = torch.empty((batch, L, N), dtype=x.dtype, device=dev) if C is None else C
    ws_bytes = mamba_selection_fwd_workspace_size(batch, L, D, N, R, io)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    st = lib.mamba_selection_fwd(
        batch, L, D, N, R, io, _ptr(x, "x", x.dtype, (batch, L, D), dev), _ptr(W_x, "W_x", x.dtype, (R + 2 * N, D), dev),
        _ptr(W_dt, "W_dt", x.dtype, (D, R), dev), _ptr(delta, "delta", x.dtype, (batch, L, D), dev),
        _ptr(B, "B", x.dtype, (batch, L, N), dev), _ptr(C, "C", x.dtype, (batch, L, N), dev),
        _ptr(workspace, "workspace", device=dev),
        workspace.numel() * workspace.element_size() if workspace is not None else 0, _stream(dev))
    if st != 0:
        raise MambaError("mamba_selection_fwd", st)
    return delta, B, C


def mamba_ssm_fwd_workspace_size(batch, seqlen, dim, dstate, dt_rank, io_dtype) -> int:
    return int(load_library().mamba_ssm_fwd_workspace_size(batch, seqlen, dim, dstate, dt_rank, io_dtype))


def mamba_ssm_fwd(x, W_x, W_dt, A, z=None, dt_bias=None, Dskip=None, delta_softplus=True, h0=None, out=None,
                  last_state=None, workspace=None, return_last_state=True, check=False):
    """Selection projections followed by the scan (u = x).  Returns (out, last_state)."""
    import torch

    lib = load_library()
    batch, L, D = x.shape
    N = A.shape[1]
    R = W_dt.shape[1]
    io = _io_dtype(x)
    dev = x.device
    f32 = torch.float32
    out = torch.empty_like(x) if out is None else out
    if last_state is None and return_last_state:
        last_state = torch.empty((batch, D, N), dtype=f32, device=dev)
    ws_bytes = mamba_ssm_fwd_workspace_size(batch, L, D, N, R, io)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    st = lib.mamba_ssm_fwd(
        batch, L, D, N, R, io, _ptr(x, "x", x.dtype, (batch, L, D), dev), _ptr(z, "z", x.dtype, (batch, L, D), dev),
        _ptr(W_x, "W_x", x.dtype, (R + 2 * N, D), dev), _ptr(W_dt, "W_dt", x.dtype, (D, R), dev),
        _ptr(dt_bias, "dt_bias", f32, (D,), dev), _ptr(A, "A", f32, (D, N), dev), _ptr(Dskip, "Dskip", f32, (D,), dev),
        int(bool(delta_softplus)), _ptr(h0, "h0", f32, (batch, D, N), dev), _ptr(out, "out", x.dtype, (batch, L, D), dev),
        _ptr(last_state, "last_state", f32, (batch, D, N), dev), _ptr(workspace, "workspace", device=dev),
        workspace.numel() * workspace.element_size() if workspace is not None else 0, _stream(dev))
    if st != 0:
        raise MambaError("mamba_ssm_fwd", st)
    if check:
        _check_status("mamba_ssm_fwd", dev)
    return out, last_state


def mamba_block_fwd_workspace_size(batch, seqlen, d_model, dim, dstate, dt_rank, io_dtype) -> int:
    return int(load_library().mamba_block_fwd_workspace_size(batch, seqlen, d_model, dim, dstate, dt_rank, io_dtype))


def mamba_block_fwd(hidden, W_in, W_x, W_dt, A, W_out, dt_bias=None, Dskip=None, delta_softplus=True, h0=None,
                    out=None, last_state=None, workspace=None, return_last_state=True, check=False):
    """One Mamba block: hidden (batch, L, d_model); W_in (2 D, d_model); W_out (d_model, D);
    W_x, W_dt, A, dt_bias, Dskip as for mamba_ssm_fwd.  Returns (out (batch, L, d_model), last_state)."""
    import torch

    lib = load_library()
    batch, L, dm = hidden.shape
    D = W_out.shape[1]
    N = A.shape[1]
    R = W_dt.shape[1]
    io = _io_dtype(hidden)
    dev = hidden.device
    f32 = torch.float32
    t = hidden.dtype
    out = torch.empty_like(hidden) if out is None else out
    if last_state is None and return_last_state:
        last_state = torch.empty((batch, D, N), dtype=f32, device=dev)
    ws_bytes = mamba_block_fwd_workspace_size(batch, L, dm, D, N, R, io)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    st = lib.mamba_block_fwd(
        batch, L, dm, D, N, R, io, _ptr(hidden, "hidden", t, (batch, L, dm), dev),
        _ptr(W_in, "W_in", t, (2 * D, dm), dev), _ptr(W_x, "W_x", t, (R + 2 * N, D), dev),
        _ptr(W_dt, "W_dt", t, (D, R), dev), _ptr(dt_bias, "dt_bias", f32, (D,), dev), _ptr(A, "A", f32, (D, N), dev),
        _ptr(Dskip, "Dskip", f32, (D,), dev), _ptr(W_out, "W_out", t, (dm, D), dev), int(bool(delta_softplus)),
        _ptr(h0, "h0", f32, (batch, D, N), dev), _ptr(out, "out", t, (batch, L, dm), dev),
        _ptr(last_state, "last_state", f32, (batch, D, N), dev), _ptr(workspace, "workspace", device=dev),
        workspace.numel() * workspace.element_size() if workspace is not None else 0, _stream(dev))
    if st != 0:
        raise MambaError("mamba_block_fwd", st)
    if check:
        _check_status("mamba_block_fwd", dev)
    return out, last_state
