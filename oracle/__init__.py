"""fp64 CPU oracle of the selective scan (S6) -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(``selective_state_space_22_amd``) and the library never imports it.

Two independent implementations of the same definition live here:
  * ``scan`` / ``step``: the C oracle ``s6_oracle.c`` (fp64, libm, OpenMP over
    (batch, channel)), called through ctypes;
  * ``scan_numpy``: a numpy fp64 twin vectorised over (batch, channel, state)
    with a Python loop over tokens, used to cross-check the C code;
  * ``scan_bwd``: the C oracle's backward, the derivative of the same
    definition, pinned against central finite differences of ``scan``;
  * ``scan_complex``: the forward with complex diagonal A (the page's
    -1/2 + ni initialisation), real x, B, C and output Re(C . h);
  * ``selection``: the section 3.2 projections (B, C = Linear_N(x), dt from a
    rank-R projection of x expanded to the D channels), fp64 matrix products;
  * ``block``: a Mamba block as Figure 3 and section 5 describe it (input
    projection to a SiLU-activated SSM branch and a gate branch, the selective
    SSM, output projection), composed of ``selection`` and ``scan``.
Both follow "Mamba 状态空间模型原理与 Transformer 对比" (kb.agiseed.tech):
section 2.1 eq. (2) (ZOH), eq. (3a)/(3b) (recurrence and readout),
section 3.2 (selection: per-token dt through softplus, B/C shared by channels)
and the Figure 3 caption (SiLU gate).  Readings where the page is silent:
bias before softplus, skip term Dskip*x before the gate, gate z*sigmoid(z),
zero initial state unless h0 is given.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "s6_oracle.c")
_LIB = os.path.join(_HERE, "libs6oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (fp64, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
               "-ffp-contract=off", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.s6_oracle_scan.argtypes = [I64, I64, I64, I64, P, P, P, P, P, P, P, P, ctypes.c_int, P, P, P, ctypes.c_int]
        lib.s6_oracle_scan.restype = ctypes.c_int
        lib.s6_oracle_step.argtypes = [I64, I64, I64, P, P, P, P, P, P, P, P, P, ctypes.c_int, P, ctypes.c_int]
        lib.s6_oracle_step.restype = ctypes.c_int
        lib.s6_oracle_scan_bwd.argtypes = [I64, I64, I64, I64] + [P] * 8 + [ctypes.c_int] + [P] * 12 + [ctypes.c_int]
        lib.s6_oracle_scan_bwd.restype = ctypes.c_int
        lib.s6_oracle_scan_complex.argtypes = [I64, I64, I64, I64, P, P, P, P, P, P, P, P, ctypes.c_int, P, P, P,
                                               ctypes.c_int]
        lib.s6_oracle_scan_complex.restype = ctypes.c_int
        lib.s6_oracle_max_threads.argtypes = []
        lib.s6_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().s6_oracle_max_threads())


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def scan(u, delta, A, B, C, delta_bias=None, Dskip=None, z=None, softplus=True, h0=None,
         nthreads: int | None = None):
    """fp64 forward scan.  Returns (out (batch,L,D), last_state (batch,D,N))."""
    u, delta, A, B, C = (_f64(x) for x in (u, delta, A, B, C))
    delta_bias, Dskip, z, h0 = (_f64(x) for x in (delta_bias, Dskip, z, h0))
    batch, L, D = u.shape
    N = A.shape[1]
    assert delta.shape == u.shape and A.shape == (D, N)
    assert B.shape == (batch, L, N) and C.shape == (batch, L, N)
    assert z is None or z.shape == u.shape
    assert h0 is None or h0.shape == (batch, D, N)
    out = np.empty((batch, L, D), dtype=np.float64)
    last = np.empty((batch, D, N), dtype=np.float64)
    nt = nthreads if nthreads else max_threads()
    rc = _load().s6_oracle_scan(batch, L, D, N, _ptr(u), _ptr(delta), _ptr(delta_bias), _ptr(A), _ptr(B), _ptr(C),
                                _ptr(Dskip), _ptr(z), int(bool(softplus)), _ptr(h0), _ptr(out), _ptr(last), nt)
    if rc != 0:
        raise RuntimeError(f"s6_oracle_scan failed with {rc}")
    return out, last


def step(state, u, delta, A, B, C, delta_bias=None, Dskip=None, z=None, softplus=True, nthreads: int | None = None):
    """One fp64 decode step.  state (batch,D,N) is copied, advanced and returned with out (batch,D)."""
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    u, delta, A, B, C = (_f64(x) for x in (u, delta, A, B, C))
    delta_bias, Dskip, z = (_f64(x) for x in (delta_bias, Dskip, z))
    batch, D = u.shape
    N = A.shape[1]
    assert st.shape == (batch, D, N) and B.shape == (batch, N) and C.shape == (batch, N)
    out = np.empty((batch, D), dtype=np.float64)
    nt = nthreads if nthreads else max_threads()
    rc = _load().s6_oracle_step(batch, D, N, _ptr(st), _ptr(u), _ptr(delta), _ptr(delta_bias), _ptr(A), _ptr(B),
                                _ptr(C), _ptr(Dskip), _ptr(z), int(bool(softplus)), _ptr(out), nt)
    if rc != 0:
        raise RuntimeError(f"s6_oracle_step failed with {rc}")
    return out, st


def scan_complex(u, delta, A, B, C, delta_bias=None, Dskip=None, z=None, softplus=True, h0=None,
                 nthreads: int | None = None):
    """fp64 forward scan with complex diagonal A (D, N) (a numpy complex array).
    Returns (out (batch, L, D) real, last_state (batch, D, N) complex); h0 complex or None."""
    u, delta, B, C = (_f64(x) for x in (u, delta, B, C))
    delta_bias, Dskip, z = (_f64(x) for x in (delta_bias, Dskip, z))
    Ac = np.ascontiguousarray(np.stack([np.real(A), np.imag(A)], axis=-1), dtype=np.float64)
    h0c = None if h0 is None else np.ascontiguousarray(np.stack([np.real(h0), np.imag(h0)], axis=-1), np.float64)
    batch, L, D = u.shape
    N = Ac.shape[1]
    out = np.empty((batch, L, D))
    last = np.empty((batch, D, N, 2))
    nt = nthreads if nthreads else max_threads()
    rc = _load().s6_oracle_scan_complex(batch, L, D, N, _ptr(u), _ptr(delta), _ptr(delta_bias), _ptr(Ac), _ptr(B),
                                        _ptr(C), _ptr(Dskip), _ptr(z), int(bool(softplus)), _ptr(h0c), _ptr(out),
                                        _ptr(last), nt)
    if rc != 0:
        raise RuntimeError(f"s6_oracle_scan_complex failed with {rc}")
    return out, last[..., 0] + 1j * last[..., 1]


def scan_bwd(u, delta, A, B, C, dout, delta_bias=None, Dskip=None, z=None, softplus=True, h0=None, dlast=None,
             nthreads: int | None = None):
    """fp64 gradients of sum(dout*out) + sum(dlast*last_state).

    Returns a dict with du, ddelta, dA, dB, dC and, when the matching input is
    given, dDskip, dz, dbias, dh0."""
    u, delta, A, B, C, dout = (_f64(x) for x in (u, delta, A, B, C, dout))
    delta_bias, Dskip, z, h0, dlast = (_f64(x) for x in (delta_bias, Dskip, z, h0, dlast))
    batch, L, D = u.shape
    N = A.shape[1]
    assert dout.shape == u.shape and (dlast is None or dlast.shape == (batch, D, N))
    g = {"du": np.empty((batch, L, D)), "ddelta": np.empty((batch, L, D)), "dA": np.empty((D, N)),
         "dB": np.empty((batch, L, N)), "dC": np.empty((batch, L, N))}
    g["dDskip"] = np.empty(D) if Dskip is not None else None
    g["dz"] = np.empty((batch, L, D)) if z is not None else None
    g["dbias"] = np.empty(D) if delta_bias is not None else None
    g["dh0"] = np.empty((batch, D, N)) if h0 is not None else None
    nt = nthreads if nthreads else max_threads()
    rc = _load().s6_oracle_scan_bwd(batch, L, D, N, _ptr(u), _ptr(delta), _ptr(delta_bias), _ptr(A), _ptr(B),
                                    _ptr(C), _ptr(Dskip), _ptr(z), int(bool(softplus)), _ptr(h0), _ptr(dout),
                                    _ptr(dlast), _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]),
                                    _ptr(g["dC"]), _ptr(g["dDskip"]), _ptr(g["dz"]), _ptr(g["dbias"]),
                                    _ptr(g["dh0"]), nt)
    if rc != 0:
        raise RuntimeError(f"s6_oracle_scan_bwd failed with {rc}")
    return {k: v for k, v in g.items() if v is not None}


def scan_inputs(inp, h0=None, nthreads=None, softplus=None):
    """Oracle scan of a ``workloads.ScanInputs`` (uses the exact values the GPU sees)."""
    sp = inp.softplus if softplus is None else softplus
    return scan(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.delta_bias, inp.Dskip, inp.z, sp, h0, nthreads)


def scan_numpy(u, delta, A, B, C, delta_bias=None, Dskip=None, z=None, softplus=True, h0=None):
    """Independent numpy fp64 twin of ``scan`` (vectorised over batch, channel, state)."""
    u = np.asarray(u, np.float64)
    dt = np.asarray(delta, np.float64)
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    C = np.asarray(C, np.float64)
    batch, L, D = u.shape
    N = A.shape[1]
    if delta_bias is not None:
        dt = dt + np.asarray(delta_bias, np.float64)[None, None, :]
    if softplus:
        dt = np.logaddexp(0.0, dt)  # log(e^0 + e^v)
    h = np.zeros((batch, D, N)) if h0 is None else np.array(h0, np.float64, copy=True)
    out = np.empty((batch, L, D))
    for t in range(L):
        x = dt[:, t, :, None] * A[None, :, :]                         # (batch, D, N)
        abar = np.exp(x)
        safe = np.where(x == 0.0, 1.0, x)
        phi = np.where(x == 0.0, 1.0, np.expm1(x) / safe)
        bbar = phi * dt[:, t, :, None] * B[:, t, None, :]
        h = abar * h + bbar * u[:, t, :, None]
        y = np.einsum("bdn,bn->bd", h, C[:, t, :])
        if Dskip is not None:
            y = y + np.asarray(Dskip, np.float64)[None, :] * u[:, t, :]
        if z is not None:
            zt = np.asarray(z, np.float64)[:, t, :]
            y = y * (zt / (1.0 + np.exp(-zt)))
        out[:, t, :] = y
    return out, h


def selection(x, W_x, W_dt, dstate, store=None, store_delta=True):
    """fp64 selection projections (section 3.2).  x (batch, L, D), W_x (R + 2N, D),
    W_dt (D, R).  Returns (delta_raw (batch, L, D), B (batch, L, N), C (batch, L, N)):
    xdbl = x W_x^T; B, C = its columns R..R+N and R+N..R+2N; delta = xdbl[:, :R] W_dt^T.

    ``store`` (optional) maps an fp64 array to the values of the type the
    projected tensors are kept in (xdbl before the dt projection, and the three
    results); None keeps fp64 throughout.  ``store_delta=False`` leaves delta
    unrounded (a consumer that projects dt itself never stores it)."""
    keep = store if store is not None else (lambda a: a)
    x = np.asarray(x, np.float64)
    W_x = np.asarray(W_x, np.float64)
    W_dt = np.asarray(W_dt, np.float64)
    R = W_dt.shape[1]
    N = int(dstate)
    assert W_x.shape == (R + 2 * N, x.shape[-1]) and W_dt.shape == (x.shape[-1], R)
    xdbl = keep(x @ W_x.T)
    delta = xdbl[..., :R] @ W_dt.T
    if store_delta:
        delta = keep(delta)
    return delta, np.ascontiguousarray(xdbl[..., R:R + N]), np.ascontiguousarray(xdbl[..., R + N:])


def _silu64(v):
    v = np.asarray(v, np.float64)
    return v / (1.0 + np.exp(-v))


def block(hidden, W_in, W_x, W_dt, dt_bias, A, Dskip, W_out, dstate, softplus=True, h0=None, store=None,
          nthreads: int | None = None):
    """fp64 forward of one Mamba block (Figure 3; section 5: the block widens the
    model dimension by an expansion factor through linear projections around the SSM).
    hidden (batch, L, d_model); W_in (2 D, d_model): its first D rows project to the
    SSM branch, the last D rows to the gate branch; W_out (d_model, D).
        x   = SiLU(hidden W_in[:D]^T)        (the activation that replaces H3's first gate)
        z   = hidden W_in[D:]^T              (the gate branch)
        delta, B, C = selection(x, W_x, W_dt)
        y   = scan(x, delta, A, B, C, dt_bias, Dskip, z)   (skip term, then the SiLU(z) gate)
        out = y W_out^T
    The page shows no convolution in the block; none is applied.  ``store`` maps
    fp64 values to the type the intermediate per-token tensors (x, z, the selection
    results, y) are kept in; None keeps fp64.  Returns (out, last_state)."""
    keep = store if store is not None else (lambda a: a)
    hidden = np.asarray(hidden, np.float64)
    W_in = np.asarray(W_in, np.float64)
    W_out = np.asarray(W_out, np.float64)
    D = W_in.shape[0] // 2
    assert W_in.shape == (2 * D, hidden.shape[-1]) and W_out.shape == (hidden.shape[-1], D)
    x = keep(_silu64(hidden @ W_in[:D].T))
    z = keep(hidden @ W_in[D:].T)
    delta, B, C = selection(x, W_x, W_dt, dstate, store=store)
    y, last = scan(x, delta, A, B, C, dt_bias, Dskip, z, softplus, h0, nthreads=nthreads)
    return keep(y) @ W_out.T, last
