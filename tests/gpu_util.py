"""Helpers shared by the GPU tests: moving seeded inputs to the device,
calling the HIP path through the C ABI, and the parity error metric."""
from __future__ import annotations

import contextlib

import numpy as np

# Max relative error allowed against the fp64 oracle (fp32 state in both cases).
TOL = {"f32": 1e-4, "bf16": 2e-2}


def parity_error(got, ref) -> float:
    """max_i |g_i - r_i| / max(|r_i|, rms(r)): relative where r is not small,
    relative to the tensor's rms where it is (so values near zero do not
    make the ratio meaningless)."""
    g = np.asarray(got, np.float64).ravel()
    r = np.asarray(ref, np.float64).ravel()
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    den = np.maximum(np.abs(r), rms if rms > 0 else 1e-300)
    return float(np.max(np.abs(g - r) / den))


def torch_io(arr, io, device):
    """Host array -> device tensor of the I/O dtype (bf16 from the exact bf16 values)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    if io == "bf16":
        t = t.to(torch.bfloat16)  # values are already bf16-exact: no rounding happens
    return t.to(device)


def to_device(inp, device="cuda"):
    import torch

    def f32(x):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)

    return dict(u=torch_io(inp.u, inp.io, device), delta=torch_io(inp.delta, inp.io, device),
                A=f32(inp.A), B=torch_io(inp.B, inp.io, device), C=torch_io(inp.C, inp.io, device),
                delta_bias=f32(inp.delta_bias), Dskip=f32(inp.Dskip),
                z=None if inp.z is None else torch_io(inp.z, inp.io, device))


def to_host(t):
    import torch

    return t.detach().to(torch.float32).cpu().numpy()


def gpu_scan(inp, h0=None, device="cuda", softplus=None, dev_inputs=None):
    import torch
    from selective_state_space_22_amd import mamba_scan_fwd

    d = dev_inputs or to_device(inp, device)
    h0t = None if h0 is None else torch.from_numpy(np.ascontiguousarray(h0, np.float32)).to(device)
    out, last = mamba_scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["delta_bias"], d["Dskip"], d["z"],
                               inp.softplus if softplus is None else softplus, h0t, check=True)
    torch.cuda.synchronize()
    return to_host(out), to_host(last)


@contextlib.contextmanager
def library_option(option, value):
    """Set a process-wide library option (MAMBA_OPT_*) for the body of a with-block and
    restore the previous value afterwards; value None leaves the option as it is."""
    from selective_state_space_22_amd import binding

    old = binding.mamba_get_option(option)
    if value is not None:
        binding.mamba_set_option(option, value)
    try:
        yield
    finally:
        binding.mamba_set_option(option, old)


def force_engine(request, engine):
    """Pin the forward engine for one test ("default" = the library's own choice) and
    restore it when the test ends."""
    from selective_state_space_22_amd import binding

    cm = library_option(binding.MAMBA_OPT_ENGINE, binding.ENGINES["auto" if engine == "default" else engine])
    cm.__enter__()
    request.addfinalizer(lambda: cm.__exit__(None, None, None))
