"""mamba_scan_fwd_noalloc (the forward scan whose workspace is the library's fixed
per-GPU scratch array) against mamba_scan_fwd (the caller's workspace) through the
C ABI, on the GPU, and against the fp64 oracle.

Each case runs two calls in a row on the no-allocation entry point, the second on a
smaller input, so the second starts from the scratch contents the first left behind:
chained chunks (flags and carries in the scratch, which the kernels must clear) and
two-pass chunks (per-chunk aggregates).  The two entry points run the same kernels on
the same plan, so their results are compared bit for bit; both are held to the
oracle's tolerance (1e-4 for fp32 I/O, 2e-2 for bf16 I/O)."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, force_engine, library_option, parity_error, to_device, to_host
from selective_state_space_22_amd import binding
from selective_state_space_22_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(inp, label):
    d = to_device(inp)
    args = (d["u"], d["delta"], d["A"], d["B"], d["C"], d["delta_bias"], d["Dskip"], d["z"], True)
    ref_out, ref_last = binding.mamba_scan_fwd(*args, check=True)
    out = torch.empty_like(d["u"])
    last = torch.empty((inp.batch, inp.dim, inp.dstate), dtype=torch.float32, device="cuda")
    binding.mamba_scan_fwd_noalloc(*args, out=out, last_state=last, check=True)
    torch.cuda.synchronize()
    go, gl = to_host(out), to_host(last)
    assert np.array_equal(go, to_host(ref_out)), label
    assert np.array_equal(gl, to_host(ref_last)), label
    ro, rl = oracle.scan_inputs(inp)
    eo, el = parity_error(go, ro), parity_error(gl, rl)
    print(f"{label}: out err {eo:.3e} last err {el:.3e}, identical to mamba_scan_fwd", flush=True)
    assert eo <= TOL[inp.io] and el <= TOL[inp.io], label


# (engine, chunk option, first shape, second (smaller) shape); shape = (batch, L, D, N, io)
CASES = [
    ("wg", 256, (5, 1100, 4096, 16, "f32"), (3, 800, 6000, 16, "bf16")),       # chained chunks
    ("default", None, (2, 20000, 256, 16, "f32"), (1, 5000, 128, 16, "bf16")),  # two passes
    ("lane", None, (1, 8192, 64, 4, "f32"), (1, 3000, 64, 4, "bf16")),          # lane engine, chunked
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_scan_fwd_on_two_calls(case, request):
    _need_gpu()
    engine, chunk, first, second = case
    force_engine(request, engine)
    with library_option(binding.MAMBA_OPT_CHUNK, chunk):
        for i, shape in enumerate((first, second)):
            need = binding.mamba_scan_fwd_workspace_size(*shape[:4], 1 if shape[4] == "bf16" else 0)
            assert 0 < need <= binding.NOALLOC_MAX_WORKSPACE, (shape, need)
            print(f"\n[gpu-test] no-alloc scan call {i + 1}: {shape} engine={engine} scratch {need} B", flush=True)
            _both(W.generate(*shape, seed=600 + i), f"{engine} call {i + 1} {shape}")


def test_noalloc_rejects_a_workspace_beyond_its_scratch(request):
    """The chained workgroup engine at 16 k channel blocks needs 64 MiB of workspace:
    refused before anything is enqueued; the outputs stay untouched."""
    _need_gpu()
    force_engine(request, "wg")
    batch, L, D, N = 64, 1, 16384, 16
    assert binding.mamba_scan_fwd_workspace_size(batch, L, D, N, 0) > binding.NOALLOC_MAX_WORKSPACE
    x = torch.zeros((batch, L, D), dtype=torch.float32, device="cuda")
    bc = torch.zeros((batch, L, N), dtype=torch.float32, device="cuda")
    A = -torch.ones((D, N), dtype=torch.float32, device="cuda")
    out = torch.full_like(x, 7.0)
    with pytest.raises(binding.MambaError) as ex:
        binding.mamba_scan_fwd_noalloc(x, x, A, bc, bc, out=out)
    assert ex.value.status == 5  # MAMBA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
