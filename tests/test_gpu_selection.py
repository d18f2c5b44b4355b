"""Selection front end (section 3.2 projections, on the matrix cores) and the
selective SSM that runs it before the scan, against the fp64 oracle on the GPU.

Tolerances: 1e-4 for fp32 I/O and 2e-2 for bf16 I/O (parity_error, as for the
scan).  The products accumulate in fp32 over D (x_proj) or R (dt_proj) terms.
With bf16 I/O the projected tensors (xdbl, delta, B, C) are bf16 tensors, like
every other per-token tensor of that I/O type; the oracle keeps the same
storage type for them (fp64 arithmetic, results rounded to bf16 where they are
stored), so the comparison measures the kernels, not the storage choice."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, library_option, parity_error, to_device, to_host, torch_io
from selective_state_space_22_amd import binding
from selective_state_space_22_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _announce(msg):
    print(f"\n[gpu-test] {msg}", flush=True)


def _store(io):
    if io != "bf16":
        return None
    return lambda a: W.bf16_round(np.asarray(a, np.float32))[1].reshape(np.shape(a)).astype(np.float64)


def _inputs(batch, L, D, N, R, io, seed):
    inp = W.generate(batch, L, D, N, io, seed=seed)
    sw = W.selection_weights(D, N, R, io, seed=seed)
    return inp, sw


def _gpu_selection(inp, sw, N):
    from selective_state_space_22_amd import mamba_selection_fwd

    x = torch_io(inp.u, inp.io, "cuda")
    wx = torch_io(sw.W_x, inp.io, "cuda")
    wdt = torch_io(sw.W_dt, inp.io, "cuda")
    d, B, C = mamba_selection_fwd(x, wx, wdt, N)
    torch.cuda.synchronize()
    return to_host(d), to_host(B), to_host(C)


@pytest.mark.parametrize("case", [
    (2, 77, 96, 16, 8, "f32"),     # both products on MFMA, ragged M, N = 40 columns
    (2, 77, 96, 16, 6, "f32"),     # dt rank not a multiple of 4: dt projection on the vector path
    (1, 1, 64, 16, 4, "f32"),      # one token
    (2, 300, 136, 16, 16, "bf16"),
    (1, 50, 70, 8, 5, "bf16"),     # D and R not multiples of 8: vector path for both
    (3, 129, 1536, 16, 48, "bf16"),  # Mamba-130M layer width and dt rank
    (1, 64, 256, 1, 1, "f32"),     # the page's rank-one dt projection, N = 1
], ids=str)
def test_selection_matches_oracle(case):
    _need_gpu()
    batch, L, D, N, R, io = case
    _announce(f"selection {case}")
    inp, sw = _inputs(batch, L, D, N, R, io, seed=300 + L + R)
    got = _gpu_selection(inp, sw, N)
    ref = oracle.selection(inp.u, sw.W_x, sw.W_dt, N, store=_store(io))
    errs = [parity_error(g, r) for g, r in zip(got, ref)]
    print(f"{case}: delta {errs[0]:.2e} B {errs[1]:.2e} C {errs[2]:.2e}")
    assert max(errs) <= TOL[io], errs


def test_selection_mamba3b_layer_sampled_rows():
    """Full Mamba-3B layer shape (M = 16384 token rows, D 5120, R 160); the oracle on 256 sampled rows."""
    _need_gpu()
    _announce("selection mamba3b_layer (4, 4096, 5120, 16, R 160) bf16, 256 sampled token rows")
    inp = W.generate_workload("mamba3b_layer")
    sw = W.selection_weights(5120, 16, W.dt_rank_for(5120), "bf16", seed=W.WORKLOADS["mamba3b_layer"].seed)
    got = _gpu_selection(inp, sw, 16)
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(4 * 4096, 256, replace=False))
    x = inp.u.reshape(-1, 5120)[rows][None]
    ref = oracle.selection(x, sw.W_x, sw.W_dt, 16, store=_store("bf16"))
    errs = [parity_error(g.reshape(-1, g.shape[-1])[rows][None], r) for g, r in zip(got, ref)]
    print(f"mamba3b selection: delta {errs[0]:.2e} B {errs[1]:.2e} C {errs[2]:.2e}")
    assert max(errs) <= TOL["bf16"], errs


SSM_CASES = [
    # batch, L, D, N, io, dt rank (None: d_model/16).  With the fused projection switched on, the
    # workgroup engine projects dt on the matrix cores when the rank's rows are 16-byte
    # multiples; otherwise (and by default) a GEMM writes delta
    (1, 256, 64, 16, "f32", None),       # R 2: unfused
    (2, 300, 130, 16, "f32", None),      # R 5: unfused
    (2, 1000, 1536, 16, "bf16", None),   # R 48: fused, chained chunks
    (2, 300, 256, 16, "f32", 8),         # fused fp32 (four MFMAs per K slice), ragged tail
    (1, 777, 5120, 16, "bf16", 160),     # fused, Mamba-3B width and rank
    (2, 400, 128, 8, "bf16", 16),        # fused, N = 8 (four waves)
    (1, 8192, 64, 16, "f32", 8),         # fused, one channel block: two-pass chunked mode
    (2, 129, 200, 16, "bf16", 256),      # fused at the largest rank kept in registers
]


@pytest.mark.parametrize("fused", ["on", "off"])
@pytest.mark.parametrize("case", SSM_CASES, ids=str)
def test_ssm_matches_selection_then_scan_oracle(case, fused, request):
    _need_gpu()
    from selective_state_space_22_amd import mamba_ssm_fwd

    batch, L, D, N, io, R = case
    R = R or W.dt_rank_for(D)
    cm = library_option(binding.MAMBA_OPT_FUSED_DT, 1 if fused == "on" else 0)
    cm.__enter__()
    request.addfinalizer(lambda: cm.__exit__(None, None, None))
    _announce(f"ssm (selection + scan) {case} R {R} fused={fused}")
    inp, sw = _inputs(batch, L, D, N, R, io, seed=400 + L)
    d = to_device(inp)
    out, last = mamba_ssm_fwd(d["u"], torch_io(sw.W_x, io, "cuda"), torch_io(sw.W_dt, io, "cuda"), d["A"], z=d["z"],
                              dt_bias=d["delta_bias"], Dskip=d["Dskip"])
    torch.cuda.synchronize()
    # the fused path keeps the projected dt in fp32 (no delta tensor is stored)
    e = 2 if io == "bf16" else 4
    fused_path = fused == "on" and N in (8, 16) and (R * e) % 16 == 0 and R * e <= 512
    delta, B, C = oracle.selection(inp.u, sw.W_x, sw.W_dt, N, store=_store(io), store_delta=not fused_path)
    ro, rl = oracle.scan(inp.u, delta, inp.A, B, C, inp.delta_bias, inp.Dskip, inp.z, True)
    eo, el = parity_error(to_host(out), ro), parity_error(to_host(last), rl)
    print(f"{case}: out {eo:.2e} last_state {el:.2e}")
    assert eo <= TOL[io] and el <= TOL[io], (eo, el)
