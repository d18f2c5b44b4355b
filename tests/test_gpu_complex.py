"""Parity of the complex-A forward scan (mamba_scan_fwd_complex, through the C
ABI) with the fp64 oracle's complex scan, on the GPU.

A_n = -1/2 + n i (the complex row of the page's A-initialisation ablation),
real dt, x, B, C; out = Re(C . h) with the skip and the gate; the state is
complex.  Small problems are compared element by element; the Mamba-3B layer
shape on sampled (batch row, channel) pairs over the whole sequence.
Tolerance as for the real scan: 1e-4 (fp32 I/O), 2e-2 (bf16 I/O)."""
import dataclasses

import numpy as np
import pytest

import oracle
from gpu_util import TOL, force_engine, gpu_scan, parity_error, to_device, to_host
from selective_state_space_22_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _announce(msg):
    print(f"\n[gpu-test] {msg}", flush=True)


def _cinputs(batch, L, D, N, io, seed, A=None):
    inp = W.generate(batch, L, D, N, io, seed=seed)
    Ac = W.a_init_complex(D, N) if A is None else A
    return inp, Ac


def _h0(batch, D, N, seed):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((batch, D, N)) + 1j * rng.standard_normal((batch, D, N))
    return (0.5 * h).astype(np.complex64)


def gpu_cscan(inp, Ac, h0=None, softplus=None, dev_inputs=None):
    from selective_state_space_22_amd import mamba_scan_fwd_complex

    d = dev_inputs or to_device(inp, "cuda")
    At = torch.from_numpy(np.ascontiguousarray(Ac, np.complex64)).to("cuda")
    h0t = None if h0 is None else torch.from_numpy(np.ascontiguousarray(h0, np.complex64)).to("cuda")
    out, last = mamba_scan_fwd_complex(d["u"], d["delta"], At, d["B"], d["C"], d["delta_bias"], d["Dskip"], d["z"],
                                       inp.softplus if softplus is None else softplus, h0t)
    torch.cuda.synchronize()
    return to_host(out), last.cpu().numpy()


def ref_cscan(inp, Ac, h0=None, softplus=None):
    return oracle.scan_complex(inp.u, inp.delta, Ac.astype(np.complex128), inp.B, inp.C, inp.delta_bias, inp.Dskip,
                               inp.z, inp.softplus if softplus is None else softplus,
                               None if h0 is None else h0.astype(np.complex128))


def cerr(g, r):
    """Parity error of a complex tensor: over its real and imaginary parts together."""
    return parity_error(np.stack([g.real, g.imag], -1), np.stack([r.real, r.imag], -1))


def check(inp, Ac, h0=None, softplus=None, label=""):
    go, gl = gpu_cscan(inp, Ac, h0, softplus)
    ro, rl = ref_cscan(inp, Ac, h0, softplus)
    assert np.isfinite(go).all() and np.isfinite(gl).all(), label
    eo, el = parity_error(go, ro), cerr(gl, rl)
    tol = TOL[inp.io]
    assert eo <= tol and el <= tol, f"{label}: out err {eo:.3e}, last_state err {el:.3e}, tol {tol}"
    return eo, el


def _engine(request, engine):
    """N = 8 and 16 run on the workgroup engine by default; the engine option set to
    "lane" forces the lane-per-channel kernels so that both are covered."""
    force_engine(request, "lane" if engine == "lane" else "default")


@pytest.mark.parametrize("engine", ["default", "lane"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 2, 4, 8, 16])
def test_small_full(io, N, engine, request):
    _need_gpu()
    _engine(request, engine)
    _announce(f"complex A: (2, 300, 130, {N}) {io}, with h0, engine={engine}")
    inp, Ac = _cinputs(2, 300, 130, N, io, seed=W.SEED_BASE + 41 + N)
    eo, el = check(inp, Ac, h0=_h0(2, 130, N, 5), label=f"N={N} {io} {engine}")
    print(f"N={N} {io} {engine}: out err {eo:.3e} last err {el:.3e}")


# Shapes that reach every mode of the workgroup engine with complex states:
# chained with one chunk per channel block, chained with chunks handed between
# workgroups (> 256 blocks), and the two-pass split (few blocks, long rows).
WG_CASES = [
    (3, 700, 4096, 16, "bf16"),    # 192 blocks, chained, one chunk
    (5, 1100, 4096, 16, "bf16"),   # 320 blocks, chained, 3 chunks (last one ragged)
    (1, 4096, 64, 16, "f32"),      # 1 block, split into 64 chunks
    (2, 3000, 200, 16, "bf16"),    # 8 blocks with a ragged channel tail, split
    (3, 900, 4096, 8, "f32"),      # N = 8, chained
    (1, 5000, 128, 8, "bf16"),     # N = 8, split
]


@pytest.mark.parametrize("case", WG_CASES, ids=[f"b{c[0]}_L{c[1]}_D{c[2]}_N{c[3]}_{c[4]}" for c in WG_CASES])
def test_workgroup_engine_modes(case, request):
    _need_gpu()
    _engine(request, "default")
    batch, L, D, N, io = case
    _announce(f"complex A, workgroup engine case {case}, with h0")
    inp, Ac = _cinputs(batch, L, D, N, io, seed=W.SEED_BASE + 66 + L + N)
    eo, el = check(inp, Ac, h0=_h0(batch, D, N, 9), label=str(case))
    print(f"{case}: out err {eo:.3e} last err {el:.3e}")


def test_scan_only_no_softplus():
    """Without skip, gate and softplus, so nothing masks the scan's error."""
    _need_gpu()
    inp, Ac = _cinputs(1, 200, 64, 16, "f32", seed=W.SEED_BASE + 61)
    inp = dataclasses.replace(inp, z=None, Dskip=None, delta_bias=None, delta=np.abs(inp.delta) * 0.1 + 1e-3)
    check(inp, Ac, softplus=False, label="scan only")


@pytest.mark.parametrize("engine", ["default", "lane"])
def test_long_sequence_is_chunked(engine, request):
    """One row of 8192 tokens over 128 channels: the plan cuts it into chunks whose
    end states are composed through complex carries."""
    _need_gpu()
    _engine(request, engine)
    _announce("complex A: (1, 8192, 128, 16) f32, chunked, with h0")
    inp, Ac = _cinputs(1, 8192, 128, 16, "f32", seed=W.SEED_BASE + 62)
    eo, el = check(inp, Ac, h0=_h0(1, 128, 16, 6), label="long")
    print(f"long: out err {eo:.3e} last err {el:.3e}")


def test_random_complex_a_with_zero_and_large_rotation():
    """Per-channel random A (decay rates spread over two decades, rotations up to
    20 rad per unit dt), one A_n = 0 (input weight dt) and one purely imaginary."""
    _need_gpu()
    rng = np.random.default_rng(3)
    D, N = 96, 8
    Ac = (-np.exp(rng.uniform(-2.5, 1.5, (D, N))) + 1j * rng.uniform(-20, 20, (D, N))).astype(np.complex64)
    Ac[5, 3] = 0
    Ac[7, 2] = 4j
    inp, _ = _cinputs(2, 700, D, N, "f32", seed=W.SEED_BASE + 63)
    check(inp, Ac, h0=_h0(2, D, N, 7), label="random A")


def test_zero_imaginary_part_matches_the_real_scan():
    """With Im A = 0 the complex path computes the real scan: same outputs as
    mamba_scan_fwd on the real parts, and a real final state."""
    _need_gpu()
    inp, _ = _cinputs(2, 513, 64, 16, "f32", seed=W.SEED_BASE + 64)
    Ac = inp.A.astype(np.complex64)
    go, gl = gpu_cscan(inp, Ac)
    ro, rl = gpu_scan(inp)
    assert parity_error(go, ro) <= 5e-5
    assert parity_error(gl.real, rl) <= 5e-5
    assert np.all(gl.imag == 0)


def test_empty_sequence_returns_h0():
    _need_gpu()
    inp, Ac = _cinputs(2, 0, 64, 4, "f32", seed=W.SEED_BASE + 65)
    h0 = _h0(2, 64, 4, 8)
    go, gl = gpu_cscan(inp, Ac, h0)
    assert go.shape == (2, 0, 64)
    np.testing.assert_array_equal(gl, h0)


def test_mamba3b_layer_sampled():
    """Full (4, 4096, 5120, 16) bf16 layer on the GPU, sampled channels against the oracle."""
    _need_gpu()
    _announce("complex A: mamba3b_layer shape bf16, sampled channels")
    w = W.WORKLOADS["mamba3b_layer"]
    inp = W.generate_workload("mamba3b_layer")
    Ac = W.a_init_complex(w.dim, w.dstate)
    go, gl = gpu_cscan(inp, Ac)
    assert np.isfinite(go).all() and np.isfinite(gl).all()
    rng = np.random.default_rng(11)
    chans = np.unique(np.concatenate([[0, 63, 64, w.dim - 1], rng.choice(w.dim, 20, replace=False)]))
    bs = np.arange(w.batch)
    sub = W.channel_subset(inp, bs, chans)
    ro, rl = ref_cscan(sub, Ac[chans])
    eo = parity_error(go[bs][:, :, chans], ro)
    el = cerr(gl[bs][:, chans], rl)
    print(f"mamba3b complex sampled: out err {eo:.3e} last err {el:.3e}")
    assert eo <= TOL["bf16"] and el <= TOL["bf16"]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 2, 4, 8, 16])
def test_decode_matches_oracle(io, N):
    """L one-token steps of mamba_state_update_complex from a complex h0 equal the
    oracle's complex scan over the same L tokens: every step's output and the final state."""
    _need_gpu()
    from selective_state_space_22_amd import mamba_state_update_complex

    _announce(f"complex decode (3, 24 steps, 130, {N}) {io}")
    L, D, batch = 24, 130, 3
    inp, Ac = _cinputs(batch, L, D, N, io, seed=W.SEED_BASE + 81 + N)
    h0 = _h0(batch, D, N, 10)
    d = to_device(inp, "cuda")
    At = torch.from_numpy(np.ascontiguousarray(Ac)).to("cuda")
    state = torch.from_numpy(np.ascontiguousarray(h0)).to("cuda")
    outs = []
    for t in range(L):
        sl = lambda x: None if x is None else x[:, t].contiguous()
        outs.append(mamba_state_update_complex(state, sl(d["u"]), sl(d["delta"]), At, sl(d["B"]), sl(d["C"]),
                                               d["delta_bias"], d["Dskip"], sl(d["z"]), True))
    torch.cuda.synchronize()
    go = to_host(torch.stack(outs, 1))
    gl = state.cpu().numpy()
    ro, rl = ref_cscan(inp, Ac, h0)
    eo, el = parity_error(go, ro), cerr(gl, rl)
    print(f"complex decode N={N} {io}: out err {eo:.3e} state err {el:.3e}")
    assert eo <= TOL[io] and el <= TOL[io]


def test_decode_continues_the_scan():
    """A scan over the first 40 tokens, then 8 decode steps from its last state,
    equals the scan over all 48 tokens (outputs of the last 8, final state)."""
    _need_gpu()
    from selective_state_space_22_amd import mamba_state_update_complex

    inp, Ac = _cinputs(2, 48, 96, 16, "f32", seed=W.SEED_BASE + 99)
    d = to_device(inp, "cuda")
    go_all, gl_all = gpu_cscan(inp, Ac)
    head = dataclasses.replace(inp, seqlen=40, **{k: np.ascontiguousarray(getattr(inp, k)[:, :40])
                                                  for k in ("u", "delta", "z", "B", "C")})
    _, gl_head = gpu_cscan(head, Ac)
    At = torch.from_numpy(np.ascontiguousarray(Ac)).to("cuda")
    state = torch.from_numpy(np.ascontiguousarray(gl_head)).to("cuda")
    outs = []
    for t in range(40, 48):
        sl = lambda x: x[:, t].contiguous()
        outs.append(mamba_state_update_complex(state, sl(d["u"]), sl(d["delta"]), At, sl(d["B"]), sl(d["C"]),
                                               d["delta_bias"], d["Dskip"], sl(d["z"]), True))
    torch.cuda.synchronize()
    assert parity_error(to_host(torch.stack(outs, 1)), go_all[:, 40:]) <= 1e-5
    assert cerr(state.cpu().numpy(), gl_all) <= 1e-5


@pytest.mark.parametrize("engine", ["default", "lane"])
def test_angles_in_every_sin_cos_range(engine, request):
    """Per-token angles dt Im A_n from below 1/4 rad to ~40 rad, so that waves take the
    short series, the pi/4 series and the reduced evaluation of sin and cos."""
    _need_gpu()
    _engine(request, engine)
    rng = np.random.default_rng(12)
    D, N = 128, 16
    Ac = (-rng.uniform(0.2, 3.0, (D, N)) + 1j * rng.uniform(-200.0, 200.0, (D, N))).astype(np.complex64)
    Ac[:64] = (Ac[:64].real + 1j * rng.uniform(-1.0, 1.0, (64, N))).astype(np.complex64)  # one wave of small angles
    inp, _ = _cinputs(2, 400, D, N, "f32", seed=W.SEED_BASE + 100)
    inp = dataclasses.replace(inp, delta_bias=None, delta=(np.abs(inp.delta) * 0.05).astype(np.float32))
    eo, el = check(inp, Ac, h0=_h0(2, D, N, 13), softplus=False, label=f"angles {engine}")
    print(f"angle ranges {engine}: out err {eo:.3e} last err {el:.3e}")
