"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on the GPU.

Small problems are compared element by element in full; the full-size
workloads are run whole on the GPU and compared on sampled (batch row,
channel) pairs, each over the whole sequence, which the oracle computes one
channel at a time (channels are independent SSMs).  Tolerance: max relative
error 1e-4 for fp32 I/O, 2e-2 for bf16 I/O (fp32 state in both cases)."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, gpu_scan, parity_error, to_device, to_host
from selective_state_space_22_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _announce(msg):
    print(f"\n[gpu-test] {msg}", flush=True)


def check(inp, h0=None, softplus=None, label=""):
    """Full element-by-element comparison of out and last_state."""
    go, gl = gpu_scan(inp, h0=h0, softplus=softplus)
    ro, rl = oracle.scan_inputs(inp, h0=h0, softplus=softplus)
    eo, el = parity_error(go, ro), parity_error(gl, rl)
    tol = TOL[inp.io]
    assert np.isfinite(go).all() and np.isfinite(gl).all(), label
    assert eo <= tol and el <= tol, f"{label}: out err {eo:.3e}, last_state err {el:.3e}, tol {tol}"
    return eo, el


def test_tiny_workload_full():
    _need_gpu()
    _announce("tiny workload (1, 256, 64, 16) fp32, full comparison")
    inp = W.generate_workload("tiny")
    eo, el = check(inp, label="tiny")
    print(f"tiny: out err {eo:.3e} last err {el:.3e}")


def test_tiny_workload_scan_only():
    """Without skip and gate, so the skip term cannot mask scan error."""
    _need_gpu()
    inp = W.generate_workload("tiny")
    inp.z = None
    inp.Dskip = None
    eo, el = check(inp, label="tiny scan-only")
    print(f"tiny scan-only: out err {eo:.3e} last err {el:.3e}")


_CACHE = {}


def _workload(name):
    """Seeded inputs of a named workload, generated once per session."""
    if name not in _CACHE:
        _CACHE.clear()  # keep one large workload in host memory at a time
        _CACHE[name] = W.generate_workload(name)
    return _CACHE[name]


def _sampled(name, nchan=24, batches=None, scan_only=False):
    _need_gpu()
    _announce(f"{name}: full GPU run, sampled oracle channels (scan_only={scan_only})")
    w = W.WORKLOADS[name]
    inp = _workload(name)
    if scan_only:
        import dataclasses

        inp = dataclasses.replace(inp, z=None, Dskip=None)
    go, gl = gpu_scan(inp)
    assert np.isfinite(go).all() and np.isfinite(gl).all()
    rng = np.random.default_rng(7)
    chans = np.unique(np.concatenate([[0, 63, 64, w.dim - 1], rng.choice(w.dim, nchan, replace=False)]))
    bs = batches if batches is not None else sorted({0, w.batch - 1})
    sub = W.channel_subset(inp, bs, chans)
    ro, rl = oracle.scan_inputs(sub)
    eo = parity_error(go[np.ix_(bs, np.arange(w.seqlen), chans)], ro)
    el = parity_error(gl[np.ix_(bs, chans)], rl)
    tol = TOL[w.io]
    print(f"{name}: out err {eo:.3e} last err {el:.3e} (tol {tol})")
    assert eo <= tol and el <= tol, f"{name}: out {eo:.3e} last {el:.3e}"


def test_mamba130m_layer_sampled():
    _sampled("mamba130m_layer")


def test_mamba130m_layer_scan_only_sampled():
    _sampled("mamba130m_layer", scan_only=True)


def test_mamba3b_layer_sampled():
    _sampled("mamba3b_layer")


def test_million_tokens_sampled():
    _sampled("million_tokens", nchan=6)


def test_decode_64_steps():
    """64 one-token steps from a zero state == the scan over the same 64 tokens == the oracle."""
    _need_gpu()
    _announce("decode: 64 steps of (256, 5120, 16) bf16")
    from selective_state_space_22_amd import mamba_state_update

    inp = W.generate_workload("decode")
    d = to_device(inp)
    batch, L, D, N = inp.batch, inp.seqlen, inp.dim, inp.dstate
    state = torch.zeros((batch, D, N), dtype=torch.float32, device="cuda")
    steps = {k: [d[k][:, t].contiguous() for t in range(L)] for k in ("u", "delta", "B", "C", "z")}
    outs = []
    for t in range(L):
        o = mamba_state_update(state, steps["u"][t], steps["delta"][t], d["A"], steps["B"][t], steps["C"][t],
                               d["delta_bias"], d["Dskip"], steps["z"][t], True)
        outs.append(o)
    torch.cuda.synchronize()
    dec = np.stack([to_host(o) for o in outs], axis=1)
    st = to_host(state)
    so, sl = gpu_scan(inp, dev_inputs=d)
    # the two GPU entry points agree
    assert parity_error(dec, so) <= TOL["bf16"] and parity_error(st, sl) <= 1e-5
    # and both agree with the oracle on sampled channels
    rng = np.random.default_rng(3)
    chans = np.unique(np.concatenate([[0, D - 1], rng.choice(D, 16, replace=False)]))
    bs = [0, 97, batch - 1]
    sub = W.channel_subset(inp, bs, chans)
    ro, rl = oracle.scan_inputs(sub)
    eo = parity_error(dec[np.ix_(bs, np.arange(L), chans)], ro)
    el = parity_error(st[np.ix_(bs, chans)], rl)
    print(f"decode: out err {eo:.3e} state err {el:.3e}; decode vs scan identical: "
          f"{np.array_equal(dec, so)} / {np.array_equal(st, sl)}")
    assert eo <= TOL["bf16"] and el <= TOL["bf16"]


EDGE = [
    # batch, L, D, N, io, kwargs
    (1, 1, 64, 16, "f32", {}),
    (3, 1, 64, 16, "bf16", {}),
    (2, 1000, 100, 16, "f32", {}),          # ragged channel tail, chunked L with a ragged last chunk
    (1, 2048, 64, 16, "f32", {}),           # chunked, 8 chunks
    (2, 777, 130, 16, "bf16", {}),
    (1, 300, 64, 1, "f32", {}),
    (1, 300, 64, 2, "bf16", {}),
    (2, 300, 96, 4, "f32", {}),
    (1, 600, 64, 8, "bf16", {}),
    (2, 513, 64, 16, "f32", {"a_kind": "exp_normal"}),
    (2, 513, 64, 16, "bf16", {"a_kind": "neg_half"}),
    (1, 256, 64, 16, "f32", {"with_z": False, "with_dskip": False, "with_bias": False}),
    (1, 256, 320, 16, "f32", {"with_z": False}),
    (1, 4096, 32, 16, "f32", {}),           # fewer channels than a wave, many chunks
]


ENGINES = ["default", "lane"]


def _engine(monkeypatch, engine):
    """The library picks its engine from the shape; MAMBA_MI355X_LANE_ENGINE=1 forces the
    lane-per-channel engine so that both engines are covered on the same cases."""
    if engine == "lane":
        monkeypatch.setenv("MAMBA_MI355X_LANE_ENGINE", "1")
    else:
        monkeypatch.delenv("MAMBA_MI355X_LANE_ENGINE", raising=False)


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("case", EDGE, ids=[f"b{c[0]}_L{c[1]}_D{c[2]}_N{c[3]}_{c[4]}_{i}" for i, c in enumerate(EDGE)])
def test_edge_cases(case, engine, monkeypatch):
    _need_gpu()
    _engine(monkeypatch, engine)
    batch, L, D, N, io, kw = case
    _announce(f"edge case {case} engine={engine}")
    inp = W.generate(batch, L, D, N, io, seed=500 + L + D + N, **kw)
    check(inp, label=f"{case} {engine}")


# Shapes that reach every mode of the workgroup engine (N = 16 and 8):
#   chained, one chunk per channel block (<= 256 channel blocks);
#   chained, several chunks per block handed between workgroups (> 256 blocks);
#   split into two passes (few blocks, long sequence).
WG_CASES = [
    (3, 700, 4096, 16, "bf16"),    # 192 blocks, chained, one chunk
    (5, 1100, 4096, 16, "bf16"),   # 320 blocks, chained, 3 chunks (last one ragged)
    (3, 1500, 6000, 16, "f32"),    # 282 blocks with a ragged channel tail, 3 chunks
    (1, 4096, 64, 16, "f32"),      # 1 block, split into 64 chunks
    (2, 3000, 200, 16, "bf16"),    # 8 blocks with a ragged tail, split
    (3, 900, 4096, 8, "f32"),      # N = 8: 4 waves per workgroup
    (1, 5000, 128, 8, "bf16"),     # N = 8, split
]


@pytest.mark.parametrize("case", WG_CASES, ids=[f"b{c[0]}_L{c[1]}_D{c[2]}_N{c[3]}_{c[4]}" for c in WG_CASES])
def test_workgroup_engine_modes(case, monkeypatch):
    _need_gpu()
    _engine(monkeypatch, "default")
    batch, L, D, N, io = case
    _announce(f"workgroup engine case {case}")
    inp = W.generate(batch, L, D, N, io, seed=900 + L + D + N)
    eo, el = check(inp, label=str(case))
    print(f"{case}: out err {eo:.3e} last err {el:.3e}")


@pytest.mark.parametrize("case", [(5, 1100, 4096, 16, "f32"), (1, 4096, 64, 16, "f32")], ids=["chained", "split"])
def test_workgroup_engine_initial_state(case, monkeypatch):
    _need_gpu()
    _engine(monkeypatch, "default")
    batch, L, D, N, io = case
    inp = W.generate(batch, L, D, N, io, seed=77)
    h0 = np.random.default_rng(78).standard_normal((batch, D, N)).astype(np.float32)
    check(inp, h0=h0, label=f"h0 {case}")


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("chunked", [False, True])
def test_initial_state(chunked, engine, monkeypatch):
    _need_gpu()
    _engine(monkeypatch, engine)
    L = 4096 if chunked else 200
    inp = W.generate(2, L, 64, 16, "f32", seed=71)
    h0 = np.random.default_rng(72).standard_normal((2, 64, 16)).astype(np.float32)
    check(inp, h0=h0, label=f"h0 chunked={chunked}")


def test_no_softplus_positive_dt():
    _need_gpu()
    inp = W.generate(2, 300, 64, 16, "f32", seed=73, with_bias=False)
    inp.delta = np.abs(inp.delta) * 0.002  # dt = delta itself: positive, no softplus
    check(inp, softplus=False, label="no softplus")


def test_empty_sequence_returns_initial_state():
    _need_gpu()
    from selective_state_space_22_amd import mamba_scan_fwd

    u = torch.zeros((2, 0, 64), device="cuda")
    A = -torch.ones((64, 16), device="cuda")
    B = torch.zeros((2, 0, 16), device="cuda")
    h0 = torch.randn((2, 64, 16), device="cuda")
    out, last = mamba_scan_fwd(u, u, A, B, B, h0=h0)
    torch.cuda.synchronize()
    assert out.shape == (2, 0, 64) and torch.equal(last, h0)
    out, last = mamba_scan_fwd(u, u, A, B, B)
    torch.cuda.synchronize()
    assert torch.count_nonzero(last) == 0


# ------------------------------------------------------------ invariants


def _run(inp, **kw):
    return gpu_scan(inp, **kw)


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("L", [300, 3000])
def test_causality_bit_exact(L, engine, monkeypatch):
    _need_gpu()
    _engine(monkeypatch, engine)
    inp = W.generate(2, L, 128, 16, "f32", seed=80)
    o1, _ = _run(inp)
    t0 = L // 2 + 3
    for name in ("u", "delta", "z", "B", "C"):
        arr = getattr(inp, name)
        saved = arr.copy()
        arr[:, t0] += 0.5
        o2, _ = _run(inp)
        setattr(inp, name, saved)
        assert np.array_equal(o1[:, :t0], o2[:, :t0]), name
        assert not np.array_equal(o1[:, t0:], o2[:, t0:]), name


@pytest.mark.parametrize("engine", ENGINES)
def test_hold_is_exact(engine, monkeypatch):
    """dt = 0 (no softplus, raw = -bias) keeps the state bit-exactly."""
    _need_gpu()
    _engine(monkeypatch, engine)
    inp = W.generate(2, 400, 64, 16, "f32", seed=81)
    inp.delta = np.broadcast_to(-inp.delta_bias, inp.u.shape).astype(np.float32).copy()
    h0 = np.random.default_rng(82).standard_normal((2, 64, 16)).astype(np.float32)
    o, last = _run(inp, h0=h0, softplus=False)
    assert np.array_equal(last, h0)
    ro, _ = oracle.scan_inputs(inp, h0=h0, softplus=False)
    assert parity_error(o, ro) <= TOL["f32"]


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("L", [200, 3000])
def test_reset_forgets_the_prefix_exactly(L, engine, monkeypatch):
    _need_gpu()
    _engine(monkeypatch, engine)
    inp = W.generate(1, L, 64, 16, "f32", seed=83)
    tr = L // 2 + 11
    inp.delta[:, tr] = 60.0  # dt*A <= -60 * log2(e): Abar underflows to exactly 0
    o1, l1 = _run(inp)
    rng = np.random.default_rng(84)
    for name in ("u", "z", "B", "C"):
        getattr(inp, name)[:, :tr] = rng.standard_normal(getattr(inp, name)[:, :tr].shape)
    inp.delta[:, :tr] = rng.uniform(-4, -2, inp.delta[:, :tr].shape)
    o2, l2 = _run(inp)
    assert np.array_equal(o1[:, tr:], o2[:, tr:]) and np.array_equal(l1, l2)


@pytest.mark.parametrize("shape", [(2, 3000, 256), (5, 1100, 4096)], ids=["split", "chained"])
def test_run_to_run_determinism(shape):
    """Also a race smoke test: the chained mode hands states between workgroups."""
    _need_gpu()
    inp = W.generate(*shape, 16, "bf16", seed=85)
    d = to_device(inp)
    a = gpu_scan(inp, dev_inputs=d)
    b = gpu_scan(inp, dev_inputs=d)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_linearity():
    _need_gpu()
    inp = W.generate(1, 500, 64, 16, "f32", seed=86, with_z=False)
    o1, h1 = _run(inp)
    u1 = inp.u.copy()
    u2 = np.random.default_rng(87).standard_normal(u1.shape).astype(np.float32)
    inp.u = u2
    o2, h2 = _run(inp)
    inp.u = (0.5 * u1 - 1.25 * u2).astype(np.float32)
    o3, h3 = _run(inp)
    assert parity_error(o3, 0.5 * o1.astype(np.float64) - 1.25 * o2) <= 1e-4
    assert parity_error(h3, 0.5 * h1.astype(np.float64) - 1.25 * h2) <= 1e-4


@pytest.mark.parametrize("case", [(3, 12, 70, 1, "f32"), (2, 9, 64, 2, "bf16"), (4, 10, 100, 4, "f32"),
                                  (2, 8, 130, 8, "bf16"), (1, 5, 33, 16, "f32")], ids=str)
def test_decode_small_dstate(case):
    """Decode steps for every supported N against the oracle's step (and the GPU scan)."""
    _need_gpu()
    from selective_state_space_22_amd import mamba_state_update

    batch, L, D, N, io = case
    _announce(f"decode {case}")
    inp = W.generate(batch, L, D, N, io, seed=900 + N)
    d = to_device(inp)
    h0 = np.random.default_rng(N).standard_normal((batch, D, N)).astype(np.float32)
    state = torch.from_numpy(h0.copy()).cuda()
    st_ref = h0.astype(np.float64)
    outs = []
    for t in range(L):
        # fresh copies: a slice of a batch-1 tensor is already contiguous and keeps its (unaligned) offset
        o = mamba_state_update(state, d["u"][:, t].clone(), d["delta"][:, t].clone(), d["A"],
                               d["B"][:, t].clone(), d["C"][:, t].clone(), d["delta_bias"], d["Dskip"],
                               d["z"][:, t].clone(), True)
        outs.append(to_host(o))
        ro, st_ref = oracle.step(st_ref, inp.u[:, t], inp.delta[:, t], inp.A, inp.B[:, t], inp.C[:, t],
                                 inp.delta_bias, inp.Dskip, inp.z[:, t], True)
        assert parity_error(outs[-1], ro) <= TOL[io], f"step {t}"
    torch.cuda.synchronize()
    assert parity_error(to_host(state), st_ref) <= TOL[io]
    so, sl = gpu_scan(inp, h0=h0)
    assert parity_error(np.stack(outs, 1), so) <= TOL[io] and parity_error(to_host(state), sl) <= 1e-5
