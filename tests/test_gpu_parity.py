"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on the GPU.

Every comparison is element by element over whole tensors: the full-size
workloads are run whole on the GPU and the oracle covers them in groups of
channels (channels are independent SSMs), so its host memory stays bounded.
Tolerance: max relative
error 1e-4 for fp32 I/O, 2e-2 for bf16 I/O (fp32 state in both cases)."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, force_engine, gpu_scan, library_option, parity_error, to_device, to_host
from selective_state_space_22_amd import binding, workloads as W

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


def _full(name, group, scan_only=False):
    """Run a full-size workload whole on the GPU and compare every output element and
    every end state with the oracle, which runs over groups of `group` channels
    (channels are independent SSMs) to bound its host memory."""
    _need_gpu()
    _announce(f"{name}: full GPU run, whole-tensor oracle comparison in groups of {group} channels "
              f"(scan_only={scan_only})")
    w = W.WORKLOADS[name]
    inp = _workload(name)
    if scan_only:
        import dataclasses

        inp = dataclasses.replace(inp, z=None, Dskip=None)
    go, gl = gpu_scan(inp)
    assert np.isfinite(go).all() and np.isfinite(gl).all()
    ro = np.empty(go.shape, np.float64)
    rl = np.empty(gl.shape, np.float64)
    rows = np.arange(w.batch)
    for d0 in range(0, w.dim, group):
        d1 = min(d0 + group, w.dim)
        ro[:, :, d0:d1], rl[:, d0:d1] = oracle.scan_inputs(W.channel_subset(inp, rows, np.arange(d0, d1)))
    eo, el = parity_error(go, ro), parity_error(gl, rl)
    tol = TOL[w.io]
    print(f"{name}: out err {eo:.3e} last err {el:.3e} over every element (tol {tol})")
    assert eo <= tol and el <= tol, f"{name}: out {eo:.3e} last {el:.3e}"


def test_mamba130m_layer_full():
    _full("mamba130m_layer", group=512)


def test_mamba130m_layer_scan_only_full():
    _full("mamba130m_layer", group=512, scan_only=True)


def test_mamba3b_layer_full():
    _full("mamba3b_layer", group=512)


def test_million_tokens_full():
    _full("million_tokens", group=32)


def test_decode_64_steps():
    """64 one-token steps from a zero state == the scan over the same 64 tokens == the
    oracle, on every output of every step and every end state."""
    _need_gpu()
    _announce("decode: 64 steps of (256, 5120, 16) bf16, whole-tensor comparison")
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
    # and both agree with the oracle everywhere
    ro, rl = oracle.scan_inputs(inp)
    eo, el = parity_error(dec, ro), parity_error(st, rl)
    eso = parity_error(so, ro)
    print(f"decode: out err {eo:.3e} state err {el:.3e} scan out err {eso:.3e}; decode vs scan identical: "
          f"{np.array_equal(dec, so)} / {np.array_equal(st, sl)}")
    assert eo <= TOL["bf16"] and el <= TOL["bf16"] and eso <= TOL["bf16"]


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
    # mixed launches of the default engine (one state per lane for the last blocks)
    (1, 1, 12288, 16, "f32", {}),           # a single token, 192 blocks
    (2, 17, 10240, 16, "bf16", {}),         # one whole tile and one token, 320 blocks
    (1, 100, 12288, 16, "f32", {"a_kind": "exp_normal"}),
]


ENGINES = ["default", "wg", "lane"]


def _engine(request, engine):
    """The library picks its engine from the shape; the engine option forces the
    lane-per-channel engine ("lane"), the workgroup engine whose waves split the states
    ("wg") or leaves the choice to the library ("default", the wave-private engine for
    N = 8 and 16), so that every engine is covered on the same cases."""
    force_engine(request, engine)


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("case", EDGE, ids=[f"b{c[0]}_L{c[1]}_D{c[2]}_N{c[3]}_{c[4]}_{i}" for i, c in enumerate(EDGE)])
def test_edge_cases(case, engine, request):
    _need_gpu()
    _engine(request, engine)
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


@pytest.mark.parametrize("engine", ["default", "wg"])
@pytest.mark.parametrize("case", WG_CASES, ids=[f"b{c[0]}_L{c[1]}_D{c[2]}_N{c[3]}_{c[4]}" for c in WG_CASES])
def test_workgroup_engine_modes(case, engine, request):
    _need_gpu()
    _engine(request, engine)
    batch, L, D, N, io = case
    _announce(f"workgroup engine case {case} engine={engine}")
    inp = W.generate(batch, L, D, N, io, seed=900 + L + D + N)
    eo, el = check(inp, label=str(case))
    print(f"{case}: out err {eo:.3e} last err {el:.3e}")


@pytest.mark.parametrize("engine", ["default", "wg"])
@pytest.mark.parametrize("case", [(5, 1100, 4096, 16, "f32"), (1, 4096, 64, 16, "f32")], ids=["chained", "split"])
def test_workgroup_engine_initial_state(case, engine, request):
    _need_gpu()
    _engine(request, engine)
    batch, L, D, N, io = case
    inp = W.generate(batch, L, D, N, io, seed=77)
    h0 = np.random.default_rng(78).standard_normal((batch, D, N)).astype(np.float32)
    check(inp, h0=h0, label=f"h0 {case}")


def test_chained_wait_timeout_is_reported(request):
    """A chained chunk whose wait for its predecessor's end state gives up must say so:
    with the wait bound set to 0 every chunk after the first gives up at once, the
    stream status reports MAMBA_ERR_TIMEOUT (and the binding raises), those chunks'
    outputs and the end states are NaN, and the first chunk's outputs still match the
    oracle.  The status is cleared by the query, and the next call with the default
    bound is clean and correct."""
    _need_gpu()
    from gpu_util import library_option
    from selective_state_space_22_amd import binding, mamba_scan_fwd

    force_engine(request, "wg")
    batch, L, D, N, io = 5, 1100, 4096, 16, "f32"   # 320 channel blocks: chained, chunks of 256
    _announce(f"chained wait with bound 0 on {(batch, L, D, N, io)}")
    inp = W.generate(batch, L, D, N, io, seed=31)
    d = to_device(inp)
    assert binding.mamba_stream_status() == 0
    with library_option(binding.MAMBA_OPT_CHUNK, 256), library_option(binding.MAMBA_OPT_SPIN_LIMIT, 0):
        with pytest.raises(binding.MambaError) as ex:
            mamba_scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["delta_bias"], d["Dskip"], d["z"], True,
                           check=True)
        assert ex.value.status == binding.MAMBA_ERR_TIMEOUT
        assert binding.mamba_stream_status() == 0  # reported once
        out, last = mamba_scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["delta_bias"], d["Dskip"], d["z"],
                                   True)
        assert binding.mamba_stream_status() == binding.MAMBA_ERR_TIMEOUT
        go, gl = to_host(out), to_host(last)
    ro, _ = oracle.scan_inputs(inp)
    assert np.isnan(go[:, 256:]).all() and np.isnan(gl).all()
    assert parity_error(go[:, :256], ro[:, :256]) <= TOL[io]
    # the default bound: every wait ends, the status stays clear
    with library_option(binding.MAMBA_OPT_CHUNK, 256):
        check(inp, label="chained after a timeout")
    assert binding.mamba_stream_status() == 0


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("chunked", [False, True])
def test_initial_state(chunked, engine, request):
    _need_gpu()
    _engine(request, engine)
    L = 4096 if chunked else 200
    inp = W.generate(2, L, 64, 16, "f32", seed=71)
    h0 = np.random.default_rng(72).standard_normal((2, 64, 16)).astype(np.float32)
    check(inp, h0=h0, label=f"h0 chunked={chunked}")


def test_no_softplus_positive_dt():
    _need_gpu()
    inp = W.generate(2, 300, 64, 16, "f32", seed=73, with_bias=False)
    inp.delta = np.abs(inp.delta) * 0.002  # dt = delta itself: positive, no softplus
    check(inp, softplus=False, label="no softplus")


def _input_weight_stress(L, D, N, seed):
    """Inputs that sweep dt * A_n over the whole range the input weight must cover:
    per channel a bias putting softplus(delta + bias) anywhere in [1e-7, 3], and per
    state an A_n among 0, tiny and large magnitudes of either sign (A_n = 0, tiny or
    positive only where dt is small, so that every state stays O(1)).  States that do
    not decay, driven with a large dt, grow to hundreds over 300 tokens; outputs of a
    few units are then sums of such terms that cancel, and the relative metric
    measures fp32 cancellation in the readout (7.8e-5 with the guarded input weight,
    1.1e-4 with the bracket form, with dt up to 30 on the mixed-launch shape below),
    not the input weight."""
    inp = W.generate(2, L, D, N, "f32", seed=seed)
    g = np.random.default_rng(seed)
    dt_target = np.exp(g.uniform(np.log(1e-7), np.log(3.0), D))
    inp.delta_bias = (np.log(np.expm1(dt_target)) + 3.0).astype(np.float32)  # delta ~ U(-4, -2)
    A = -np.exp(g.uniform(np.log(0.1), np.log(1e3), (D, N)))
    slow = dt_target < 0.1  # states that do not decay only where dt is small, so they stay O(1)
    A[slow, 0] = 0.0
    A[slow, 1] = -1e-6
    A[dt_target < 1e-3, 2] = 0.5   # positive A_n where dt A_n stays below 5e-4 (growth e^0.15 over 300 tokens)
    A[dt_target < 1e-4, 3] = 20.0  # and below 2e-3
    inp.A = A.astype(np.float32)
    return inp


IW_CASES = [((300, 128, 16), e) for e in ("default", "wg", "lane", "wp")] + [
    ((300, 128, 8), "default"), ((300, 128, 8), "wp"), ((200, 96, 4), "default"),
    ((300, 8704, 16), "default"),  # 272 channel blocks: the mixed launch (two- and one-state waves)
]


@pytest.mark.parametrize("shape,engine", IW_CASES, ids=[f"L{c[0][0]}_D{c[0][1]}_N{c[0][2]}_{c[1]}" for c in IW_CASES])
def test_input_weight_over_the_whole_range(shape, engine, request):
    """dt * A_n from 0 and 1e-13 up to 3e3 in magnitude, A_n = 0, A_n > 0: the bracket form of the
    input weight (softplus on) against the oracle at the fp32 bound, on every engine
    and layout that computes it."""
    _need_gpu()
    _engine(request, engine)
    L, D, N = shape
    _announce(f"input weight over the whole range {shape} engine={engine}")
    inp = _input_weight_stress(L, D, N, seed=4242 + N)
    check(inp, label=f"input weight {shape} {engine}")


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


# Mixed launches (N = 16, unchunked, 128-256 or 256-384 (batch row, 64-channel
# block) units): the last units run with one state per lane in the same launch.
MIXED_CASES = [
    (1, 300, 20480, 16, "bf16"),   # 320 units: 256 two-state + 64 one-state, ragged L
    (3, 777, 4100, 16, "bf16"),    # 195 units, ragged channel tail in the one-state part
    (2, 500, 6000, 16, "f32"),     # 188 units, fp32
]


@pytest.mark.parametrize("variant", ["plain", "h0", "no_gate_skip", "no_softplus"])
@pytest.mark.parametrize("case", MIXED_CASES, ids=[f"b{c[0]}_L{c[1]}_D{c[2]}_{c[4]}" for c in MIXED_CASES])
def test_mixed_launch(case, variant):
    _need_gpu()
    batch, L, D, N, io = case
    _announce(f"mixed launch {case} {variant}")
    inp = W.generate(batch, L, D, N, io, seed=700 + L + D)
    h0 = None
    softplus = None
    if variant == "h0":
        h0 = np.random.default_rng(701).standard_normal((batch, D, N)).astype(np.float32)
    elif variant == "no_gate_skip":
        inp.z = None
        inp.Dskip = None
    elif variant == "no_softplus":
        softplus = False
        inp.delta_bias = np.zeros(D, np.float32)
        inp.delta = np.abs(inp.delta) * 0.01  # dt = delta itself: positive without softplus
        if io == "bf16":
            inp.delta = W.bf16_round(inp.delta)[1].reshape(inp.delta.shape)
    eo, el = check(inp, h0=h0, softplus=softplus, label=f"mixed {case} {variant}")
    print(f"{case} {variant}: out err {eo:.3e} last err {el:.3e}")


# Two-pass scans with reset tokens: each chunk's end-state pass may start where the
# rest of the chunk decays the state before it below 2^-200 (MAMBA_OPT_AGG_SKIP).
SKIP_CASES = [
    (1, 65536, 64, 16, "f32"),
    (2, 20000, 200, 16, "bf16"),
    (1, 30000, 128, 8, "f32"),
]


@pytest.mark.parametrize("engine", ["default", "wg", "wp"])
@pytest.mark.parametrize("case", SKIP_CASES, ids=[f"b{c[0]}_L{c[1]}_D{c[2]}_N{c[3]}_{c[4]}" for c in SKIP_CASES])
def test_split_scan_with_reset_tokens(case, engine, request):
    """Against the oracle with the skip on and off, and the two runs against each other."""
    _need_gpu()
    _engine(request, engine)
    batch, L, D, N, io = case
    _announce(f"split scan with reset tokens {case} engine={engine}")
    inp = W.generate(batch, L, D, N, io, seed=610 + L + D, reset_frac=0.01)
    ro, rl = oracle.scan_inputs(inp)
    runs = {}
    for skip in (1, 0):
        with library_option(binding.MAMBA_OPT_AGG_SKIP, skip):
            go, gl = gpu_scan(inp)
        eo, el = parity_error(go, ro), parity_error(gl, rl)
        print(f"{case} skip={skip}: out err {eo:.3e} last err {el:.3e}")
        assert eo <= TOL[io] and el <= TOL[io], f"skip={skip}: out {eo:.3e} last {el:.3e}"
        runs[skip] = (go, gl)
    # the skipped terms are below 2^-200 of the state: the runs differ by rounding only
    agree = 1e-5 if io == "f32" else 2e-2
    assert parity_error(runs[1][0], runs[0][0]) <= agree and parity_error(runs[1][1], runs[0][1]) <= agree


@pytest.mark.parametrize("engine", ["default", "wg", "wp"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_aggregate_skip_keeps_what_reaches_the_chunk_end(io, engine, request):
    """dt is set token by token (bias 0): a period of five 16-token tiles holds a mild
    reset (dt = softplus(2) at the start of tile 1) and a strong one (three tokens of
    dt = softplus(50) at the start of tile 3).  A_0 = -1 decays slowly and the other
    states fast (A_n = -100), so a start taken from the fastest decay would drop the
    state 0 that survives the mild reset (2^-3 of it), a start one tile late would drop
    the tokens after the strong reset, and a start from the wrong chunk or block would
    drop whole chunks: each shows up against the oracle."""
    _need_gpu()
    _engine(request, engine)
    batch, L, D, N = 2, 8000, 96, 16
    _announce(f"aggregate start bound case {(batch, L, D, N, io)} engine={engine}")
    inp = W.generate(batch, L, D, N, io, seed=640)
    inp.delta_bias = np.zeros(D, np.float32)
    A = np.full((D, N), -100.0, np.float32)
    A[:, 0] = -1.0
    inp.A = A
    raw = np.full((batch, L), -5.0, np.float32)
    for p0 in range(0, L, 80):
        raw[:, p0 + 16:p0 + 17] = 2.0
        raw[:, p0 + 48:p0 + 51] = 50.0
    raw[1] = np.roll(raw[1], 37)  # the second row's resets fall elsewhere in the chunks
    inp.delta = np.repeat(raw[:, :, None], D, axis=2).astype(np.float32)
    inp.z = None  # the scan alone: skip and gate would dilute the states' share of the output
    inp.Dskip = None
    with library_option(binding.MAMBA_OPT_AGG_SKIP, 1):
        check(inp, label=f"aggregate start {io} {engine}")


# ------------------------------------------------------------ invariants


def _run(inp, **kw):
    return gpu_scan(inp, **kw)


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("L", [300, 3000])
def test_causality_bit_exact(L, engine, request):
    _need_gpu()
    _engine(request, engine)
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
def test_hold_is_exact(engine, request):
    """dt = 0 (no softplus, raw = -bias) keeps the state bit-exactly."""
    _need_gpu()
    _engine(request, engine)
    inp = W.generate(2, 400, 64, 16, "f32", seed=81)
    inp.delta = np.broadcast_to(-inp.delta_bias, inp.u.shape).astype(np.float32).copy()
    h0 = np.random.default_rng(82).standard_normal((2, 64, 16)).astype(np.float32)
    o, last = _run(inp, h0=h0, softplus=False)
    assert np.array_equal(last, h0)
    ro, _ = oracle.scan_inputs(inp, h0=h0, softplus=False)
    assert parity_error(o, ro) <= TOL["f32"]


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("L", [200, 3000])
def test_reset_forgets_the_prefix_exactly(L, engine, request):
    _need_gpu()
    _engine(request, engine)
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
