"""The Mamba block (mamba_block_fwd: input projection with the SiLU SSM branch
and the gate branch, selective SSM, output projection) against the fp64 oracle's
block on the GPU.  Tolerances as everywhere: 1e-4 for fp32 I/O, 2e-2 for bf16 I/O;
with bf16 I/O the intermediate tensors x, z, delta, B, C and y are bf16 on both sides."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, parity_error, to_host, torch_io
from selective_state_space_22_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _store(io):
    if io != "bf16":
        return None
    return lambda a: W.bf16_round(np.asarray(a, np.float32))[1].reshape(np.shape(a)).astype(np.float64)


def _problem(batch, L, dm, D, N, R, io, seed):
    inp = W.generate(batch, 1, D, N, io, seed=seed)  # A, dt_bias and Dskip of the workload recipe
    sw = W.selection_weights(D, N, R, io, seed=seed)
    bw = W.block_weights(dm, D, io, seed=seed)
    hidden = W.block_hidden(batch, L, dm, io, seed=seed)
    return inp, sw, bw, hidden


def _gpu_block(inp, sw, bw, hidden, io, h0=None):
    from selective_state_space_22_amd import mamba_block_fwd

    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    out, last = mamba_block_fwd(torch_io(hidden, io, "cuda"), torch_io(bw.W_in, io, "cuda"),
                                torch_io(sw.W_x, io, "cuda"), torch_io(sw.W_dt, io, "cuda"), f(inp.A),
                                torch_io(bw.W_out, io, "cuda"), dt_bias=f(inp.delta_bias), Dskip=f(inp.Dskip),
                                h0=None if h0 is None else f(h0))
    torch.cuda.synchronize()
    return to_host(out), last.cpu().numpy()


@pytest.mark.parametrize("case", [
    (2, 77, 48, 96, 16, 8, "f32"),      # every projection on MFMA, ragged token count
    (2, 300, 64, 128, 16, 8, "bf16"),
    (1, 64, 40, 72, 4, 5, "bf16"),      # rows not 16-byte aligned: vector GEMM paths
    (1, 129, 768, 1536, 16, 48, "bf16"),  # Mamba-130M block widths
    (2, 200, 96, 192, 8, 12, "f32"),
    (2, 600, 520, 1040, 16, 66, "bf16"),  # large-block GEMM kernel: ragged rows, columns and K
    (2, 600, 520, 1040, 8, 66, "f32"),
    (2, 520, 512, 1036, 16, 66, "bf16"),  # large-block input projection, output rows 8-byte but not 16-byte aligned
    (2, 520, 512, 1034, 8, 66, "bf16"),   # D not a multiple of 4: input projection on the general kernel
    (2, 600, 256, 1024, 8, 66, "f32"),    # both input-projection halves in one launch
    (2, 3800, 512, 1280, 16, 66, "bf16"),  # one launch, ragged rows, split last round with x and z blocks
], ids=str)
def test_block_matches_oracle(case):
    _need_gpu()
    batch, L, dm, D, N, R, io = case
    print(f"\n[gpu-test] mamba block {case}", flush=True)
    inp, sw, bw, hidden = _problem(batch, L, dm, D, N, R, io, seed=W.SEED_BASE + 300 + L)
    go, gl = _gpu_block(inp, sw, bw, hidden, io)
    ro, rl = oracle.block(hidden, bw.W_in, sw.W_x, sw.W_dt, inp.delta_bias, inp.A, inp.Dskip, bw.W_out, N,
                          store=_store(io))
    assert np.isfinite(go).all()
    eo, el = parity_error(go, ro), parity_error(gl, rl)
    print(f"block {case}: out err {eo:.3e} last err {el:.3e}")
    assert eo <= TOL[io] and el <= TOL[io]


def test_block_mamba3b_shape_row_sampled():
    """Mamba-3B block widths (d_model 2560, D 5120, N 16, dt rank 160), batch 4 x 4096
    tokens in bf16 on the GPU; batch row 0 against the oracle (every token and channel)."""
    _need_gpu()
    print("\n[gpu-test] mamba block (4, 4096, 2560 -> 5120, 16, R 160) bf16, row 0 against the oracle", flush=True)
    w = W.WORKLOADS["mamba3b_layer"]
    inp, sw, bw, hidden = _problem(4, 4096, 2560, 5120, 16, 160, "bf16", seed=w.seed)
    go, gl = _gpu_block(inp, sw, bw, hidden, "bf16")
    ro, rl = oracle.block(hidden[:1], bw.W_in, sw.W_x, sw.W_dt, inp.delta_bias, inp.A, inp.Dskip, bw.W_out, 16,
                          store=_store("bf16"))
    eo, el = parity_error(go[:1], ro), parity_error(gl[:1], rl)
    print(f"mamba3b block row 0: out err {eo:.3e} last err {el:.3e}")
    assert np.isfinite(go).all() and eo <= TOL["bf16"] and el <= TOL["bf16"]


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_block_initial_state_matches_oracle(io):
    """An initial state h0 enters the selective SSM of the block (the oracle's block with the same h0)."""
    _need_gpu()
    batch, L, dm, D, N, R = 2, 150, 96, 192, 16, 12
    print(f"\n[gpu-test] mamba block with h0 {io}", flush=True)
    inp, sw, bw, hidden = _problem(batch, L, dm, D, N, R, io, seed=W.SEED_BASE + 410)
    h0 = np.random.default_rng(7).standard_normal((batch, D, N)).astype(np.float32)
    go, gl = _gpu_block(inp, sw, bw, hidden, io, h0=h0)
    ro, rl = oracle.block(hidden, bw.W_in, sw.W_x, sw.W_dt, inp.delta_bias, inp.A, inp.Dskip, bw.W_out, N,
                          h0=h0.astype(np.float64), store=_store(io))
    eo, el = parity_error(go, ro), parity_error(gl, rl)
    print(f"block with h0 {io}: out err {eo:.3e} last err {el:.3e}")
    assert eo <= TOL[io] and el <= TOL[io]


def test_block_chains_over_the_sequence():
    """Two calls over the halves of a sequence, the second from the first one's last state, give the
    outputs and last state of one call over the whole sequence (the projections act per token)."""
    _need_gpu()
    batch, L, dm, D, N, R, io = 2, 300, 64, 128, 16, 8, "f32"
    print("\n[gpu-test] mamba block chained over two halves", flush=True)
    inp, sw, bw, hidden = _problem(batch, L, dm, D, N, R, io, seed=W.SEED_BASE + 420)
    full_o, full_l = _gpu_block(inp, sw, bw, hidden, io)
    o1, l1 = _gpu_block(inp, sw, bw, np.ascontiguousarray(hidden[:, :L // 2]), io)
    o2, l2 = _gpu_block(inp, sw, bw, np.ascontiguousarray(hidden[:, L // 2:]), io, h0=l1)
    eo = parity_error(np.concatenate([o1, o2], axis=1), full_o)
    el = parity_error(l2, full_l)
    print(f"chained block: out err {eo:.3e} last err {el:.3e}")
    assert eo <= TOL[io] and el <= TOL[io]


def test_block_empty_sequence_passes_the_state():
    """No tokens: no output rows, and the last state is the initial state (zero without one)."""
    _need_gpu()
    batch, dm, D, N, R, io = 2, 64, 128, 16, 8, "f32"
    print("\n[gpu-test] mamba block with no tokens", flush=True)
    inp, sw, bw, _ = _problem(batch, 1, dm, D, N, R, io, seed=W.SEED_BASE + 430)
    hidden = np.zeros((batch, 0, dm), np.float32)
    h0 = np.random.default_rng(3).standard_normal((batch, D, N)).astype(np.float32)
    o, last = _gpu_block(inp, sw, bw, hidden, io, h0=h0)
    assert o.shape == (batch, 0, dm)
    assert np.array_equal(last, h0)
    _, last0 = _gpu_block(inp, sw, bw, hidden, io)
    assert not np.any(last0)
