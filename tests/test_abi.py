"""C ABI of libmamba_mi355x.so on the host: symbols, status strings, workspace
sizing and argument validation.  No kernel is launched: every call here is
rejected by the host-side checks before the HIP runtime is touched (the fake
device pointers are never dereferenced)."""
import ctypes
import os
import re

import pytest

from selective_state_space_22_amd import binding
from selective_state_space_22_amd import build as lib_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mamba_mi355x.h")

OK, ERR_NULL, ERR_DIM, ERR_UNSUPPORTED, ERR_DTYPE, ERR_WORKSPACE, ERR_ALIGN, ERR_HIP = range(8)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        lib_build.build()
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mamba_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "mamba_block_fwd", "mamba_block_fwd_workspace_size", "mamba_calibrate_copy", "mamba_get_option", "mamba_scan_bwd",
        "mamba_scan_bwd_workspace_size", "mamba_scan_fwd", "mamba_scan_fwd_complex",
        "mamba_scan_fwd_complex_workspace_size", "mamba_scan_fwd_noalloc", "mamba_scan_fwd_workspace_size",
        "mamba_selection_fwd",
        "mamba_selection_fwd_workspace_size", "mamba_set_option", "mamba_ssm_fwd", "mamba_ssm_fwd_workspace_size",
        "mamba_state_update", "mamba_state_update_complex", "mamba_status_string", "mamba_stream_status",
        "mamba_version"])


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(binding.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_version_and_status_strings(lib):
    assert lib.mamba_version() == 200
    seen = set()
    for st in range(10):
        s = binding.status_string(st)
        assert s and s not in seen
        seen.add(s)
    assert binding.status_string(99) == "unknown status"


def test_workspace_size_is_a_pure_function_of_shape(lib):
    ws = binding.mamba_scan_fwd_workspace_size
    assert ws(4, 4096, 5120, 16, 1) == ws(4, 4096, 5120, 16, 1)
    # the wave-private engine (N = 8, 16) runs every channel group through the whole
    # sequence when there are enough of them: no workspace
    assert ws(4, 4096, 5120, 16, 1) == 0
    assert ws(8, 2048, 1536, 16, 1) == 0
    # the lane engine (other N) runs short sequences in one piece: no workspace
    assert ws(1, 256, 64, 4, 0) == 0
    # few channel blocks and a long sequence: two passes over chunks, the workspace
    # holds the (batch, chunks, D, N+1) chunk aggregates after a 256-byte header, then
    # one int32 aggregate start per (batch, chunk, 64-channel block)
    w = ws(1, 1 << 20, 256, 16, 0)
    assert w > 256 and (w - 256) % (256 * 17 * 4 + 4 * 4) == 0
    # rejected shapes report 0
    assert ws(1, 16, 64, 3, 0) == 0
    assert ws(1, 16, 64, 16, 7) == 0
    assert ws(-1, 16, 64, 16, 0) == 0



@pytest.fixture
def restore_options(lib):
    keep = {k: binding.mamba_get_option(k) for k in range(1, 9)}
    yield
    for k, v in keep.items():
        binding.mamba_set_option(k, v)


def test_options_round_trip_and_validation(lib, restore_options):
    opts = [binding.MAMBA_OPT_ENGINE, binding.MAMBA_OPT_CHUNK, binding.MAMBA_OPT_WG_WAVES, binding.MAMBA_OPT_FUSED_DT,
            binding.MAMBA_OPT_BWD_CHUNK, binding.MAMBA_OPT_GEMM_GENERAL, binding.MAMBA_OPT_SPIN_LIMIT,
            binding.MAMBA_OPT_AGG_SKIP]
    assert opts == list(range(1, 9))
    # the wait bound starts at 2^24 sleeps (a few seconds) unless the environment set it
    for k, good, bad in [(binding.MAMBA_OPT_ENGINE, 3, 4), (binding.MAMBA_OPT_WG_WAVES, 4, 5),
                         (binding.MAMBA_OPT_FUSED_DT, 1, 2), (binding.MAMBA_OPT_GEMM_GENERAL, 1, -1),
                         (binding.MAMBA_OPT_CHUNK, 2048, -1), (binding.MAMBA_OPT_SPIN_LIMIT, 0, 1 << 32),
                         (binding.MAMBA_OPT_AGG_SKIP, 0, 2)]:
        binding.mamba_set_option(k, good)
        assert binding.mamba_get_option(k) == good
        with pytest.raises(binding.MambaError) as ex:
            binding.mamba_set_option(k, bad)
        assert ex.value.status == 9
        assert binding.mamba_get_option(k) == good  # a refused value leaves the option alone
    for k in (0, 9, 99, -1):
        assert binding.mamba_get_option(k) == -1
        with pytest.raises(binding.MambaError):
            binding.mamba_set_option(k, 0)


def test_workspace_follows_the_engine_option(lib, restore_options):
    ws = binding.mamba_scan_fwd_workspace_size
    shape = (4, 4096, 5120, 16, 1)
    binding.mamba_set_option(binding.MAMBA_OPT_ENGINE, binding.ENGINES["auto"])
    auto = ws(*shape)
    binding.mamba_set_option(binding.MAMBA_OPT_ENGINE, binding.ENGINES["wp"])
    assert ws(*shape) == auto == 0
    # the workgroup engine chains sequence chunks through a flag and carry workspace,
    # the lane engine's chunks store their aggregates
    binding.mamba_set_option(binding.MAMBA_OPT_ENGINE, binding.ENGINES["wg"])
    assert ws(*shape) > 0
    binding.mamba_set_option(binding.MAMBA_OPT_ENGINE, binding.ENGINES["lane"])
    assert ws(*shape) > 0
    binding.mamba_set_option(binding.MAMBA_OPT_ENGINE, binding.ENGINES["auto"])
    assert ws(*shape) == auto


def test_noalloc_refuses_shapes_beyond_its_scratch(lib, restore_options):
    """The no-allocation scan checks the workspace the shape needs against its fixed
    scratch array on the host, before the HIP runtime is touched."""
    assert binding.NOALLOC_MAX_WORKSPACE == 32 << 20
    binding.mamba_set_option(binding.MAMBA_OPT_ENGINE, binding.ENGINES["wg"])
    batch, L, D, N = 64, 1, 16384, 16   # 16 k chained channel blocks: 64 MiB of flags and carries
    assert binding.mamba_scan_fwd_workspace_size(batch, L, D, N, 0) > binding.NOALLOC_MAX_WORKSPACE
    st = lib.mamba_scan_fwd_noalloc(batch, L, D, N, 0, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None, 1, None,
                                    FAKE, None, None)
    assert st == ERR_WORKSPACE
    # shapes that mamba_scan_fwd rejects keep their own status
    assert lib.mamba_scan_fwd_noalloc(1, 8, 64, 3, 0, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None, 1, None,
                                      FAKE, None, None) == ERR_UNSUPPORTED

FAKE = 0x10000  # 16-byte aligned, never dereferenced


def scan_call(lib, batch=1, L=8, D=64, N=16, io=0, u=FAKE, delta=FAKE, bias=None, A=FAKE, B=FAKE, C=FAKE,
              Dskip=None, z=None, h0=None, out=FAKE, last=None, ws=None, ws_bytes=0):
    return lib.mamba_scan_fwd(batch, L, D, N, io, u, delta, bias, A, B, C, Dskip, z, 1, h0, out, last, ws, ws_bytes,
                              None)


def step_call(lib, batch=2, D=64, N=16, io=0, state=FAKE, u=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, out=FAKE,
              z=None):
    return lib.mamba_state_update(batch, D, N, io, state, u, delta, None, A, B, C, None, z, 1, out, None)


@pytest.mark.parametrize("field", ["u", "delta", "A", "B", "C", "out"])
def test_scan_rejects_null_required_pointer(lib, field):
    assert scan_call(lib, N=3, **{field: None}) == ERR_UNSUPPORTED  # shape checks come first
    assert scan_call(lib, **{field: None}) == ERR_NULL


def test_scan_rejects_bad_shapes_and_dtype(lib):
    assert scan_call(lib, io=2) == ERR_DTYPE
    assert scan_call(lib, batch=-1) == ERR_DIM
    assert scan_call(lib, L=-5) == ERR_DIM
    assert scan_call(lib, N=0) == ERR_DIM
    assert scan_call(lib, batch=70000) == ERR_DIM
    for n in (3, 5, 17, 32):
        assert scan_call(lib, N=n) == ERR_UNSUPPORTED


def test_scan_rejects_misaligned_pointers(lib):
    for field in ("u", "delta", "A", "B", "C", "out", "bias", "Dskip", "z", "h0", "last"):
        assert scan_call(lib, **{field: FAKE + 2}) == ERR_ALIGN, field


def test_scan_rejects_missing_or_small_workspace(lib):
    need = binding.mamba_scan_fwd_workspace_size(1, 1 << 20, 256, 16, 0)
    assert need > 0
    assert scan_call(lib, L=1 << 20, D=256) == ERR_WORKSPACE
    assert scan_call(lib, L=1 << 20, D=256, ws=FAKE, ws_bytes=need - 1) == ERR_WORKSPACE


def test_state_update_validation(lib):
    assert step_call(lib, io=5) == ERR_DTYPE
    assert step_call(lib, N=7) == ERR_UNSUPPORTED
    assert step_call(lib, D=-1) == ERR_DIM
    for field in ("state", "u", "delta", "A", "B", "C", "out"):
        assert step_call(lib, **{field: None}) == ERR_NULL, field
        assert step_call(lib, **{field: FAKE + 4}) == ERR_ALIGN, field
    assert step_call(lib, z=FAKE + 8) == ERR_ALIGN


def test_empty_problems_need_no_pointers(lib):
    # nothing to read or write: accepted without touching the device
    assert scan_call(lib, batch=0, u=None, delta=None, A=None, B=None, C=None, out=None) == OK
    assert scan_call(lib, D=0, u=None, delta=None, A=None, B=None, C=None, out=None) == OK
    assert step_call(lib, batch=0, state=None, u=None, delta=None, A=None, B=None, C=None, out=None) == OK


def test_python_binding_refuses_cpu_tensors(lib):
    torch = pytest.importorskip("torch")
    u = torch.zeros(1, 4, 64)
    with pytest.raises((ValueError, TypeError)):
        binding.mamba_scan_fwd(u, u, torch.zeros(64, 16), torch.zeros(1, 4, 16), torch.zeros(1, 4, 16))


def bwd_call(lib, batch=1, L=8, D=64, N=16, io=0, u=FAKE, delta=FAKE, bias=None, A=FAKE, B=FAKE, C=FAKE,
             Dskip=None, z=None, h0=None, dout=FAKE, dlast=None, du=FAKE, ddelta=FAKE, dA=FAKE, dB=FAKE, dC=FAKE,
             dDskip=None, dz=None, dbias=None, dh0=None, ws=None, ws_bytes=0):
    return lib.mamba_scan_bwd(batch, L, D, N, io, u, delta, bias, A, B, C, Dskip, z, 1, h0, dout, dlast, du, ddelta,
                              dA, dB, dC, dDskip, dz, dbias, dh0, ws, ws_bytes, None)


def test_bwd_workspace_size(lib):
    ws = binding.mamba_scan_bwd_workspace_size
    # per-chunk carries, tile-start states every 8 tokens and per-block dB/dC partials
    batch, L, D, N = 4, 4096, 5120, 16
    w = ws(batch, L, D, N, 1)
    assert w == ws(batch, L, D, N, 1)
    tile_states = batch * (L // 8) * D * N * 4
    partials = batch * (D // 64) * L * 2 * N * 4
    assert tile_states + partials < w < 1.2 * (tile_states + partials)
    assert ws(1, 0, 64, 16, 0) == 0
    assert ws(1, 16, 64, 3, 0) == 0 and ws(1, 16, 64, 16, 9) == 0


@pytest.mark.parametrize("field", ["u", "delta", "A", "B", "C", "dout", "du", "ddelta", "dA", "dB", "dC"])
def test_bwd_rejects_null_required_pointer(lib, field):
    need = binding.mamba_scan_bwd_workspace_size(1, 8, 64, 16, 0)
    assert bwd_call(lib, N=5, ws=FAKE, ws_bytes=need, **{field: None}) == ERR_UNSUPPORTED
    assert bwd_call(lib, ws=FAKE, ws_bytes=need, **{field: None}) == ERR_NULL


def test_bwd_rejects_misaligned_pointers_and_small_workspace(lib):
    need = binding.mamba_scan_bwd_workspace_size(1, 8, 64, 16, 0)
    for field in ("u", "delta", "A", "B", "C", "dout", "du", "ddelta", "dA", "dB", "dC", "bias", "Dskip", "z", "h0",
                  "dlast", "dDskip", "dz", "dbias", "dh0"):
        assert bwd_call(lib, ws=FAKE, ws_bytes=need, **{field: FAKE + 4}) == ERR_ALIGN, field
    assert bwd_call(lib) == ERR_WORKSPACE
    assert bwd_call(lib, ws=FAKE, ws_bytes=need - 1) == ERR_WORKSPACE
    assert bwd_call(lib, io=3) == ERR_DTYPE and bwd_call(lib, L=-1) == ERR_DIM


def test_bwd_empty_channel_dimension_is_a_no_op(lib):
    assert bwd_call(lib, D=0, u=None, delta=None, A=None, B=None, C=None, dout=None, du=None, ddelta=None, dA=None,
                    dB=None, dC=None) == OK


def test_selection_and_ssm_validation(lib):
    sel = lib.mamba_selection_fwd
    need = binding.mamba_selection_fwd_workspace_size(1, 8, 64, 16, 4, 0)
    assert need >= 8 * 40 * 4
    ok = dict(x=FAKE, wx=FAKE, wdt=FAKE, d=FAKE, b=FAKE, c=FAKE)

    def call(R=4, io=0, ws=FAKE, ws_bytes=need, **kw):
        p = {**ok, **kw}
        return sel(1, 8, 64, 16, R, io, p["x"], p["wx"], p["wdt"], p["d"], p["b"], p["c"], ws, ws_bytes, None)

    assert call(R=0) == ERR_DIM
    assert call(io=4) == ERR_DTYPE
    for k in ok:
        assert call(**{k: None}) == ERR_NULL, k
        assert call(**{k: FAKE + 2}) == ERR_ALIGN, k
    assert call(ws=None) == ERR_WORKSPACE and call(ws_bytes=need - 1) == ERR_WORKSPACE
    assert binding.mamba_selection_fwd_workspace_size(1, 8, 64, 16, 0, 0) == 0
    # the fused call checks the same way before touching the device
    ssm = lib.mamba_ssm_fwd
    nss = binding.mamba_ssm_fwd_workspace_size(1, 8, 64, 16, 4, 0)
    assert nss > need
    assert ssm(1, 8, 64, 16, 4, 0, FAKE, None, FAKE, FAKE, None, FAKE, None, 1, None, FAKE, None, FAKE, nss - 1,
               None) == ERR_WORKSPACE
    assert ssm(1, 8, 64, 16, 4, 0, None, None, FAKE, FAKE, None, FAKE, None, 1, None, FAKE, None, FAKE, nss,
               None) == ERR_NULL
    assert ssm(1, 8, 64, 16, 0, 0, FAKE, None, FAKE, FAKE, None, FAKE, None, 1, None, FAKE, None, FAKE, nss,
               None) == ERR_DIM


def test_complex_scan_validation_and_workspace(lib):
    ws = binding.mamba_scan_fwd_complex_workspace_size
    # the real scan's plans with two floats per state: N = 8, 16 hand (re, im) carries between
    # chunks of a channel block (64 channels x N x 2 floats per block, after the work counters) ...
    chains = 4 * 5120 // 64
    w = ws(4, 4096, 5120, 16, 1)
    assert chains * 64 * 16 * 8 <= w <= chains * 64 * 16 * 8 + 4096 + 4 * chains
    # ... or keep (batch, chunks, D, 2N+1) chunk aggregates after a 256-byte header
    w = ws(1, 1 << 20, 256, 16, 0)
    assert w > 256 and (w - 256) % (256 * 33 * 4) == 0
    # other N: the lane engine, no workspace for short rows
    assert ws(1, 256, 64, 4, 0) == 0
    assert ws(1, 16, 64, 3, 0) == 0 and ws(1, 16, 64, 16, 9) == 0

    def call(batch=1, L=8, D=64, N=16, io=0, u=FAKE, A=FAKE, out=FAKE, h0=None, ws_ptr=None, ws_bytes=0):
        return lib.mamba_scan_fwd_complex(batch, L, D, N, io, u, FAKE, None, A, FAKE, FAKE, None, None, 1, h0, out,
                                          None, ws_ptr, ws_bytes, None)

    assert call(io=3) == ERR_DTYPE
    assert call(N=5) == ERR_UNSUPPORTED
    assert call(L=-1) == ERR_DIM
    assert call(u=None) == ERR_NULL and call(A=None) == ERR_NULL and call(out=None) == ERR_NULL
    assert call(A=FAKE + 8) == ERR_ALIGN and call(h0=FAKE + 4) == ERR_ALIGN
    assert call(L=1 << 20, D=256) == ERR_WORKSPACE
    assert call(L=1 << 20, D=256, ws_ptr=FAKE, ws_bytes=w - 1) == ERR_WORKSPACE
    assert call(batch=0, u=None, A=None, out=None) == OK


def test_complex_state_update_validation(lib):
    def call(batch=2, D=64, N=16, io=0, state=FAKE, u=FAKE, A=FAKE, out=FAKE):
        return lib.mamba_state_update_complex(batch, D, N, io, state, u, FAKE, None, A, FAKE, FAKE, None, None, 1,
                                              out, None)

    assert call(io=4) == ERR_DTYPE
    assert call(N=3) == ERR_UNSUPPORTED
    assert call(D=-1) == ERR_DIM
    for field in ("state", "u", "A", "out"):
        assert call(**{field: None}) == ERR_NULL, field
        assert call(**{field: FAKE + 4}) == ERR_ALIGN, field
    assert call(batch=0, state=None, u=None, A=None, out=None) == OK


def test_block_validation_and_workspace(lib):
    ws = binding.mamba_block_fwd_workspace_size
    # x, z and y of the block ahead of the selective SSM's workspace
    tok, D = 4 * 4096, 5120
    need = ws(4, 4096, 2560, D, 16, 160, 1)
    assert need >= 3 * tok * D * 2 + binding.mamba_ssm_fwd_workspace_size(4, 4096, D, 16, 160, 1)
    assert ws(1, 8, 0, 64, 16, 4, 0) == 0 and ws(1, 8, 32, 64, 16, 0, 0) == 0 and ws(1, 8, 32, 64, 5, 4, 0) == 0

    def call(d_model=32, R=4, N=16, io=0, hidden=FAKE, W_in=FAKE, W_out=FAKE, out=FAKE, ws_ptr=None, ws_bytes=0):
        return lib.mamba_block_fwd(1, 8, d_model, 64, N, R, io, hidden, W_in, FAKE, FAKE, None, FAKE, None, W_out, 1,
                                   None, out, None, ws_ptr, ws_bytes, None)

    assert call(io=2) == ERR_DTYPE
    assert call(N=3) == ERR_UNSUPPORTED
    assert call(d_model=0) == ERR_DIM and call(R=0) == ERR_DIM
    for field in ("hidden", "W_in", "W_out", "out"):
        assert call(**{field: None}) == ERR_NULL, field
        assert call(**{field: FAKE + 2}) == ERR_ALIGN, field
    assert call() == ERR_WORKSPACE
    assert call(ws_ptr=FAKE, ws_bytes=ws(1, 8, 32, 64, 16, 4, 0) - 1) == ERR_WORKSPACE
