"""The C-ABI calls captured in a HIP graph (through torch.cuda.CUDAGraph): each
replay, with eager work and synchronisation in between, must reproduce the
eager result bit for bit.  The scan's work counters are cleared by a small
fill kernel (no memset node), which is what these replays exercise."""
import numpy as np
import pytest

from gpu_util import to_device
from selective_state_space_22_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


SCAN_GRAPH_CASES = [((5, 1100, 4096, 16, "bf16"), "default"),  # the wave-private mixed launch
                    ((5, 1100, 4096, 16, "bf16"), "wg"),       # chained chunks: ticket, flags, carries
                    ((1, 4096, 64, 16, "f32"), "default"),     # two passes over chunks
                    ((1, 300, 64, 4, "f32"), "default")]       # lane engine


@pytest.mark.parametrize("shape,engine", SCAN_GRAPH_CASES, ids=["wave_private", "chained", "split", "lane"])
def test_scan_graph_replays_match_eager(shape, engine, request):
    _need_gpu()
    from gpu_util import force_engine
    from selective_state_space_22_amd import binding

    force_engine(request, engine)
    batch, L, D, N, io = shape
    print(f"\n[gpu-test] graph replay of mamba_scan_fwd {shape} engine={engine}", flush=True)
    inp = W.generate(batch, L, D, N, io, seed=123)
    d = to_device(inp)
    out = torch.empty_like(d["u"])
    last = torch.empty((batch, D, N), dtype=torch.float32, device="cuda")
    ws_bytes = binding.mamba_scan_fwd_workspace_size(batch, L, D, N, 1 if io == "bf16" else 0)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def call():
        binding.mamba_scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["delta_bias"], d["Dskip"], d["z"], True,
                               None, out=out, last_state=last, workspace=ws)

    call()
    torch.cuda.synchronize()
    ref_out, ref_last = out.clone(), last.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm the stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        out.fill_(float("nan"))
        last.fill_(float("nan"))
        ws.fill_(rep * 37 % 256)  # scratch contents must not matter
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {rep}: out differs"
        assert torch.equal(last, ref_last), f"replay {rep}: last_state differs"
        _ = (d["u"].float() * 2).sum().item()  # unrelated eager work between replays


def test_decode_graph_replays_match_eager():
    _need_gpu()
    from selective_state_space_22_amd import mamba_state_update

    print("\n[gpu-test] graph replay of 16 decode steps", flush=True)
    inp = W.generate(8, 16, 640, 16, "bf16", seed=321)
    d = to_device(inp)
    steps = [{k: d[k][:, t].contiguous() for k in ("u", "delta", "B", "C", "z")} for t in range(16)]
    state = torch.zeros((8, 640, 16), dtype=torch.float32, device="cuda")
    outs = [torch.empty_like(steps[0]["u"]) for _ in range(16)]

    def run():
        for t in range(16):
            st = steps[t]
            mamba_state_update(state, st["u"], st["delta"], d["A"], st["B"], st["C"], d["delta_bias"], d["Dskip"],
                               st["z"], True, out=outs[t])

    run()
    torch.cuda.synchronize()
    ref_outs = [o.clone() for o in outs]
    ref_state = state.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        state.zero_()
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        state.zero_()
        for o in outs:
            o.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(outs, ref_outs)), f"replay {rep}: outputs differ"
        assert torch.equal(state, ref_state), f"replay {rep}: state differs"
        _ = float(np.asarray(state[0, 0].cpu()).sum())


def _stream_status():
    """The library's chained-wait status of the current device ("ok" or the error it reports)."""
    from selective_state_space_22_amd import binding

    try:
        binding._check_status("replay", torch.device("cuda"))
        return "ok"
    except Exception as ex:  # the status itself is the diagnostic here
        return str(ex)


def _replay_matches(call, outputs, reps=3):
    """Capture call() in a graph; every replay (with eager work in between) reproduces the eager outputs."""
    call()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outputs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(reps):
        for o in outputs:
            o.fill_(float("nan") if o.is_floating_point() else 0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outputs, ref)):
            if not torch.equal(o, r):
                of, rf = o.float(), r.float()
                bad = of != rf
                raise AssertionError(
                    f"replay {rep}: output {i} differs at {int(bad.sum())} of {o.numel()} elements "
                    f"({int(torch.isnan(of).sum())} NaN), largest difference "
                    f"{float((of - rf).abs().nan_to_num(0).max()):.3e}, first at {bad.nonzero()[:3].tolist()}; "
                    f"stream status: {_stream_status()}")
        _ = float(outputs[0].float().sum().item())  # unrelated eager work between replays


def test_backward_graph_replays_match_eager():
    _need_gpu()
    from selective_state_space_22_amd import binding

    print("\n[gpu-test] graph replay of mamba_scan_bwd (2, 700, 200, 16) bf16", flush=True)
    inp = W.generate(2, 700, 200, 16, "bf16", seed=55)
    gi = W.grad_inputs(2, 700, 200, 16, "bf16", seed=55)
    d = to_device(inp)
    dout = torch.from_numpy(gi.dout).cuda().to(torch.bfloat16)
    dl = torch.from_numpy(gi.dlast).cuda()
    grads = {"du": torch.empty_like(d["u"]), "ddelta": torch.empty_like(d["u"]), "dz": torch.empty_like(d["u"]),
             "dB": torch.empty_like(d["B"]), "dC": torch.empty_like(d["C"]),
             "dA": torch.empty((200, 16), device="cuda"), "dDskip": torch.empty(200, device="cuda"),
             "ddelta_bias": torch.empty(200, device="cuda"), "dh0": torch.empty((2, 200, 16), device="cuda")}
    ws = torch.empty(binding.mamba_scan_bwd_workspace_size(2, 700, 200, 16, 1), dtype=torch.uint8, device="cuda")

    def call():
        binding.mamba_scan_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], dout, d["delta_bias"], d["Dskip"], d["z"],
                               True, None, dl, grads=grads, workspace=ws)

    _replay_matches(call, list(grads.values()))


def test_ssm_graph_replays_match_eager():
    _need_gpu()
    from selective_state_space_22_amd import binding

    print("\n[gpu-test] graph replay of mamba_ssm_fwd (2, 600, 256, 16) bf16", flush=True)
    inp = W.generate(2, 600, 256, 16, "bf16", seed=66)
    sw = W.selection_weights(256, 16, 8, "bf16", seed=66)
    d = to_device(inp)
    wx = torch.from_numpy(sw.W_x).cuda().to(torch.bfloat16)
    wdt = torch.from_numpy(sw.W_dt).cuda().to(torch.bfloat16)
    out = torch.empty_like(d["u"])
    last = torch.empty((2, 256, 16), device="cuda")
    ws = torch.empty(binding.mamba_ssm_fwd_workspace_size(2, 600, 256, 16, 8, 1), dtype=torch.uint8, device="cuda")

    def call():
        binding.mamba_ssm_fwd(d["u"], wx, wdt, d["A"], z=d["z"], dt_bias=d["delta_bias"], Dskip=d["Dskip"], out=out,
                              last_state=last, workspace=ws)

    _replay_matches(call, [out, last])


@pytest.mark.parametrize("shape", [(5, 1100, 4096, 16, "bf16"), (1, 4096, 64, 16, "f32"), (1, 600, 64, 4, "f32")],
                         ids=["chained", "split", "lane"])
def test_complex_scan_graph_replays_match_eager(shape):
    """mamba_scan_fwd_complex on the workgroup engine (chained and split, whose carry
    pass composes complex aggregates) and on the lane kernels."""
    _need_gpu()
    from selective_state_space_22_amd import binding

    batch, L, D, N, io = shape
    print(f"\n[gpu-test] graph replay of mamba_scan_fwd_complex {shape}", flush=True)
    inp = W.generate(batch, L, D, N, io, seed=321)
    d = to_device(inp)
    A = torch.from_numpy(W.a_init_complex(D, N)).cuda()
    h0 = torch.randn((batch, D, N), dtype=torch.complex64, device="cuda")
    out = torch.empty_like(d["u"])
    last = torch.empty((batch, D, N, 2), device="cuda")
    ws = torch.empty(max(binding.mamba_scan_fwd_complex_workspace_size(batch, L, D, N, 1 if io == "bf16" else 0), 1),
                     dtype=torch.uint8, device="cuda")

    def call():
        binding.mamba_scan_fwd_complex(d["u"], d["delta"], A, d["B"], d["C"], d["delta_bias"], d["Dskip"], d["z"], True,
                                       h0, out=out, last_state=last, workspace=ws)

    _replay_matches(call, [out, last])


def test_complex_decode_graph_replays_match_eager():
    _need_gpu()
    from selective_state_space_22_amd import binding

    print("\n[gpu-test] graph replay of 8 mamba_state_update_complex steps (4, 512, 16) bf16", flush=True)
    inp = W.generate(4, 8, 512, 16, "bf16", seed=77)
    d = to_device(inp)
    A = torch.from_numpy(W.a_init_complex(512, 16)).cuda()
    state0 = torch.randn((4, 512, 16), dtype=torch.complex64, device="cuda")
    state = state0.clone()
    steps = [(d["u"][:, t].contiguous(), d["delta"][:, t].contiguous(), d["B"][:, t].contiguous(),
              d["C"][:, t].contiguous(), d["z"][:, t].contiguous()) for t in range(8)]
    outs = [torch.empty_like(steps[0][0]) for _ in range(8)]
    view = torch.view_as_real(state)

    def call():
        state.copy_(state0)
        for (u, dl, B, C, z), o in zip(steps, outs):
            binding.mamba_state_update_complex(state, u, dl, A, B, C, d["delta_bias"], d["Dskip"], z, True, out=o)

    _replay_matches(call, outs + [view])


def test_block_graph_replays_match_eager():
    """mamba_block_fwd captured whole: the projections on the persistent large-product
    kernel, the selection GEMMs with their split-K reduction, and the scan."""
    _need_gpu()
    from selective_state_space_22_amd import binding
    from gpu_util import torch_io

    batch, L, dm, D, N, R, io = 2, 600, 520, 1040, 16, 66, "bf16"
    print(f"\n[gpu-test] graph replay of mamba_block_fwd {(batch, L, dm, D, N, R, io)}", flush=True)
    inp = W.generate(batch, 1, D, N, io, seed=321)
    sw = W.selection_weights(D, N, R, io, seed=321)
    bw = W.block_weights(dm, D, io, seed=321)
    hidden = torch_io(W.block_hidden(batch, L, dm, io, seed=321), io, "cuda")
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    win, wx, wdt, wout = (torch_io(w, io, "cuda") for w in (bw.W_in, sw.W_x, sw.W_dt, bw.W_out))
    A, bias, dskip = f(inp.A), f(inp.delta_bias), f(inp.Dskip)
    out = torch.empty_like(hidden)
    last = torch.empty((batch, D, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(binding.mamba_block_fwd_workspace_size(batch, L, dm, D, N, R, 1), 1), dtype=torch.uint8,
                     device="cuda")

    def call():
        binding.mamba_block_fwd(hidden, win, wx, wdt, A, wout, dt_bias=bias, Dskip=dskip, out=out, last_state=last,
                                workspace=ws)

    call()
    torch.cuda.synchronize()
    ref_out, ref_last = out.clone(), last.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm the stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        out.fill_(float("nan"))
        last.fill_(float("nan"))
        ws.fill_(rep * 37 % 256)  # scratch contents must not matter
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {rep}: out differs"
        assert torch.equal(last, ref_last), f"replay {rep}: last_state differs"
        _ = (hidden.float() * 2).sum().item()  # unrelated eager work between replays
