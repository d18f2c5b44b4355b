#!/usr/bin/env python3
"""Benchmark of the MI355X selective scan (S6) forward pass.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one mamba_scan_fwd call over the whole workload (all of the
discretisation, scan, readout and epilogue), inputs already resident in HBM.
Prints ONE JSON line.  Default workload: the Mamba-3B layer shape
(batch 4, L 4096, D 5120, N 16, bf16 I/O, fp32 state), seeded synthetic data.

Other workloads (--workload): tiny, mamba130m_layer, million_tokens, decode
(decode: one step = 64 one-token state updates of (256, 5120, 16)).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
VALU_FP32_PEAK_TFLOPS = 78.6    # 256 CU x 4 SIMD x 16 lanes x 2 (FMA) x 2.4 GHz, non-packed fp32
VALU_FP32_PACKED_TFLOPS = 157.3  # published fp32 vector peak (packed fp32, not used by this code)
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix peak, published
MFMA_F32_PEAK_TFLOPS = 157.3     # dense fp32 matrix peak, published
# Algorithmic fp32 operations (FMA = 2, other ops and transcendentals = 1):
# per (b, l, d, n): dt*A (1), exp (1), input weight (Abar - 1)/A as one FMA (2), B*x (1), beta*Bx (1),
# h FMA (2), readout FMA (2); the small-dt*A guard of the input weight is not counted
FLOPS_PER_ELEMENT = 10.0
FLOPS_PER_TOKEN_CHANNEL = 15.0   # per (b, l, d): bias add, softplus (6), skip FMA, SiLU (5), gate mul
# Backward, per (b, l, d, n) on top of the recomputed forward: gradient recurrence FMA, dC and dB products,
# du FMA, d(beta) and d(Abar) products, ddt FMAs, d beta/d A (series or difference), two dA FMAs, state-gradient decay
BWD_FLOPS_PER_ELEMENT = 22.0
# Complex A, per (b, l, d, n): dt*A (2), |Abar| exp and the sin/cos pair (3), Abar (2), (Abar-1)/A (7),
# B*x (1), beta*Bx (2), complex h update (8), readout FMA on Re h (2)
COMPLEX_FLOPS_PER_ELEMENT = 27.0


def algorithmic_bytes(batch, L, D, N, io_bytes, decode=False):
    """Bytes a perfect kernel must move: each input read once, each output written once."""
    if decode:  # per step: state read + write, per-token operands
        return 8 * batch * D * N + 4 * io_bytes * batch * D + 2 * io_bytes * batch * N + 4 * D * N + 8 * D
    return 4 * io_bytes * batch * L * D + 2 * io_bytes * batch * L * N + 4 * D * N + 8 * D + 4 * batch * D * N


# The headline metric: forward elements per second on the Mamba-3B layer shape,
# reported with the achieved HBM bandwidth.
FWD_METRIC = "selective-scan fwd elements(B\u00b7L\u00b7D\u00b7N)/s + achieved HBM GB/s, Mamba-3B layer"


def cpu_baseline(inp, name, which="fwd"):
    """The fp64 oracle on a bounded sample of the same workload, timed on the host cores."""
    import numpy as np

    import oracle
    from selective_state_space_22_amd import workloads as W

    rows = {"mamba3b_layer": 2, "mamba130m_layer": 2, "tiny": 1, "million_tokens": 1, "decode": 64}.get(name, 1)
    if name == "million_tokens":
        sub = W.channel_subset(inp, [0], np.arange(0, inp.dim, 4))  # 64 channels, all 2^20 tokens
        what = "batch row 0, 64 of 256 channels, all 1048576 tokens"
    elif name == "decode":
        sub = W.channel_subset(inp, np.arange(rows), np.arange(inp.dim))
        what = f"{rows} of 256 sequences, all 5120 channels, 64 tokens"
    else:
        rows = min(rows, inp.batch)
        sub = W.channel_subset(inp, np.arange(rows), np.arange(inp.dim))
        what = f"batch rows 0..{rows - 1} of {inp.batch}, all channels and tokens"
    args = [np.ascontiguousarray(x, np.float64) if x is not None else None
            for x in (sub.u, sub.delta, sub.A, sub.B, sub.C, sub.delta_bias, sub.Dskip, sub.z)]
    threads = oracle.max_threads()
    min_s, max_calls = 10.0, 64  # repeat the sample until about 10 s of CPU work has run

    def timed(fn):
        calls, t0 = 0, time.perf_counter()
        while True:
            fn()
            calls += 1
            el = time.perf_counter() - t0
            if el >= min_s or calls >= max_calls:
                return el / calls, calls

    if which == "complex":
        Ac = W.a_init_complex(sub.dim, sub.dstate).astype(np.complex128)
        dt, calls = timed(lambda: oracle.scan_complex(args[0], args[1], Ac, args[3], args[4], args[5], args[6],
                                                      args[7], softplus=True, nthreads=threads))
        what += " (complex A)"
    elif which == "bwd":
        if name != "million_tokens":  # one batch row: the backward oracle is ~3x the forward's work
            sub = W.channel_subset(inp, [0], np.arange(inp.dim))
            what = f"batch row 0 of {inp.batch}, all channels and tokens"
            args = [np.ascontiguousarray(x, np.float64) if x is not None else None
                    for x in (sub.u, sub.delta, sub.A, sub.B, sub.C, sub.delta_bias, sub.Dskip, sub.z)]
        gi = W.grad_inputs(sub.batch, sub.seqlen, sub.dim, sub.dstate, "f32", seed=1)
        dt, calls = timed(lambda: oracle.scan_bwd(args[0], args[1], args[2], args[3], args[4], gi.dout, args[5],
                                                  args[6], args[7], softplus=True, dlast=gi.dlast, nthreads=threads))
        what += " (backward)"
    else:
        dt, calls = timed(lambda: oracle.scan(*args, softplus=True, nthreads=threads))
    elems = sub.batch * sub.seqlen * sub.dim * sub.dstate
    return {"value": elems / dt, "unit": "elements/s", "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{what}; {elems} elements per call, {calls} calls, {dt:.3f} s wall per call "
                      "(fp64, OpenMP over (batch, channel))"}


def cpu_model():
    """The host CPU's model name (first processor entry of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def source_sha256(files):
    """Hash of the named HIP source files (csrc/): counter readings taken on other sources do not apply."""
    import hashlib

    h = hashlib.sha256()
    for name in sorted(files):
        h.update(name.encode())
        with open(os.path.join(ROOT, "selective_state_space_22_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, which="fwd"):
    """HBM bytes per launch of the dominant kernel from the committed PMC readings, or None
    when there is no reading or the kernel's sources changed since it was taken."""
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            rec = json.load(f)
        w = rec["workloads"].get(workload if which == "fwd" else f"{workload}:{which}")
        if w is None or source_sha256(w["sources"]) != w["source_sha256"]:
            return None
        return int(w["bytes"])
    except (OSError, ValueError, KeyError):
        return None


def calibrate_copy(torch, dev, mib, steps, flush, settle_ms):
    """HBM reference for the memory-bound kernels: the library's hand-written
    streaming copy (and torch's copy_) of mib MiB, each launch reading and writing
    mib MiB, warm or with the Infinity Cache evicted before every launch; one JSON
    line per grid size."""
    from selective_state_space_22_amd import binding

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    flush_buf = torch.empty(1 << 28, dtype=torch.float32, device=dev) if flush else None
    kernels = [(f"hip stream copy, {g} blocks", lambda g=g: binding.mamba_calibrate_copy(src, dst, g))
               for g in (2048, 4096, 16384)]
    kernels += [("hip block copy", lambda: binding.mamba_calibrate_copy(src, dst, 0)),
                ("hip block copy, non-temporal", lambda: binding.mamba_calibrate_copy(src, dst, -1)),
                ("hip in place", lambda: binding.mamba_calibrate_copy(src, dst, -2)),
                ("hip in place, non-temporal", lambda: binding.mamba_calibrate_copy(src, dst, -3))]
    kernels.append(("torch copy_", lambda: dst.copy_(src)))
    best = None
    for name, fn in kernels:
        for _ in range(3):
            fn()
        # settle the clock as for the scan
        t_end = time.perf_counter() + settle_ms / 1e3
        while time.perf_counter() < t_end:
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
        for k in range(steps):
            if flush:
                flush_buf.fill_(float(k))
            ev[2 * k].record()
            fn()
            ev[2 * k + 1].record()
        torch.cuda.synchronize()
        ms = sum(ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(steps)) / steps
        gbps = 8 * n / (ms * 1e-3) / 1e9
        rec = {"calibration": name, "bytes_read": 4 * n, "bytes_written": 4 * n, "flushed": bool(flush),
               "launches": steps, "ms_per_copy": ms, "gbps": gbps}
        print(json.dumps(rec), flush=True)
        if name.startswith("hip") and (best is None or gbps > best["gbps"]):
            best = rec
    print(json.dumps({"calibration_best": best}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mamba3b_layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=150.0,
                    help="untimed steps for this long before the warmup (the clock rises under load); 0 = none")
    ap.add_argument("--flush", action="store_true", help="evict the 256 MB Infinity Cache before every step")
    ap.add_argument("--graph", choices=["auto", "on", "off"], default="auto",
                    help="replay each step from a captured HIP graph (auto: on for decode, whose step is 64 launches)")
    ap.add_argument("--pass", dest="which", choices=["fwd", "bwd", "sel", "ssm", "complex", "block"], default="fwd",
                    help="fwd: mamba_scan_fwd (the headline); bwd: mamba_scan_bwd on the same workload; "
                         "complex: mamba_scan_fwd_complex with A_n = -1/2 + n i; "
                         "block: mamba_block_fwd, d_model = D / 2 (input and output projections around ssm); "
                         "sel: the selection projections (mamba_selection_fwd, dt rank d_model/16); "
                         "ssm: selection then scan (mamba_ssm_fwd)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run plain device copies of MIB MiB (the hand-written streaming copy at several grid "
                         "sizes, and torch's): the HBM reference for memory-bound kernels and for byte counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: measures one GPU only (the scan shards over batch and channels with no "
              "exchange; each GPU would run this kernel on its share); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from selective_state_space_22_amd import binding
    from selective_state_space_22_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        calibrate_copy(torch, dev, args.calibrate_copy, args.steps, args.flush, args.settle_ms)
        return
    w = W.WORKLOADS[args.workload]
    if args.which != "fwd" and w.decode_steps > 0:
        print("bench.py: --pass bwd/sel/ssm/complex/block apply to the full-sequence workloads, not decode",
              file=sys.stderr)
        sys.exit(2)
    inp = W.generate_workload(args.workload)
    tdt = torch.bfloat16 if w.io == "bf16" else torch.float32
    io_bytes = 2 if w.io == "bf16" else 4

    def t(x):
        return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev).to(tdt)

    def f(x):
        return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)

    u, delta, z, B, C = t(inp.u), t(inp.delta), t(inp.z), t(inp.B), t(inp.C)
    A, bias, dskip = f(inp.A), f(inp.delta_bias), f(inp.Dskip)
    decode = w.decode_steps > 0
    stream = torch.cuda.current_stream(dev)
    flush_buf = torch.empty(1 << 28, dtype=torch.float32, device=dev) if args.flush else None

    if decode:
        batch, L, D, N = w.batch, w.seqlen, w.dim, w.dstate
        steps_in = [(u[:, k].contiguous(), delta[:, k].contiguous(), B[:, k].contiguous(), C[:, k].contiguous(),
                     z[:, k].contiguous()) for k in range(L)]
        state = torch.zeros((batch, D, N), dtype=torch.float32, device=dev)
        outs = [torch.empty_like(steps_in[0][0]) for _ in range(L)]

        def step():  # the state carries over between steps; the work per step is the same
            for k in range(L):
                uu, dd, bb, cc, zz = steps_in[k]
                binding.mamba_state_update(state, uu, dd, A, bb, cc, bias, dskip, zz, True, out=outs[k])

        units = batch * L * D * N
        bytes_per_step = algorithmic_bytes(batch, L, D, N, io_bytes, decode=True) * L
    elif args.which == "bwd":
        from selective_state_space_22_amd import workloads as Wl

        gi = Wl.grad_inputs(w.batch, w.seqlen, w.dim, w.dstate, w.io, seed=w.seed)
        dout, dlast = t(gi.dout), f(gi.dlast)
        grads = {"du": torch.empty_like(u), "ddelta": torch.empty_like(u), "dz": torch.empty_like(u),
                 "dB": torch.empty_like(B), "dC": torch.empty_like(C),
                 "dA": torch.empty((w.dim, w.dstate), dtype=torch.float32, device=dev),
                 "dDskip": torch.empty(w.dim, dtype=torch.float32, device=dev),
                 "ddelta_bias": torch.empty(w.dim, dtype=torch.float32, device=dev),
                 "dh0": torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device=dev)}
        ws_bytes = binding.mamba_scan_bwd_workspace_size(w.batch, w.seqlen, w.dim, w.dstate,
                                                         1 if w.io == "bf16" else 0)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

        def step():
            binding.mamba_scan_bwd(u, delta, A, B, C, dout, bias, dskip, z, True, None, dlast, grads=grads,
                                   workspace=ws)

        units = w.elements
        # inputs u, delta, z, dout, B, C read once; du, ddelta, dz, dB, dC written once
        bytes_per_step = (4 * io_bytes * w.batch * w.seqlen * w.dim + 2 * io_bytes * w.batch * w.seqlen * w.dstate
                          + 3 * io_bytes * w.batch * w.seqlen * w.dim + 2 * io_bytes * w.batch * w.seqlen * w.dstate
                          + 8 * w.dim * w.dstate + 16 * w.dim + 8 * w.batch * w.dim * w.dstate)
    elif args.which == "block":
        R = W.dt_rank_for(w.dim)
        dm = w.dim // 2
        sw = W.selection_weights(w.dim, w.dstate, R, w.io, seed=w.seed)
        bw = W.block_weights(dm, w.dim, w.io, seed=w.seed)
        hidden = t(W.block_hidden(w.batch, w.seqlen, dm, w.io, seed=w.seed))
        wx, wdt, win, wout = t(sw.W_x), t(sw.W_dt), t(bw.W_in), t(bw.W_out)
        out = torch.empty_like(hidden)
        last = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device=dev)
        ws = torch.empty(max(binding.mamba_block_fwd_workspace_size(w.batch, w.seqlen, dm, w.dim, w.dstate, R,
                                                                    1 if w.io == "bf16" else 0), 1),
                         dtype=torch.uint8, device=dev)

        def step():
            binding.mamba_block_fwd(hidden, win, wx, wdt, A, wout, dt_bias=bias, Dskip=dskip, out=out,
                                    last_state=last, workspace=ws)

        units = w.elements
        M = w.batch * w.seqlen
        # matrix-core work: input projection (2 D outputs), x_proj, dt_proj, output projection
        block_mfma_flops = 2.0 * M * (2 * w.dim * dm + w.dim * (R + 2 * w.dstate) + R * w.dim + dm * w.dim)
        bytes_per_step = io_bytes * (2 * M * dm + 3 * w.dim * dm + M * w.dim) + 8 * w.dim + 4 * w.dim * w.dstate
    elif args.which in ("sel", "ssm"):
        R = W.dt_rank_for(w.dim)
        sw = W.selection_weights(w.dim, w.dstate, R, w.io, seed=w.seed)
        wx, wdt = t(sw.W_x), t(sw.W_dt)
        M = w.batch * w.seqlen
        if args.which == "sel":
            sel_out = (torch.empty_like(u), torch.empty_like(B), torch.empty_like(C))
            ws = torch.empty(max(binding.mamba_selection_fwd_workspace_size(w.batch, w.seqlen, w.dim, w.dstate, R,
                                                                            1 if w.io == "bf16" else 0), 1),
                             dtype=torch.uint8, device=dev)

            def step():
                binding.mamba_selection_fwd(u, wx, wdt, w.dstate, *sel_out, workspace=ws)

            units = M * w.dim  # output elements of delta
            bytes_per_step = io_bytes * (2 * M * w.dim + (R + 2 * w.dstate) * w.dim + w.dim * R + 2 * M * w.dstate)
            sel_flops = 2.0 * M * w.dim * (R + 2 * w.dstate) + 2.0 * M * R * w.dim
        else:
            out = torch.empty_like(u)
            last = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device=dev)
            ws = torch.empty(max(binding.mamba_ssm_fwd_workspace_size(w.batch, w.seqlen, w.dim, w.dstate, R,
                                                                      1 if w.io == "bf16" else 0), 1),
                             dtype=torch.uint8, device=dev)

            def step():
                binding.mamba_ssm_fwd(u, wx, wdt, A, z=z, dt_bias=bias, Dskip=dskip, out=out, last_state=last,
                                      workspace=ws)

            units = w.elements
            bytes_per_step = (3 * io_bytes * M * w.dim + io_bytes * ((R + 2 * w.dstate) * w.dim + w.dim * R)
                              + 8 * w.dim + 4 * w.dim * w.dstate + 4 * w.batch * w.dim * w.dstate)
    elif args.which == "complex":
        Ac = torch.from_numpy(W.a_init_complex(w.dim, w.dstate)).to(dev)
        out = torch.empty_like(u)
        last = torch.empty((w.batch, w.dim, w.dstate, 2), dtype=torch.float32, device=dev)
        ws = torch.empty(max(binding.mamba_scan_fwd_complex_workspace_size(w.batch, w.seqlen, w.dim, w.dstate,
                                                                          1 if w.io == "bf16" else 0), 1),
                         dtype=torch.uint8, device=dev)

        def step():
            binding.mamba_scan_fwd_complex(u, delta, Ac, B, C, bias, dskip, z, True, None, out=out, last_state=last,
                                           workspace=ws)

        units = w.elements
        # as the real scan, with A (D, N) and last_state (batch, D, N) complex
        bytes_per_step = (algorithmic_bytes(w.batch, w.seqlen, w.dim, w.dstate, io_bytes)
                          + 4 * w.dim * w.dstate + 4 * w.batch * w.dim * w.dstate)
    else:
        out = torch.empty_like(u)
        last = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device=dev)
        ws_bytes = binding.mamba_scan_fwd_workspace_size(w.batch, w.seqlen, w.dim, w.dstate,
                                                         1 if w.io == "bf16" else 0)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

        def step():
            binding.mamba_scan_fwd(u, delta, A, B, C, bias, dskip, z, True, None, out=out, last_state=last,
                                   workspace=ws)

        units = w.elements
        bytes_per_step = algorithmic_bytes(w.batch, w.seqlen, w.dim, w.dstate, io_bytes)

    use_graph = args.graph == "on" or (args.graph == "auto" and decode)
    if use_graph:
        eager_step = step
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            eager_step()  # warm up on a side stream before capture
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            eager_step()

        def step():
            graph.replay()

    # Clock settle: after the idle time of input generation the shader clock takes
    # a few tens of milliseconds of load to come back up (measured: the first ~40
    # steps of the Mamba-3B layer run 0.82 -> 0.57 ms).  Untimed steps run for
    # --settle-ms before the warmup, so that the timed steps see the clock a
    # continuously running job sees; their count is reported.
    settle_steps = 0
    if args.settle_ms > 0:
        t_end = time.perf_counter() + args.settle_ms / 1e3
        while time.perf_counter() < t_end and settle_steps < 10000:
            for _ in range(4):
                step()
            settle_steps += 4
            torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps + 2)]
    if args.flush:
        total_ms = 0.0
        for k in range(args.steps):
            flush_buf.fill_(float(k))
            ev[2 * k].record(stream)
            step()
            ev[2 * k + 1].record(stream)
        torch.cuda.synchronize()
        total_ms = sum(ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(args.steps))
    else:
        torch.cuda.synchronize()
        ev[0].record(stream)
        for _ in range(args.steps):
            step()
        ev[1].record(stream)
        torch.cuda.synchronize()
        total_ms = ev[0].elapsed_time(ev[1])
    ms = total_ms / args.steps
    value = units / (ms * 1e-3)
    gbps = bytes_per_step / (ms * 1e-3) / 1e9
    flops = units * FLOPS_PER_ELEMENT + (units / w.dstate) * FLOPS_PER_TOKEN_CHANNEL
    tflops = flops / (ms * 1e-3) / 1e12
    traffic = measured_traffic(args.workload, args.which)
    if args.which == "complex":
        flops = units * COMPLEX_FLOPS_PER_ELEMENT + (units / w.dstate) * FLOPS_PER_TOKEN_CHANNEL
        tflops = flops / (ms * 1e-3) / 1e12
    if args.which == "bwd":
        # per (b, l, d, n): forward recompute (9) as above plus the reverse step (~20 fp32 ops, FMA = 2)
        flops = units * (FLOPS_PER_ELEMENT + BWD_FLOPS_PER_ELEMENT) + (units / w.dstate) * 30.0
        tflops = flops / (ms * 1e-3) / 1e12
    if args.which == "block":
        peak = MFMA_BF16_PEAK_TFLOPS if w.io == "bf16" else MFMA_F32_PEAK_TFLOPS
        mt = block_mfma_flops / (ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(mt, 2), "peak": peak, "unit": "TFLOP/s", "frac": round(mt / peak, 4),
                "traffic": traffic, "scan_alu_tflops": round(tflops, 2),
                "note": "projection flops over the whole step, whose time includes the VALU-bound scan"}
    elif args.which == "sel":
        peak = MFMA_BF16_PEAK_TFLOPS if w.io == "bf16" else MFMA_F32_PEAK_TFLOPS
        roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "mfma_tflops": round(sel_flops / (ms * 1e-3) / 1e12, 2), "mfma_peak": peak,
                "note": "two GEMMs of arithmetic intensity below the MFMA/HBM ridge: HBM-bound"}
    elif decode:
        roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": bytes_per_step // L}
    else:
        roof = {"bound": "alu", "achieved": round(tflops, 2), "peak": VALU_FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / VALU_FP32_PEAK_TFLOPS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": bytes_per_step,
                "note": "fp32 VALU without packed-fp32 instructions; frac vs the packed 157.3 TFLOP/s "
                        f"figure: {tflops / VALU_FP32_PACKED_TFLOPS:.4f}"}
    rec = {
        "metric": {"fwd": FWD_METRIC,
                   "bwd": "selective-scan bwd elements(B*L*D*N)/s (all gradients, states recomputed)",
                   "sel": "selection projections: delta elements (B*L*D)/s (x_proj + dt_proj GEMMs)",
                   "ssm": "selective SSM from x: elements(B*L*D*N)/s (selection GEMMs + scan)",
                   "complex": "selective-scan fwd with complex A: elements(B*L*D*N)/s",
                   "block": "Mamba block fwd (projections + selection + scan): elements(B*L*D*N)/s"}[args.which],
        "value": value,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.io,  # I/O type of the per-token tensors; the state and the arithmetic are fp32
        "data": "synthetic",
        "config": {"workload": args.workload, "pass": args.which, "batch": w.batch, "seqlen": w.seqlen, "dim": w.dim,
                   "dstate": w.dstate, "io_dtype": w.io, "state_dtype": "f32",
                   "flush_infinity_cache": bool(args.flush), "hip_graph": bool(use_graph),
                   "clock_settle": {"ms": args.settle_ms, "untimed_steps": settle_steps},
                   "parallelism": "single-gpu"},
        "hbm_gbps": round(gbps, 1),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": bytes_per_step,
        "roofline": roof,
    }
    if not args.no_cpu_baseline and args.which in ("fwd", "bwd", "complex"):
        rec["cpu_baseline"] = cpu_baseline(inp, args.workload, args.which)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
