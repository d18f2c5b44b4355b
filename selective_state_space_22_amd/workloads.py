"""Seeded synthetic inputs for the selective scan (S6).

This module only draws random numbers and packs them; it holds none of the
scan's own arithmetic, so both the HIP path and the fp64 oracle can be fed
from it.  Shapes and distributions follow the workloads the Mamba paper's
models imply (Mamba-130M / Mamba-3B layer shapes, expand factor E = 2, state
size N = 16) and the "S4D-real" initialisation A_n = -(n+1) from the paper's
A-initialisation ablation (kb.agiseed.tech Mamba overview, section 6.5).

Distributions (all drawn in float32 from numpy PCG64):
  dt0    ~ exp(U(ln 1e-3, ln 1e-1))        per channel, delta_bias = softplus^-1(dt0)
  A      : A[d, n] = -(n + 1) unless another real initialisation is asked for
  Dskip  ~ N(0, 1)                          per channel
  u, z   ~ N(0, 1)                          (batch, L, D)
  delta  ~ U(-4, -2)                        (batch, L, D), raw (pre-softplus)
  B, C   ~ N(0, 1)                          (batch, L, N)
  reset  (million-token workload only): Bernoulli(0.01) per (batch row, token),
         shared by all channels; at those tokens delta ~ U(30, 40).
Each tensor is drawn from its own seed stream (see ``generate``).
bf16 workloads draw in float32 and round once to bf16 (round to nearest even).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

SEED_BASE = 22_000
_BLOCK = 1 << 22  # elements per independently seeded / processed block of a large tensor


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int
    batch: int
    seqlen: int
    dim: int
    dstate: int
    io: str  # "f32" or "bf16"
    reset_frac: float = 0.0
    decode_steps: int = 0  # >0: decode workload advanced one token at a time

    @property
    def seed(self) -> int:
        return SEED_BASE + self.index

    @property
    def elements(self) -> int:
        return self.batch * self.seqlen * self.dim * self.dstate


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny", 0, 1, 256, 64, 16, "f32"),
        Workload("mamba130m_layer", 1, 8, 2048, 1536, 16, "bf16"),
        Workload("mamba3b_layer", 2, 4, 4096, 5120, 16, "bf16"),
        Workload("million_tokens", 3, 1, 1 << 20, 256, 16, "f32", reset_frac=0.01),
        Workload("decode", 4, 256, 64, 5120, 16, "bf16", decode_steps=64),
    )
}


def bf16_round(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Round float32 -> bf16 with round-to-nearest-even (NaN stays NaN).

    Returns (bits as uint16, the same values widened back to float32)."""
    from concurrent.futures import ThreadPoolExecutor

    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    bits = np.empty(x.shape, dtype=np.uint16)
    widened = np.empty(x.shape, dtype=np.float32)

    def one(j):
        sl = slice(j * _BLOCK, (j + 1) * _BLOCK)
        u = x[sl].view(np.uint32)
        r = (u >> np.uint32(16)) & np.uint32(1)
        r += np.uint32(0x7FFF)
        r += u
        r >>= np.uint32(16)
        nan = np.isnan(x[sl])
        if nan.any():
            r[nan] = (u[nan] >> np.uint32(16)) | np.uint32(0x40)
        bits[sl] = r
        r <<= np.uint32(16)
        widened[sl] = r.view(np.float32)

    nblk = max(1, -(-x.size // _BLOCK))
    if nblk == 1:
        one(0)
    else:
        with ThreadPoolExecutor(min(16, nblk)) as ex:
            list(ex.map(one, range(nblk)))
    return bits, widened


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def a_init(dim: int, dstate: int, kind: str = "s4d_real", rng: np.random.Generator | None = None) -> np.ndarray:
    """Real diagonal A of shape (D, N), one of the paper's real initialisations."""
    n = np.arange(dstate, dtype=np.float32)
    if kind == "s4d_real":  # A_n = -(n+1)
        row = -(n + 1.0)
        return np.ascontiguousarray(np.broadcast_to(row, (dim, dstate)), dtype=np.float32)
    if kind == "neg_half":  # A_n = -1/2
        return np.full((dim, dstate), -0.5, dtype=np.float32)
    if kind == "exp_normal":  # A_n = -exp(N(0,1)), independent per (d, n)
        rng = rng or np.random.default_rng(SEED_BASE + 99)
        return (-np.exp(rng.standard_normal((dim, dstate), dtype=np.float32))).astype(np.float32)
    raise ValueError(kind)


def a_init_complex(dim: int, dstate: int) -> np.ndarray:
    """Complex diagonal A of shape (D, N), complex64: A_n = -1/2 + n i, the complex
    row of the A-initialisation ablation (same for every channel)."""
    n = np.arange(dstate, dtype=np.float32)
    row = (-0.5 + 1j * n).astype(np.complex64)
    return np.ascontiguousarray(np.broadcast_to(row, (dim, dstate)))


def softplus_inverse(y: np.ndarray) -> np.ndarray:
    """x such that log(1 + e^x) = y (input recipe for delta_bias), in float64."""
    y = np.asarray(y, dtype=np.float64)
    return np.log(np.expm1(y))


@dataclasses.dataclass
class ScanInputs:
    """Host copies of one scan problem.

    *_f32 arrays hold the exact values the GPU sees (bf16 values widened);
    *_bits arrays hold the bf16 bit patterns for bf16 workloads (else None)."""
    batch: int
    seqlen: int
    dim: int
    dstate: int
    io: str
    u: np.ndarray
    delta: np.ndarray
    z: np.ndarray | None
    B: np.ndarray
    C: np.ndarray
    A: np.ndarray
    delta_bias: np.ndarray | None
    Dskip: np.ndarray | None
    u_bits: np.ndarray | None = None
    delta_bits: np.ndarray | None = None
    z_bits: np.ndarray | None = None
    B_bits: np.ndarray | None = None
    C_bits: np.ndarray | None = None
    softplus: bool = True

    def io_array(self, name: str) -> np.ndarray:
        """Array in the I/O dtype (uint16 bits for bf16, float32 otherwise)."""
        if self.io == "bf16":
            return getattr(self, name + "_bits")
        return getattr(self, name)


def _fill(seq: np.random.SeedSequence, shape, kind: str, lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    """Draw a float32 tensor from its own seed stream, in fixed-size blocks with
    per-block child streams (so the values do not depend on the thread count)."""
    from concurrent.futures import ThreadPoolExecutor

    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(-1)
    nblk = max(1, -(-flat.size // _BLOCK))
    kids = seq.spawn(nblk)

    def one(j):
        g = np.random.Generator(np.random.PCG64(kids[j]))
        part = flat[j * _BLOCK:(j + 1) * _BLOCK]
        if kind == "normal":
            g.standard_normal(out=part, dtype=np.float32)
        else:  # uniform on [lo, hi)
            g.random(out=part, dtype=np.float32)
            part *= np.float32(hi - lo)
            part += np.float32(lo)

    if nblk == 1:
        one(0)
    else:
        with ThreadPoolExecutor(min(16, nblk)) as ex:
            list(ex.map(one, range(nblk)))
    return out


def generate(batch: int, seqlen: int, dim: int, dstate: int, io: str = "f32", seed: int = SEED_BASE,
             reset_frac: float = 0.0, a_kind: str = "s4d_real", with_z: bool = True,
             with_dskip: bool = True, with_bias: bool = True) -> ScanInputs:
    """Draw one scan problem with the workload distributions above.

    Every tensor has its own stream: SeedSequence(seed).spawn(8) in the order
    dt0, Dskip, u, z, delta, B, C, reset; large tensors are drawn in blocks of
    2^22 elements, each from a child stream of the tensor's stream."""
    if io not in ("f32", "bf16"):
        raise ValueError(io)
    seqs = np.random.SeedSequence(seed).spawn(8)
    dt0 = np.exp(_fill(seqs[0], (dim,), "uniform", math.log(1e-3), math.log(1e-1)).astype(np.float64))
    dskip = _fill(seqs[1], (dim,), "normal")
    u = _fill(seqs[2], (batch, seqlen, dim), "normal")
    z = _fill(seqs[3], (batch, seqlen, dim), "normal") if with_z else None
    delta = _fill(seqs[4], (batch, seqlen, dim), "uniform", -4.0, -2.0)
    Bm = _fill(seqs[5], (batch, seqlen, dstate), "normal")
    Cm = _fill(seqs[6], (batch, seqlen, dstate), "normal")
    if reset_frac > 0:
        g = np.random.Generator(np.random.PCG64(seqs[7]))
        mask = g.random((batch, seqlen)) < reset_frac
        nres = int(mask.sum())
        delta[mask] = g.uniform(30.0, 40.0, size=(nres, dim)).astype(np.float32)
    A = a_init(dim, dstate, a_kind, np.random.Generator(np.random.PCG64(seed + 1_000_000)))
    bias = softplus_inverse(dt0).astype(np.float32)
    inp = ScanInputs(batch, seqlen, dim, dstate, io, u, delta, z, Bm, Cm, A,
                     bias if with_bias else None, dskip if with_dskip else None)
    if io == "bf16":
        for name in ("u", "delta", "z", "B", "C"):
            arr = getattr(inp, name)
            if arr is None:
                continue
            bits, widened = bf16_round(arr)
            setattr(inp, name + "_bits", bits.reshape(arr.shape))
            setattr(inp, name, widened.reshape(arr.shape))
    return inp


@dataclasses.dataclass
class GradInputs:
    """Upstream gradients for the backward: dout (batch, L, D) in the I/O type, dlast (batch, D, N) float32."""
    dout: np.ndarray
    dlast: np.ndarray | None


def grad_inputs(batch: int, seqlen: int, dim: int, dstate: int, io: str = "f32", seed: int = SEED_BASE,
                with_dlast: bool = True) -> GradInputs:
    """Seeded upstream gradients, dout ~ N(0, 1) and dlast ~ N(0, 1), from their own
    streams (SeedSequence(seed + 500000).spawn(2)); bf16 dout is rounded once (RNE)."""
    seqs = np.random.SeedSequence(seed + 500_000).spawn(2)
    dout = _fill(seqs[0], (batch, seqlen, dim), "normal")
    if io == "bf16":
        _, widened = bf16_round(dout)
        dout = widened.reshape(dout.shape)
    dlast = _fill(seqs[1], (batch, dim, dstate), "normal") if with_dlast else None
    return GradInputs(dout, dlast)


def dt_rank_for(dim: int) -> int:
    """Size of the dt projection for a layer of D = dim channels: d_model / 16 with
    d_model = D / 2 (expand factor 2), at least 1.  The page's dt-projection
    ablation has its default model (the 371.5 M-parameter row shared with the
    state-size table) at size 64, i.e. d_model 1024 / 16."""
    return max(1, -(-(dim // 2) // 16))


@dataclasses.dataclass
class SelectionWeights:
    W_x: np.ndarray   # (R + 2N, D)
    W_dt: np.ndarray  # (D, R)


def selection_weights(dim: int, dstate: int, dt_rank: int, io: str = "f32", seed: int = SEED_BASE) -> SelectionWeights:
    """Random-init projection weights in the usual linear-layer ranges:
    W_x ~ U(-1/sqrt(D), 1/sqrt(D)), W_dt ~ U(-1/sqrt(R), 1/sqrt(R)) (own streams of
    SeedSequence(seed + 700000)); bf16 rounds once (RNE)."""
    seqs = np.random.SeedSequence(seed + 700_000).spawn(2)
    bx = 1.0 / math.sqrt(dim)
    bd = 1.0 / math.sqrt(dt_rank)
    W_x = _fill(seqs[0], (dt_rank + 2 * dstate, dim), "uniform", -bx, bx)
    W_dt = _fill(seqs[1], (dim, dt_rank), "uniform", -bd, bd)
    if io == "bf16":
        W_x = bf16_round(W_x)[1].reshape(W_x.shape)
        W_dt = bf16_round(W_dt)[1].reshape(W_dt.shape)
    return SelectionWeights(W_x, W_dt)


@dataclasses.dataclass
class BlockWeights:
    W_in: np.ndarray   # (2 D, d_model)
    W_out: np.ndarray  # (d_model, D)


def block_weights(d_model: int, dim: int, io: str = "f32", seed: int = SEED_BASE) -> BlockWeights:
    """Random-init block projections in the usual linear-layer ranges:
    W_in ~ U(-1/sqrt(d_model), 1/sqrt(d_model)), W_out ~ U(-1/sqrt(D), 1/sqrt(D))
    (own streams of SeedSequence(seed + 800000)); bf16 rounds once (RNE)."""
    seqs = np.random.SeedSequence(seed + 800_000).spawn(2)
    bi = 1.0 / math.sqrt(d_model)
    bo = 1.0 / math.sqrt(dim)
    W_in = _fill(seqs[0], (2 * dim, d_model), "uniform", -bi, bi)
    W_out = _fill(seqs[1], (d_model, dim), "uniform", -bo, bo)
    if io == "bf16":
        W_in = bf16_round(W_in)[1].reshape(W_in.shape)
        W_out = bf16_round(W_out)[1].reshape(W_out.shape)
    return BlockWeights(W_in, W_out)


def block_hidden(batch: int, seqlen: int, d_model: int, io: str = "f32", seed: int = SEED_BASE) -> np.ndarray:
    """Block input (batch, L, d_model) ~ N(0, 1) from its own stream (SeedSequence(seed + 900000)),
    bf16-rounded once for bf16 I/O."""
    h = _fill(np.random.SeedSequence(seed + 900_000), (batch, seqlen, d_model), "normal")
    if io == "bf16":
        h = bf16_round(h)[1].reshape(h.shape)
    return h


def generate_workload(name: str) -> ScanInputs:
    """The seeded inputs of a named workload (decode: the 64 tokens as one (B, 64, D) block)."""
    w = WORKLOADS[name]
    return generate(w.batch, w.seqlen, w.dim, w.dstate, w.io, seed=w.seed, reset_frac=w.reset_frac)


def channel_subset(inp: ScanInputs, batches, channels) -> ScanInputs:
    """Inputs restricted to some batch rows and channels (channels are independent SSMs)."""
    b = np.asarray(batches)
    d = np.asarray(channels)

    def sel3(x):
        return None if x is None else np.ascontiguousarray(x[b][:, :, d])

    def sel_bl(x):
        return None if x is None else np.ascontiguousarray(x[b])

    def sel1(x):
        return None if x is None else np.ascontiguousarray(x[d])

    out = ScanInputs(len(b), inp.seqlen, len(d), inp.dstate, inp.io, sel3(inp.u), sel3(inp.delta), sel3(inp.z),
                     sel_bl(inp.B), sel_bl(inp.C), np.ascontiguousarray(inp.A[d]), sel1(inp.delta_bias),
                     sel1(inp.Dskip), softplus=inp.softplus)
    return out
