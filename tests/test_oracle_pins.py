"""The fp64 oracle against what the page's mathematics fixes (CPU only)."""
import json
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
import pins

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def c_scan(u, delta, A, B, C, delta_bias=None, Dskip=None, z=None, softplus=True, h0=None):
    return oracle.scan(u, delta, A, B, C, delta_bias, Dskip, z, softplus, h0, nthreads=2)


def np_scan(u, delta, A, B, C, delta_bias=None, Dskip=None, z=None, softplus=True, h0=None):
    return oracle.scan_numpy(u, delta, A, B, C, delta_bias, Dskip, z, softplus, h0)


@pytest.mark.parametrize("impl", [c_scan, np_scan], ids=["c", "numpy"])
@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=[p.__name__ for p in pins.ALL_PINS])
def test_pin(impl, pin):
    ok, detail = pin(impl)
    assert ok, detail


def test_brute_force_without_softplus_and_single_token():
    for L in (1, 2, 5):
        ok, detail = pins.pin_brute_force(c_scan, seed=20 + L, softplus=False, L=L)
        assert ok, detail


@pytest.mark.parametrize("seed", range(4))
def test_c_matches_numpy_twin(seed):
    rng = np.random.default_rng(100 + seed)
    batch, L, D, N = 2, 33, 7, [1, 3, 8, 16][seed]
    p = pins.small_problem(rng, batch=batch, L=L, D=D, N=N, gate=seed % 2 == 0, skip=seed < 3, bias=seed != 1)
    h0 = rng.standard_normal((batch, D, N)) if seed == 2 else None
    o1, h1 = c_scan(**p, softplus=seed != 3, h0=h0)
    o2, h2 = np_scan(**p, softplus=seed != 3, h0=h0)
    assert pins.rel(o1, o2) < 1e-13
    assert pins.rel(h1, h2) < 1e-13


def test_decode_steps_equal_scan():
    """P-j: L single-token steps from a zero state reproduce the full-sequence scan."""
    rng = np.random.default_rng(30)
    p = pins.small_problem(rng, batch=3, L=11, D=4, N=5)
    out, last = c_scan(**p)
    st = np.zeros((3, 4, 5))
    for t in range(11):
        o, st = oracle.step(st, p["u"][:, t], p["delta"][:, t], p["A"], p["B"][:, t], p["C"][:, t],
                            p["delta_bias"], p["Dskip"], p["z"][:, t], True, nthreads=2)
        assert np.array_equal(o, out[:, t])
    assert np.array_equal(st, last)


def test_zero_length_and_argument_errors():
    rng = np.random.default_rng(31)
    p = pins.small_problem(rng, batch=1, L=0, D=2, N=3)
    out, last = c_scan(**p)
    assert out.shape == (1, 0, 2)
    assert np.array_equal(last, np.zeros((1, 2, 3)))
    h0 = rng.standard_normal((1, 2, 3))
    _, last = c_scan(**p, h0=h0)
    assert np.array_equal(last, h0)


def test_negative_dt_and_positive_a_are_finite():
    """Silent point: dt < 0 (no softplus) or A >= 0 are still the same formula, with no NaN."""
    rng = np.random.default_rng(32)
    p = pins.small_problem(rng, batch=1, L=8, D=2, N=3)
    p["A"] = np.abs(p["A"])
    out, last = c_scan(**p, softplus=False)
    assert np.isfinite(out).all() and np.isfinite(last).all()
    o2, h2 = np_scan(**p, softplus=False)
    assert pins.rel(out, o2) < 1e-13


def _dec(s):
    getcontext().prec = 40
    return Decimal(s)


def test_golden_zoh_halving():
    g = json.load(open(os.path.join(GOLDEN, "zoh_halving.json")))
    getcontext().prec = 40
    ln2 = Decimal(2).ln()
    closed = [1 / (2 * ln2), 1 / (4 * ln2), 1 / (8 * ln2), 9 / (16 * ln2)]
    for c, s in zip(closed, g["expected_decimal"]["out"]):
        assert abs(c - _dec(s)) < Decimal("1e-35")
    A = np.array([[-float(ln2)]])
    u = np.array(g["inputs"]["u"])[None, :, None]
    delta = np.array(g["inputs"]["delta"])[None, :, None]
    B = np.array(g["inputs"]["B"])[None, :, None]
    C = np.array(g["inputs"]["C"])[None, :, None]
    out, last = c_scan(u, delta, A, B, C, softplus=False)
    want = np.array([float(_dec(s)) for s in g["expected_decimal"]["out"]])
    assert pins.rel(out[0, :, 0], want) < 1e-14
    assert abs(last[0, 0, 0] / float(_dec(g["expected_decimal"]["last_state"][0])) - 1) < 1e-14


def test_golden_softplus_gate_two_states():
    g = json.load(open(os.path.join(GOLDEN, "softplus_gate_two_states.json")))
    getcontext().prec = 40
    ln2, ln3 = Decimal(2).ln(), Decimal(3).ln()
    k0, k1 = 1 / (2 * ln2), 3 / (4 * ln2)
    h0 = [k0 * (2 - Decimal(2) ** -t) for t in range(3)]
    h1 = [k1 * (4 - Decimal(4) ** -t) / 3 for t in range(3)]
    outs = [(h0[t] - h1[t] + 2) * ln3 * Decimal("0.75") for t in range(3)]
    for c, s in zip(outs, g["expected_decimal"]["out"]):
        assert abs(c - _dec(s)) < Decimal("1e-35")
    for c, s in zip([h0[2], h1[2]], g["expected_decimal"]["last_state"]):
        assert abs(c - _dec(s)) < Decimal("1e-35")
    e = Decimal(1).exp()
    A = np.array([[-float(ln2), -2 * float(ln2)]])
    bias = np.array([float((e - 1).ln() - Decimal("0.25"))])
    u = np.ones((1, 3, 1))
    delta = np.full((1, 3, 1), 0.25)
    B = np.tile(np.array([1.0, 2.0]), (1, 3, 1))
    C = np.tile(np.array([1.0, -1.0]), (1, 3, 1))
    z = np.full((1, 3, 1), float(ln3))
    out, last = c_scan(u, delta, A, B, C, bias, np.array([2.0]), z, True)
    want = np.array([float(_dec(s)) for s in g["expected_decimal"]["out"]])
    assert pins.rel(out[0, :, 0], want) < 1e-14
    wl = np.array([float(_dec(s)) for s in g["expected_decimal"]["last_state"]])
    assert pins.rel(last[0, 0], wl) < 1e-14
