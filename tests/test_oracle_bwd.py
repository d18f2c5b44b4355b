"""The fp64 backward oracle against central finite differences of the forward oracle.

The backward pass is not printed on the page; it is the derivative of the
forward definition ("Mamba 状态空间模型原理与 Transformer 对比", kb.agiseed.tech,
section 2.1 eq. (2), (3a), (3b), the section 3.2 softplus front end and the
Figure 3 SiLU gate).  The pin is therefore the forward oracle itself,
differentiated numerically: for every input element e,
    dLoss/de ~= (Loss(e + s) - Loss(e - s)) / 2s,
    Loss = sum(dout * out) + sum(dlast * last_state),
which shares no arithmetic with the analytic backward.  Central differences in
fp64 with s ~ 1e-6 are accurate to ~1e-9 relative here, far below any
plausible mistake (a dropped term, a wrong sign or a shifted token index moves
a gradient by O(1)).
"""
import numpy as np
import pytest

import oracle
import pins

FIELDS = ("u", "delta", "A", "B", "C", "delta_bias", "Dskip", "z", "h0")
GRAD = {"u": "du", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "delta_bias": "dbias",
        "Dskip": "dDskip", "z": "dz", "h0": "dh0"}


def _loss(p, softplus, dout, dlast):
    out, last = oracle.scan(p["u"], p["delta"], p["A"], p["B"], p["C"], p["delta_bias"], p["Dskip"], p["z"],
                            softplus, p["h0"], nthreads=1)
    val = float(np.sum(dout * out))
    if dlast is not None:
        val += float(np.sum(dlast * last))
    return val


def _fd(p, name, softplus, dout, dlast):
    x = p[name]
    g = np.empty_like(x)
    flat = x.reshape(-1)
    gf = g.reshape(-1)
    for k in range(flat.size):
        orig = flat[k]
        s = 1e-6 * max(1.0, abs(orig))
        flat[k] = orig + s
        lp = _loss(p, softplus, dout, dlast)
        flat[k] = orig - s
        lm = _loss(p, softplus, dout, dlast)
        flat[k] = orig
        gf[k] = (lp - lm) / (2 * s)
    return g


def _problem(seed, batch=2, L=6, D=3, N=4, gate=True, skip=True, bias=True, h0=True, dlast=True, **kw):
    rng = np.random.default_rng(seed)
    p = pins.small_problem(rng, batch=batch, L=L, D=D, N=N, gate=gate, skip=skip, bias=bias, **kw)
    p["h0"] = rng.standard_normal((batch, D, N)) if h0 else None
    dout = rng.standard_normal((batch, L, D))
    dl = rng.standard_normal((batch, D, N)) if dlast else None
    return p, dout, dl


def _check(p, dout, dl, softplus, tol=2e-7):
    g = oracle.scan_bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], dout, p["delta_bias"], p["Dskip"], p["z"],
                        softplus, p["h0"], dl, nthreads=2)
    for name in FIELDS:
        if p[name] is None:
            assert GRAD[name] not in g
            continue
        fd = _fd(p, name, softplus, dout, dl)
        an = g[GRAD[name]]
        assert an.shape == fd.shape, name
        err = np.abs(an - fd).max() / (np.abs(fd).max() + 1e-30)
        assert err < tol, f"{GRAD[name]}: relative error {err:.3e} against finite differences"


@pytest.mark.parametrize("softplus", [True, False], ids=["softplus", "raw_dt"])
def test_every_gradient_matches_finite_differences(softplus):
    p, dout, dl = _problem(7)
    if not softplus:  # keep dt positive without the softplus: raw dt in (0.05, 1.2)
        p["delta"] = np.random.default_rng(8).uniform(0.05, 1.2, p["delta"].shape)
        p["delta_bias"] = np.random.default_rng(9).uniform(-0.02, 0.02, p["delta_bias"].shape)
    _check(p, dout, dl, softplus)


@pytest.mark.parametrize("variant", ["no_gate", "no_skip_no_bias", "no_h0_no_dlast", "one_state", "one_token"])
def test_optional_terms(variant):
    kw = {}
    if variant == "no_gate":
        kw = dict(gate=False)
    elif variant == "no_skip_no_bias":
        kw = dict(skip=False, bias=False)
    elif variant == "no_h0_no_dlast":
        kw = dict(h0=False, dlast=False)
    elif variant == "one_state":
        kw = dict(N=1)
    elif variant == "one_token":
        kw = dict(L=1)
    p, dout, dl = _problem(11, **kw)
    _check(p, dout, dl, True)


def test_small_dt_series_branch():
    """|dt*A| below the series threshold of psi and of (e^x - 1)/x (and A_n = 0)."""
    p, dout, dl = _problem(13, a_lo=0.01, a_hi=0.5)
    rng = np.random.default_rng(14)
    p["delta"] = rng.uniform(1e-5, 1e-3, p["delta"].shape)
    p["delta_bias"] = np.zeros_like(p["delta_bias"])
    p["A"][0, 0] = 0.0
    g = oracle.scan_bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], dout, p["delta_bias"], p["Dskip"], p["z"],
                        False, p["h0"], dl, nthreads=1)
    for name in ("A", "delta", "u", "B"):
        fd = _fd(p, name, False, dout, dl)
        an = g[GRAD[name]]
        err = np.abs(an - fd).max() / (np.abs(fd).max() + 1e-30)
        assert err < 1e-6, f"{GRAD[name]}: {err:.3e}"


def test_empty_sequence_passes_dlast_to_h0():
    rng = np.random.default_rng(3)
    batch, D, N = 2, 3, 4
    A = -rng.uniform(0.5, 2.0, (D, N))
    z0 = np.zeros((batch, 0, D))
    BC0 = np.zeros((batch, 0, N))
    dl = rng.standard_normal((batch, D, N))
    g = oracle.scan_bwd(z0, z0, A, BC0, BC0, z0, np.zeros(D), np.ones(D), z0, True,
                        rng.standard_normal((batch, D, N)), dl)
    assert np.array_equal(g["dh0"], dl)
    assert not g["dA"].any() and not g["dbias"].any() and not g["dDskip"].any()
    assert g["du"].shape == (batch, 0, D) and g["dB"].shape == (batch, 0, N)


def test_thread_count_does_not_change_result_beyond_rounding():
    p, dout, dl = _problem(17, batch=3, L=20, D=9, N=8)
    a = oracle.scan_bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], dout, p["delta_bias"], p["Dskip"], p["z"], True,
                        p["h0"], dl, nthreads=1)
    b = oracle.scan_bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], dout, p["delta_bias"], p["Dskip"], p["z"], True,
                        p["h0"], dl, nthreads=4)
    for k in a:
        assert pins.rel(a[k], b[k]) < 1e-13, k
