"""The complex-A oracle (the -1/2 + ni initialisation of the page's A ablation)
against facts that do not come from it: reduction to the pinned real oracle,
the matrix-exponential brute force, conjugate symmetry of a real readout, the
closed form for constant input, and pure rotation for imaginary A."""
import numpy as np
import pytest
import scipy.linalg

import oracle
import pins

# a complex value compared as real would drop its imaginary part silently
pytestmark = pytest.mark.filterwarnings("error::numpy.exceptions.ComplexWarning")


def _problem(rng, batch=2, L=9, D=3, N=4):
    p = pins.small_problem(rng, batch=batch, L=L, D=D, N=N)
    p["A"] = -rng.uniform(0.3, 2.0, (D, N)) + 1j * rng.uniform(-3.0, 3.0, (D, N))
    return p


def crel(a, b):
    """max |a - b| / max |b| over complex arrays (both parts compared)."""
    a = np.asarray(a, np.complex128)
    b = np.asarray(b, np.complex128)
    return float(np.abs(a - b).max(initial=0.0) / max(np.abs(b).max(initial=0.0), 1e-300))


def cscan(p, h0=None, softplus=True):
    return oracle.scan_complex(p["u"], p["delta"], p["A"], p["B"], p["C"], p["delta_bias"], p["Dskip"], p["z"],
                               softplus, h0, nthreads=2)


def test_zero_imaginary_part_is_the_real_scan():
    rng = np.random.default_rng(1)
    p = pins.small_problem(rng, batch=2, L=40, D=5, N=6)
    out_r, last_r = oracle.scan(**p, nthreads=2)
    pc = dict(p)
    pc["A"] = p["A"] + 0j
    out_c, last_c = cscan(pc)
    assert pins.rel(out_c, out_r) < 1e-13
    assert pins.rel(last_c.real, last_r) < 1e-13 and not last_c.imag.any()


def test_brute_force_with_matrix_exponential():
    """eq. (2) as matrices on the complex diagonal: Abar = expm(dt A), Bbar = (dt A)^-1 (Abar - I) dt B."""
    rng = np.random.default_rng(2)
    p = _problem(rng, batch=1, L=6, D=2, N=3)
    p["z"] = None
    p["Dskip"] = None
    out, last = cscan(p)
    dt = pins.softplus64(p["delta"] + p["delta_bias"][None, None, :])
    for d in range(2):
        h = np.zeros(3, complex)
        for t in range(6):
            M = dt[0, t, d] * np.diag(p["A"][d])
            Abar = scipy.linalg.expm(M)
            Bbar = np.linalg.solve(M, (Abar - np.eye(3)) @ (dt[0, t, d] * p["B"][0, t]))
            h = Abar @ h + Bbar * p["u"][0, t, d]
            assert abs(out[0, t, d] - (p["C"][0, t] @ h).real) <= 1e-12 * max(1.0, abs(out[0, t, d]))
        assert np.allclose(last[0, d], h, rtol=1e-12, atol=1e-14)


def test_conjugate_a_gives_the_same_real_output():
    """x, B, C real: conj(A) gives conj(h), whose real part (and so y) is the same."""
    rng = np.random.default_rng(3)
    p = _problem(rng, L=30)
    h0 = rng.standard_normal((2, 3, 4)) + 1j * rng.standard_normal((2, 3, 4))
    o1, l1 = cscan(p, h0)
    q = dict(p)
    q["A"] = np.conj(p["A"])
    o2, l2 = cscan(q, np.conj(h0))
    assert pins.rel(o1, o2) < 1e-14
    assert crel(l1, np.conj(l2)) < 1e-14


def test_constant_input_closed_form():
    """x = 1, constant dt and B: h_t = -(B/A)(1 - e^{(t+1) dt A}) (complex), y_t = Re(C . h_t)."""
    rng = np.random.default_rng(4)
    L, D, N = 50, 2, 3
    A = -rng.uniform(0.2, 1.0, (D, N)) + 1j * rng.uniform(-2, 2, (D, N))
    dt = 0.3
    Bv = rng.standard_normal(N)
    Cv = rng.standard_normal(N)
    u = np.ones((1, L, D))
    delta = np.full((1, L, D), dt)
    out, last = oracle.scan_complex(u, delta, A, np.tile(Bv, (1, L, 1)), np.tile(Cv, (1, L, 1)), softplus=False)
    t = np.arange(L)[:, None, None]
    h = -(Bv / A)[None] * (1.0 - np.exp((t + 1) * dt * A[None]))
    assert pins.rel(out[0], np.einsum("tdn,n->td", h, Cv).real) < 1e-12
    assert crel(last[0], h[-1]) < 1e-12


def test_imaginary_a_rotates_the_state():
    """Re A = 0: |Abar| = 1; with x = 0 the initial state turns by dt*Im(A) per token."""
    L, D, N = 20, 1, 2
    A = 1j * np.array([[0.7, -1.9]])
    h0 = np.array([[[1.0 + 0.5j, -0.25 + 2.0j]]])
    dt = 0.4
    out, last = oracle.scan_complex(np.zeros((1, L, D)), np.full((1, L, D), dt), A, np.ones((1, L, N)),
                                    np.ones((1, L, N)), softplus=False, h0=h0)
    t = np.arange(1, L + 1)[:, None]
    h = h0[0, 0][None] * np.exp(dt * t * A[0][None])  # A is already imaginary
    assert np.allclose(out[0, :, 0], h.sum(1).real, rtol=1e-13, atol=1e-13)
    assert np.allclose(np.abs(last[0, 0]), np.abs(h0[0, 0]), rtol=1e-13)


def test_small_dt_a_series_matches_the_quotient():
    """phi1 of a tiny complex argument: the series and the direct quotient agree where both are accurate."""
    rng = np.random.default_rng(5)
    p = _problem(rng, L=12)
    p["delta"] = np.full(p["delta"].shape, 1e-3)
    p["delta_bias"] = None
    o1, _ = cscan(p, softplus=False)
    # same problem with dt slightly above the series threshold in |dt A|: continuity of the result
    q = dict(p)
    q["delta"] = p["delta"] * (1 + 1e-9)
    o2, _ = cscan(q, softplus=False)
    assert pins.rel(o1, o2) < 1e-7
