"""The error bound of the scan's input weight in its bracket form, checked in an fp32
emulation on the host (no GPU).

For dt >= 0 the kernels compute beta = dt (e^x - 1)/x, x = dt A_n, as the smaller of
two upper bounds: q = (Abar - 1)/A_n plus a margin of one ulp of 1/A_n (two when
A_n > 0), formed as one FMA Abar * ka + kc, and U = (dt / 2)(1 + Abar), the trapezoid
bound of the integral over s in [0, 1] of e^{s x}.  This test replays that arithmetic
with every fp32 rounding made explicit (an FMA rounds once) and Abar anywhere within
one ulp of 2^(x log2 e), and checks the relative error against the exact
expm1(x)/A_n: below 1.5e-5 for A_n < 0 and 2.5e-5 for A_n > 0, the bounds the design
states, and exact for A_n = 0 and for dt = 0."""
import numpy as np

F32 = np.float32
FLT_MAX = np.finfo(np.float32).max


def _fma(a, b, c):
    # the product of two fp32 values is exact in fp64; the sum rounds to fp64 and then
    # once more to fp32, which can differ from one rounding only at exact fp64 ties
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def _ka_kc(a):
    a = F32(a)
    ka = F32(FLT_MAX) if a == 0 else F32(np.clip(np.float64(1.0) / np.float64(a), -FLT_MAX, FLT_MAX))
    v = F32(-ka)
    bits = np.array([v], np.float32).view(np.uint32)[0]
    if v > 0:
        kc = np.array([bits + 1], np.uint32).view(np.float32)[0]
    elif v < -1e-37:
        kc = np.array([bits - 2], np.uint32).view(np.float32)[0]
    else:
        kc = v
    return ka, kc


def _abar_variants(x2):
    """2^x2 rounded to fp32, and its neighbours that stay within one ulp of the exact value."""
    exact = np.exp2(x2.astype(np.float64))
    r = exact.astype(np.float32)
    out = [r]
    for d in (np.inf, 0.0):
        n = np.nextafter(r, np.float32(d))
        ulp = np.where(exact < 1.0, np.minimum(np.spacing(r).astype(np.float64), 2.0 ** -24),
                       np.spacing(r).astype(np.float64))
        ok = np.abs(n.astype(np.float64) - exact) <= ulp
        out.append(np.where(ok, n, r).astype(np.float32))
    return out


def _max_rel_error(a, dt):
    ka, kc = _ka_kc(a)
    a2 = F32(F32(a) * F32(1.4426950408889634))
    x2 = (dt * a2).astype(np.float32)
    dth = (F32(0.5) * dt).astype(np.float32)
    exact = np.where(dt == 0, 0.0, np.expm1(dt.astype(np.float64) * np.float64(F32(a))) / np.float64(F32(a))) \
        if a != 0 else dt.astype(np.float64)
    worst = 0.0
    for ab in _abar_variants(x2):
        q = _fma(ab, np.full_like(ab, ka), np.full_like(ab, kc))
        u = _fma(ab, dth, dth)
        beta = np.minimum(q, u).astype(np.float64)
        nz = exact != 0
        rel = np.abs(beta[nz] - exact[nz]) / np.abs(exact[nz])
        worst = max(worst, float(rel.max()))
    return worst


def test_bracket_form_error_bound_negative_a():
    rng = np.random.default_rng(7)
    dt = (10.0 ** rng.uniform(-7, 1.5, 200_000)).astype(np.float32)
    for a in (-1.0, -2.0, -16.0, -0.5, -3.7, -1e-2, -1e-4, -123.4, -1e5):
        assert _max_rel_error(a, dt) < 1.5e-5, a


def test_bracket_form_error_bound_positive_a():
    rng = np.random.default_rng(8)
    for a in (0.3, 2.0, 16.0):
        dt = (10.0 ** rng.uniform(-7, np.log10(40.0 / a), 100_000)).astype(np.float32)
        assert _max_rel_error(a, dt) < 2.5e-5, a


def test_bracket_form_special_cases():
    dt = np.array([0.0, 1e-7, 0.3, 5.0], np.float32)
    # A_n = 0: beta = dt exactly (the quotient is huge, the trapezoid bound is dt)
    ka, kc = _ka_kc(0.0)
    ab = np.ones_like(dt)
    q = _fma(ab, np.full_like(ab, ka), np.full_like(ab, kc))
    u = _fma(ab, F32(0.5) * dt, F32(0.5) * dt)
    assert np.array_equal(np.minimum(q, u), dt)
    # dt = 0: Abar = 1, beta = 0 exactly, so the state is held
    for a in (-1.0, -16.0, 0.5):
        ka, kc = _ka_kc(a)
        q = _fma(np.ones(1, np.float32), np.full(1, ka, np.float32), np.full(1, kc, np.float32))
        u = _fma(np.ones(1, np.float32), np.zeros(1, np.float32), np.zeros(1, np.float32))
        assert np.minimum(q, u)[0] == 0.0


def test_the_margin_is_needed():
    """Without the margin the quotient's rounding error is not bounded near x = 0: a
    plain min((Abar - 1)/A_n, U) would be off by far more than the fp32 bound."""
    rng = np.random.default_rng(9)
    dt = (10.0 ** rng.uniform(-7, -3, 50_000)).astype(np.float32)
    a = -1.0
    ka = F32(-1.0)
    x2 = (dt * F32(F32(a) * F32(1.4426950408889634))).astype(np.float32)
    worst = 0.0
    exact = np.expm1(dt.astype(np.float64) * a) / a
    for ab in _abar_variants(x2):
        q = _fma(ab, np.full_like(ab, ka), np.full_like(ab, F32(-ka)))
        u = _fma(ab, F32(0.5) * dt, F32(0.5) * dt)
        worst = max(worst, float((np.abs(np.minimum(q, u) - exact) / exact).max()))
    assert worst > 1e-3
