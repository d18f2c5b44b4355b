"""Pins of the selective-scan oracle: facts fixed by the mathematics, not by the oracle.

Every pin takes a scan callable with the oracle's signature
    fn(u, delta, A, B, C, delta_bias=None, Dskip=None, z=None, softplus=True, h0=None)
        -> (out (batch, L, D), last_state (batch, D, N))
and returns (ok, detail).  The same pins run against the C oracle, its numpy
twin, and deliberately broken copies (tests/test_pin_power.py) to show that a
plausible mistake fails at least one of them.

Sources ("Mamba 状态空间模型原理与 Transformer 对比", kb.agiseed.tech):
  eq. (1a)        continuous SSM h' = A h + B x (equilibrium -B/A for constant input)
  eq. (2)         zero-order hold, written as matrices: Abar = expm(dt A),
                  Bbar = (dt A)^-1 (expm(dt A) - I) dt B
  eq. (3a)/(3b)   recurrence and readout from the updated state
  eq. (4a)/(4b)   convolution form when (dt, B, C) do not vary in time
  section 3.3     dt -> 0 ignores the token (state held); a large dt resets
  Figure 1        channels are independent SSMs
"""
from __future__ import annotations

import numpy as np
import scipy.linalg

# ---------------------------------------------------------------- helpers


def silu64(z):
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(-z))


def softplus64(v):
    return np.logaddexp(0.0, np.asarray(v, np.float64))


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = max(np.abs(b).max(initial=0.0), 1e-300)
    return float(np.abs(a - b).max(initial=0.0) / den)


def small_problem(rng, batch=2, L=9, D=3, N=4, a_lo=0.3, a_hi=3.0, gate=True, skip=True, bias=True):
    """A small random problem; dt stays in (0.05, 1.5) after softplus."""
    u = rng.standard_normal((batch, L, D))
    delta = rng.uniform(-2.5, 0.5, (batch, L, D))
    A = -rng.uniform(a_lo, a_hi, (D, N))
    B = rng.standard_normal((batch, L, N))
    C = rng.standard_normal((batch, L, N))
    db = rng.uniform(-0.5, 0.5, D) if bias else None
    Ds = rng.standard_normal(D) if skip else None
    z = rng.standard_normal((batch, L, D)) if gate else None
    return dict(u=u, delta=delta, A=A, B=B, C=C, delta_bias=db, Dskip=Ds, z=z)


def _dt(p, softplus):
    dt = np.asarray(p["delta"], np.float64)
    if p.get("delta_bias") is not None:
        dt = dt + p["delta_bias"][None, None, :]
    return softplus64(dt) if softplus else dt


def _finish(y, p, b, t, d):
    x = p["u"][b, t, d]
    if p.get("Dskip") is not None:
        y = y + p["Dskip"][d] * x
    if p.get("z") is not None:
        y = y * silu64(p["z"][b, t, d])
    return y


def _zoh_matrices(dt, a_row):
    """eq. (2) with matrices: Abar = expm(dt A), Bbar_factor = (dt A)^-1 (Abar - I) dt  (applied to B later)."""
    N = a_row.shape[0]
    dA = dt * np.diag(a_row)
    Abar = scipy.linalg.expm(dA)
    Bfac = np.linalg.solve(dA, Abar - np.eye(N)) * dt
    return Abar, Bfac


# ---------------------------------------------------------------- pins


def pin_brute_force(fn, seed=1, softplus=True, L=7):
    """P-a: y_t = sum_{s<=t} C_t (prod_{r=s+1..t} Abar_r) Bbar_s x_s, Abar/Bbar from matrix expm."""
    rng = np.random.default_rng(seed)
    p = small_problem(rng, batch=2, L=L, D=3, N=4)
    out, last = fn(**p, softplus=softplus)
    dt = _dt(p, softplus)
    batch, L, D = p["u"].shape
    N = p["A"].shape[1]
    ref = np.zeros((batch, L, D))
    ref_h = np.zeros((batch, D, N))
    for b in range(batch):
        for d in range(D):
            mats = [_zoh_matrices(dt[b, t, d], p["A"][d]) for t in range(L)]
            for t in range(L):
                acc = np.zeros(N)
                for s in range(t + 1):
                    prod = np.eye(N)
                    for r in range(s + 1, t + 1):
                        prod = mats[r][0] @ prod
                    acc += prod @ (mats[s][1] @ p["B"][b, s]) * p["u"][b, s, d]
                ref[b, t, d] = _finish(p["C"][b, t] @ acc, p, b, t, d)
                if t == L - 1:
                    ref_h[b, d] = acc
    e1, e2 = rel(out, ref), rel(last, ref_h)
    return (e1 < 1e-11 and e2 < 1e-11), f"brute force: out {e1:.2e} last {e2:.2e}"


def pin_convolution(fn, seed=2, L=48):
    """P-b: time-invariant (dt, B, C) => y = x * Kbar, Kbar_k = C Abar^k Bbar (eq. 4a/4b)."""
    rng = np.random.default_rng(seed)
    batch, D, N = 2, 3, 4
    u = rng.standard_normal((batch, L, D))
    A = -rng.uniform(0.2, 2.0, (D, N))
    raw = rng.uniform(-2.0, 0.0, D)
    delta = np.broadcast_to(raw, (batch, L, D)).copy()
    Bv = rng.standard_normal((batch, N))
    Cv = rng.standard_normal((batch, N))
    B = np.repeat(Bv[:, None, :], L, axis=1)
    C = np.repeat(Cv[:, None, :], L, axis=1)
    Ds = rng.standard_normal(D)
    z = rng.standard_normal((batch, L, D))
    out, _ = fn(u, delta, A, B, C, None, Ds, z, True, None)
    ref = np.zeros((batch, L, D))
    for b in range(batch):
        for d in range(D):
            dt = softplus64(raw[d])
            Abar, Bfac = _zoh_matrices(dt, A[d])
            Bbar = Bfac @ Bv[b]
            K = np.array([Cv[b] @ np.linalg.matrix_power(Abar, k) @ Bbar for k in range(L)])
            y = np.array([np.dot(K[: t + 1][::-1], u[b, : t + 1, d]) for t in range(L)])
            ref[b, :, d] = (y + Ds[d] * u[b, :, d]) * silu64(z[b, :, d])
    e = rel(out, ref)
    return e < 1e-10, f"convolution form: {e:.2e}"


def pin_closed_form(fn, seed=3, L=300):
    """P-c: x = 1 and constant (dt, B, C): h_t = -(B/A)(1 - e^{(t+1) dt A}) -> -B/A (eq. 1a equilibrium)."""
    rng = np.random.default_rng(seed)
    batch, D, N = 1, 4, 5
    A = -rng.uniform(0.5, 4.0, (D, N))
    dts = np.array([0.003, 0.05, 0.4, 2.0])
    Bv = rng.standard_normal(N)
    Cv = rng.standard_normal(N)
    u = np.ones((batch, L, D))
    delta = np.broadcast_to(dts, (batch, L, D)).copy()
    B = np.broadcast_to(Bv, (batch, L, N)).copy()
    C = np.broadcast_to(Cv, (batch, L, N)).copy()
    out, last = fn(u, delta, A, B, C, None, None, None, False, None)
    t = np.arange(L)[:, None, None]
    h = -(Bv[None, None, :] / A[None]) * (1.0 - np.exp((t + 1) * dts[None, :, None] * A[None]))  # (L, D, N)
    y = np.einsum("tdn,n->td", h, Cv)
    e1, e2 = rel(out[0], y), rel(last[0], h[-1])
    # the slowest-decaying channel has converged to the equilibrium -B/A
    eq = -(Bv[None, :] / A)
    e3 = rel(last[0, 3], eq[3])
    return (e1 < 1e-12 and e2 < 1e-12 and e3 < 1e-12), f"closed form: out {e1:.2e} last {e2:.2e} equilibrium {e3:.2e}"


def pin_hold(fn, seed=4, L=20):
    """P-d: dt = 0 (no softplus, raw = -bias) keeps the state: h_t = h0, y_t = C_t h0 + Dskip x_t."""
    rng = np.random.default_rng(seed)
    p = small_problem(rng, batch=2, L=L, D=3, N=4)
    p["delta"] = np.broadcast_to(-p["delta_bias"], p["u"].shape).copy()
    h0 = rng.standard_normal((2, 3, 4))
    out, last = fn(**p, softplus=False, h0=h0)
    ref = np.einsum("btn,bdn->btd", p["C"], h0)
    ref = (ref + p["Dskip"][None, None, :] * p["u"]) * silu64(p["z"])
    ok_state = np.array_equal(last, h0)
    e = rel(out, ref)
    return ok_state and e < 1e-13, f"hold: state exact={ok_state}, out {e:.2e}"


def pin_reset(fn, seed=5, L=24, t_reset=13):
    """P-e: a huge dt with A < 0 makes Abar underflow to 0: outputs from the reset token on forget the prefix."""
    rng = np.random.default_rng(seed)
    p = small_problem(rng, batch=1, L=L, D=3, N=4, a_lo=0.5, a_hi=3.0)
    p["delta"][:, t_reset, :] = 4000.0  # dt*A <= -2000: exp underflows to exactly 0
    q = {k: (None if v is None else np.array(v, copy=True)) for k, v in p.items()}
    for k in ("u", "delta", "z", "B", "C"):
        q[k][:, :t_reset] = rng.standard_normal(q[k][:, :t_reset].shape) * (0.5 if k == "delta" else 1.0)
    o1, h1 = fn(**p, softplus=False)
    o2, h2 = fn(**q, softplus=False)
    same = np.array_equal(o1[:, t_reset:], o2[:, t_reset:]) and np.array_equal(h1, h2)
    # right after the reset the state is Bbar x with Bbar -> -B/A (the equilibrium for that token)
    p1 = dict(p)
    p1.update(u=p["u"][:, : t_reset + 1], delta=p["delta"][:, : t_reset + 1], z=None, Dskip=None,
              B=p["B"][:, : t_reset + 1], C=p["C"][:, : t_reset + 1])
    _, hr = fn(**p1, softplus=False)
    dt = p["delta"][0, t_reset] + p["delta_bias"]
    href = -(p["B"][0, t_reset][None, :] / p["A"]) * p["u"][0, t_reset, :, None] * (dt[:, None] > 0)
    e = rel(hr[0], href)
    return same and e < 1e-13, f"reset: suffix identical={same}, state after reset {e:.2e}"


def pin_linearity(fn, seed=6):
    """P-g: without the gate, out is linear in x (dt does not depend on x)."""
    rng = np.random.default_rng(seed)
    p = small_problem(rng, batch=2, L=15, D=3, N=4, gate=False)
    u1 = p["u"]
    u2 = rng.standard_normal(u1.shape)
    a, b = 0.7, -1.9
    o1, h1 = fn(**p)
    p2 = dict(p, u=u2)
    o2, h2 = fn(**p2)
    p3 = dict(p, u=a * u1 + b * u2)
    o3, h3 = fn(**p3)
    e1, e2 = rel(o3, a * o1 + b * o2), rel(h3, a * h1 + b * h2)
    return (e1 < 1e-12 and e2 < 1e-12), f"linearity: out {e1:.2e} last {e2:.2e}"


def pin_causality(fn, seed=7, t0=6):
    """P-h: changing any input at t0 leaves every output before t0 bit-identical."""
    rng = np.random.default_rng(seed)
    p = small_problem(rng, batch=2, L=12, D=3, N=4)
    o1, _ = fn(**p)
    ok = True
    for k in ("u", "delta", "z", "B", "C"):
        q = dict(p)
        q[k] = np.array(p[k], copy=True)
        q[k][:, t0] += 0.75
        o2, _ = fn(**q)
        ok &= np.array_equal(o1[:, :t0], o2[:, :t0]) and not np.array_equal(o1[:, t0:], o2[:, t0:])
    return bool(ok), f"causality: {ok}"


def pin_split(fn, seed=8, m=7):
    """P-i: scanning [0, L) equals scanning [0, m) and continuing from that state over [m, L)."""
    rng = np.random.default_rng(seed)
    p = small_problem(rng, batch=2, L=16, D=3, N=4)
    o, h = fn(**p)

    def part(sl):
        return {k: (v[:, sl] if (v is not None and k in ("u", "delta", "z", "B", "C")) else v) for k, v in p.items()}

    oa, ha = fn(**part(slice(0, m)))
    ob, hb = fn(**part(slice(m, None)), h0=ha)
    e1, e2 = rel(np.concatenate([oa, ob], axis=1), o), rel(hb, h)
    return (e1 < 1e-13 and e2 < 1e-13), f"split/continue: out {e1:.2e} last {e2:.2e}"


def pin_permutation(fn, seed=9):
    """P-k: channels are independent SSMs; permuting channels permutes outputs; batch rows are independent."""
    rng = np.random.default_rng(seed)
    p = small_problem(rng, batch=3, L=10, D=5, N=4)
    o, h = fn(**p)
    perm = rng.permutation(5)
    q = dict(p)
    for k in ("u", "delta", "z"):
        q[k] = p[k][:, :, perm]
    q["A"] = p["A"][perm]
    q["delta_bias"] = p["delta_bias"][perm]
    q["Dskip"] = p["Dskip"][perm]
    o2, h2 = fn(**q)
    ok = np.array_equal(o2, o[:, :, perm]) and np.array_equal(h2, h[:, perm])
    r = {k: (v[1:2] if (v is not None and k in ("u", "delta", "z", "B", "C")) else v) for k, v in p.items()}
    o3, h3 = fn(**r)
    ok &= np.array_equal(o3[0], o[1]) and np.array_equal(h3[0], h[1])
    return bool(ok), f"permutation/batch independence: {ok}"


def pin_softplus_bias(fn, seed=10):
    """Selection front end: with the flag, dt = softplus(raw + bias); equals the unflagged scan fed that dt."""
    rng = np.random.default_rng(seed)
    p = small_problem(rng, batch=2, L=10, D=3, N=4)
    o1, h1 = fn(**p, softplus=True)
    q = dict(p, delta=softplus64(p["delta"] + p["delta_bias"][None, None, :]), delta_bias=None)
    o2, h2 = fn(**q, softplus=False)
    e1, e2 = rel(o1, o2), rel(h1, h2)
    return (e1 < 1e-13 and e2 < 1e-13), f"softplus(raw+bias): out {e1:.2e} last {e2:.2e}"


def pin_gate_skip(fn, seed=11):
    """Epilogue: out = (y + Dskip x) z sigmoid(z), y the ungated, unskipped readout."""
    rng = np.random.default_rng(seed)
    p = small_problem(rng, batch=2, L=10, D=3, N=4)
    o1, _ = fn(**p)
    o0, _ = fn(**dict(p, z=None, Dskip=None))
    ref = (o0 + p["Dskip"][None, None, :] * p["u"]) * silu64(p["z"])
    e = rel(o1, ref)
    return e < 1e-13, f"gate/skip: {e:.2e}"


ALL_PINS = [pin_brute_force, pin_convolution, pin_closed_form, pin_hold, pin_reset, pin_linearity,
            pin_causality, pin_split, pin_permutation, pin_softplus_bias, pin_gate_skip]
