"""The Mamba-block oracle (oracle.block) against facts outside its own code:
a one-token closed form of the whole block on scalars, the zero gate, and the
invariance of the output under consistent permutations of the model and the
channel dimensions (which fixes how W_in, W_x, W_dt and W_out contract)."""
import math

import numpy as np

import oracle
import pins


def _silu(v):
    return v / (1.0 + math.exp(-v))


def _softplus(v):
    return math.log1p(math.exp(v))


def test_one_token_closed_form_on_scalars():
    """d_model = D = N = R = 1 and L = 1 from a zero state: every step of the block is
    a scalar, so out = w_out * (gamma*beta*bz*x^3 + Dskip*x) * SiLU(b*h) with x = SiLU(a*h),
    dt = softplus(r*x*w + bias) and bz the ZOH weight (e^{dt A} - 1)/A."""
    a, b, r, beta, gamma, w, bias, A, Dsk, w_out = 0.7, -1.3, 0.9, 1.4, -0.6, 1.1, -0.2, -0.8, 0.35, 1.7
    for hval in (0.5, -1.2, 2.0):
        x = _silu(a * hval)
        dt = _softplus(r * x * w + bias)
        bz = math.expm1(dt * A) / A
        y = gamma * x * (bz * beta * x * x) + Dsk * x
        want = w_out * y * _silu(b * hval)
        out, last = oracle.block(np.full((1, 1, 1), hval), np.array([[a], [b]]), np.array([[r], [beta], [gamma]]),
                                 np.array([[w]]), np.array([bias]), np.array([[A]]), np.array([Dsk]),
                                 np.array([[w_out]]), 1)
        assert abs(out[0, 0, 0] - want) <= 1e-13 * max(1.0, abs(want)), (hval, out[0, 0, 0], want)
        assert abs(last[0, 0, 0] - bz * beta * x * x) <= 1e-14


def _params(rng, dm=6, D=5, N=4, R=2):
    return dict(W_in=rng.standard_normal((2 * D, dm)) * 0.5, W_x=rng.standard_normal((R + 2 * N, D)) * 0.5,
                W_dt=rng.standard_normal((D, R)) * 0.5, dt_bias=rng.uniform(-2, 0, D),
                A=-rng.uniform(0.3, 2.0, (D, N)), Dskip=rng.standard_normal(D),
                W_out=rng.standard_normal((dm, D)) * 0.5, dstate=N)


def test_zero_gate_branch_silences_the_output():
    """W_in's gate rows zero: z = 0, SiLU(0) = 0, so out = 0 while the state still
    follows the SSM branch (the same as with any other gate rows)."""
    rng = np.random.default_rng(1)
    p = _params(rng)
    h = rng.standard_normal((2, 7, 6))
    q = dict(p)
    q["W_in"] = p["W_in"].copy()
    q["W_in"][5:] = 0.0
    out, last = oracle.block(h, **q)
    assert np.all(out == 0.0)
    _, last_ref = oracle.block(h, **p)
    assert pins.rel(last, last_ref) == 0.0


def test_permuting_model_features_leaves_the_output_permuted():
    """Permuting the d_model features of hidden and W_in's columns together, and
    W_out's rows, permutes the output the same way."""
    rng = np.random.default_rng(2)
    p = _params(rng)
    h = rng.standard_normal((2, 9, 6))
    perm = rng.permutation(6)
    out, _ = oracle.block(h, **p)
    q = dict(p)
    q["W_in"] = p["W_in"][:, perm]
    q["W_out"] = p["W_out"][perm]
    out2, _ = oracle.block(h[..., perm], **q)
    assert pins.rel(out2, out[..., perm]) < 1e-13


def test_permuting_channels_consistently_leaves_the_output_unchanged():
    """Channels are independent SSMs (Figure 1): permuting them in both halves of
    W_in, in W_x's columns, W_dt's rows, A, Dskip, dt_bias and W_out's columns
    leaves the block's output unchanged and permutes the final state."""
    rng = np.random.default_rng(3)
    p = _params(rng)
    h = rng.standard_normal((2, 9, 6))
    c = rng.permutation(5)
    out, last = oracle.block(h, **p)
    q = dict(p)
    q["W_in"] = np.concatenate([p["W_in"][:5][c], p["W_in"][5:][c]])
    q["W_x"] = p["W_x"][:, c]
    q["W_dt"] = p["W_dt"][c]
    q["A"], q["Dskip"], q["dt_bias"] = p["A"][c], p["Dskip"][c], p["dt_bias"][c]
    q["W_out"] = p["W_out"][:, c]
    out2, last2 = oracle.block(h, **q)
    assert pins.rel(out2, out) < 1e-12
    assert pins.rel(last2, last[:, c]) < 1e-13


def test_swapping_branches_changes_the_output():
    """The SSM and gate halves of W_in are not interchangeable (SiLU sits on the
    first half only): swapping them changes the output."""
    rng = np.random.default_rng(4)
    p = _params(rng)
    h = rng.standard_normal((1, 5, 6))
    out, _ = oracle.block(h, **p)
    q = dict(p)
    q["W_in"] = np.concatenate([p["W_in"][5:], p["W_in"][:5]])
    out2, _ = oracle.block(h, **q)
    assert pins.rel(out2, out) > 1e-3
