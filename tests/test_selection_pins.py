"""The selection oracle (section 3.2 projections) against facts that do not
come from the oracle: the page's own form of the dt projection, exact column
selection, linearity, and the order of the two contractions."""
import numpy as np

import oracle


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_page_form_broadcast_of_a_rank_one_projection():
    """Broadcast_D(Linear_1(x)) is dt_rank = 1 with W_dt = ones: every channel of a
    token gets the same value, x_t . w."""
    rng = np.random.default_rng(1)
    x = _rand(rng, 2, 9, 12)
    N = 3
    w = _rand(rng, 12)
    W_x = np.concatenate([w[None, :], _rand(rng, 2 * N, 12)])
    delta, B, C = oracle.selection(x, W_x, np.ones((12, 1)), N)
    expect = np.einsum("bld,d->bl", x, w)
    assert np.allclose(delta, expect[:, :, None] * np.ones(12), rtol=1e-14, atol=1e-14)


def test_unit_rows_select_input_channels_exactly():
    """Rows of W_x that are unit vectors copy input channels into B and C bit for bit."""
    rng = np.random.default_rng(2)
    D, N, R = 10, 4, 2
    x = _rand(rng, 3, 7, D)
    pick_b = [3, 0, 9, 5]
    pick_c = [1, 1, 8, 2]
    W_x = np.zeros((R + 2 * N, D))
    W_x[:R] = _rand(rng, R, D)
    for n in range(N):
        W_x[R + n, pick_b[n]] = 1.0
        W_x[R + N + n, pick_c[n]] = 1.0
    _, B, C = oracle.selection(x, W_x, _rand(rng, D, R), N)
    assert np.array_equal(B, x[:, :, pick_b])
    assert np.array_equal(C, x[:, :, pick_c])


def test_linear_in_x():
    rng = np.random.default_rng(3)
    D, N, R = 16, 4, 3
    W_x, W_dt = _rand(rng, R + 2 * N, D), _rand(rng, D, R)
    x1, x2 = _rand(rng, 2, 5, D), _rand(rng, 2, 5, D)
    a = oracle.selection(2.5 * x1 - 0.75 * x2, W_x, W_dt, N)
    b1 = oracle.selection(x1, W_x, W_dt, N)
    b2 = oracle.selection(x2, W_x, W_dt, N)
    for k in range(3):
        assert np.allclose(a[k], 2.5 * b1[k] - 0.75 * b2[k], rtol=1e-12, atol=1e-12)


def test_dt_projection_equals_the_combined_weight():
    """delta = (x W_rank^T) W_dt^T = x (W_dt W_rank)^T: the other contraction order,
    written with explicit loops on a tiny case."""
    rng = np.random.default_rng(4)
    D, N, R = 6, 2, 3
    x = _rand(rng, 1, 4, D)
    W_x, W_dt = _rand(rng, R + 2 * N, D), _rand(rng, D, R)
    delta, _, _ = oracle.selection(x, W_x, W_dt, N)
    combined = np.zeros((D, D))
    for d in range(D):
        for k in range(D):
            combined[d, k] = sum(W_dt[d, r] * W_x[r, k] for r in range(R))
    ref = np.zeros((1, 4, D))
    for t in range(4):
        for d in range(D):
            ref[0, t, d] = sum(combined[d, k] * x[0, t, k] for k in range(D))
    assert np.allclose(delta, ref, rtol=1e-13, atol=1e-13)


def test_columns_are_not_mixed_up():
    """B comes from rows R..R+N of W_x and C from the last N: distinct weights, distinct outputs."""
    rng = np.random.default_rng(5)
    D, N, R = 8, 3, 2
    x = _rand(rng, 1, 3, D)
    W_x = np.zeros((R + 2 * N, D))
    W_x[R:R + N, 0] = 1.0         # B = x[..., 0] in every state
    W_x[R + N:, 1] = 2.0          # C = 2 x[..., 1]
    _, B, C = oracle.selection(x, W_x, _rand(rng, D, R), N)
    assert np.array_equal(B, np.repeat(x[..., :1], N, axis=-1))
    assert np.array_equal(C, np.repeat(2.0 * x[..., 1:2], N, axis=-1))


def test_store_applies_to_xdbl_and_results_only():
    """With a storage rounding, delta is the rounded product of the rounded xdbl."""
    rng = np.random.default_rng(6)
    D, N, R = 8, 2, 3
    x = _rand(rng, 1, 5, D)
    W_x, W_dt = _rand(rng, R + 2 * N, D), _rand(rng, D, R)
    q = lambda a: np.round(np.asarray(a) * 64.0) / 64.0  # a coarse stand-in storage type
    delta, B, C = oracle.selection(x, W_x, W_dt, N, store=q)
    xdbl = q(x @ W_x.T)
    assert np.array_equal(B, xdbl[..., R:R + N]) and np.array_equal(C, xdbl[..., R + N:])
    assert np.array_equal(delta, q(xdbl[..., :R] @ W_dt.T))


def test_store_delta_false_keeps_the_dt_projection_unrounded():
    rng = np.random.default_rng(7)
    D, N, R = 8, 2, 3
    x = _rand(rng, 1, 5, D)
    W_x, W_dt = _rand(rng, R + 2 * N, D), _rand(rng, D, R)
    q = lambda a: np.round(np.asarray(a) * 64.0) / 64.0
    delta, _, _ = oracle.selection(x, W_x, W_dt, N, store=q, store_delta=False)
    assert np.array_equal(delta, q(x @ W_x.T)[..., :R] @ W_dt.T)
