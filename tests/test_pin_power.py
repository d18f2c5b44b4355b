"""The pins are strong enough: each plausible mistake planted in a copy of the
numpy oracle twin fails at least one pin (CPU only).

The mutants below are the oracle's numpy twin with one deliberate error each;
they exist only here, to measure the pins, and are never used as references.
"""
import numpy as np
import pytest

import pins


def mutant_scan(mutation):
    def fn(u, delta, A, B, C, delta_bias=None, Dskip=None, z=None, softplus=True, h0=None):
        u = np.asarray(u, np.float64)
        dt = np.asarray(delta, np.float64)
        A = np.asarray(A, np.float64)
        B = np.asarray(B, np.float64)
        C = np.asarray(C, np.float64)
        if mutation == "swap_BC":
            B, C = C, B
        batch, L, D = u.shape
        N = A.shape[1]
        if delta_bias is not None and mutation not in ("drop_bias", "bias_after_softplus"):
            dt = dt + np.asarray(delta_bias)[None, None, :]
        if softplus:
            dt = np.log1p(np.exp(-dt)) if mutation == "softplus_sign" else np.logaddexp(0.0, dt)
        if delta_bias is not None and mutation == "bias_after_softplus":
            dt = dt + np.asarray(delta_bias)[None, None, :]
        h = np.zeros((batch, D, N)) if (h0 is None or mutation == "ignore_h0") else np.array(h0, np.float64)
        out = np.empty((batch, L, D))
        for t in range(L):
            x = dt[:, t, :, None] * A[None]
            if mutation == "a_sign":
                x = -x
            abar = np.exp(x)
            safe = np.where(x == 0.0, 1.0, x)
            phi = np.where(x == 0.0, 1.0, np.expm1(x) / safe)
            if mutation == "euler_B":
                phi = np.ones_like(phi)
            if mutation == "phi_half":
                phi = np.where(x == 0.0, 1.0, np.expm1(x / 2) / (safe / 2))
            bbar = phi * dt[:, t, :, None] * B[:, t, None, :]
            h_prev = h
            h = abar * h + bbar * u[:, t, :, None]
            if mutation == "u_twice":
                h = h + 0 * bbar
                h = abar * h_prev + bbar * u[:, t, :, None] * u[:, t, :, None]
            hr = h_prev if mutation == "readout_before_update" else h
            y = np.einsum("bdn,bn->bd", hr, C[:, t, :])
            if mutation == "readout_prev_C" and t > 0:
                y = np.einsum("bdn,bn->bd", hr, C[:, t - 1, :])
            if Dskip is not None and mutation not in ("drop_skip", "skip_after_gate"):
                y = y + np.asarray(Dskip)[None, :] * u[:, t, :]
            if z is not None:
                zt = np.asarray(z, np.float64)[:, t, :]
                g = 1.0 / (1.0 + np.exp(-zt)) if mutation == "sigmoid_gate" else zt / (1.0 + np.exp(-zt))
                y = y * g
            if Dskip is not None and mutation == "skip_after_gate":
                y = y + np.asarray(Dskip)[None, :] * u[:, t, :]
            out[:, t, :] = y
        if mutation == "state_off_by_one":
            return out, h_prev
        return out, h

    return fn


MUTATIONS = ["swap_BC", "drop_bias", "bias_after_softplus", "softplus_sign", "ignore_h0", "a_sign", "euler_B",
             "phi_half", "u_twice", "readout_before_update", "readout_prev_C", "drop_skip", "skip_after_gate",
             "sigmoid_gate", "state_off_by_one"]


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_every_planted_mistake_fails_a_pin(mutation):
    fn = mutant_scan(mutation)
    failed = []
    for pin in pins.ALL_PINS:
        with np.errstate(all="ignore"):
            try:
                ok, detail = pin(fn)
            except Exception as exc:  # a crash also counts as caught
                ok, detail = False, repr(exc)
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"mutation {mutation} passed every pin"


def test_unmutated_copy_passes_every_pin():
    fn = mutant_scan("none")
    for pin in pins.ALL_PINS:
        ok, detail = pin(fn)
        assert ok, detail
