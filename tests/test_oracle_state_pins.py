"""Pins of the oracle's stateful recurrence (CPU only).

oracle.dlr_recurrence_state runs x_k = lambda x_{k-1} + u_k from a given x_{-1}
and returns the last state ("The Annotated S4", Part 1, "Discrete-time SSM: the
recurrent representation"; the DLR of "Simplifying and Understanding State
Space Models with Diagonal Linear RNNs", section 2).  It is pinned to:

* zero state: the already pinned direct O(L^2) sum (dlr_direct);
* free response (u = 0, D = 0): unrolling the recurrence gives
  x_k = lambda^(k+1) x_{-1}, so y_k = Re sum_n W_n lambda_n^(k+1) x0_n -- the
  powers taken here as exp((k+1) log lambda), not by repeated products;
* chunking: a run split at any point and continued from the returned state
  equals the unsplit run (the state is everything the past contributes);
* superposition: the map is linear in (u, x0).

Each pin is a function of an implementation; planted mistakes (a wrong power
of lambda on the state, a dropped or conjugated state, the state returned one
step early) must each fail at least one pin.
"""
import numpy as np
import pytest

import oracle
from long_convolution_sequence_amd import inputs

RTOL = 1e-11


def _rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300)


def _case(B=2, H=3, N=5, L=37, seed=7):
    x = inputs.dlr_inputs(B, H, N, L, seed=seed)
    rng = np.random.default_rng(seed + 100)
    x0 = rng.normal(size=(B, H, N)) + 1j * rng.normal(size=(B, H, N))
    return x, x0


def pin_zero_state_is_plain(impl):
    x, _ = _case()
    y, _ = impl(x["u"], x["log_re"], x["log_im"], x["W"], x["D"], None)
    ref = oracle.dlr_direct(x["u"], x["log_re"], x["log_im"], x["W"], x["D"])
    return _rel(y, ref) < RTOL


def pin_free_response(impl):
    x, x0 = _case()
    B, H, L = x["u"].shape
    u = np.zeros_like(x["u"])
    D = np.zeros_like(x["D"])
    y, xl = impl(u, x["log_re"], x["log_im"], x["W"], D, x0)
    loglam = -np.asarray(x["log_re"], np.float64) ** 2 + 1j * np.asarray(x["log_im"], np.float64)
    w = np.asarray(x["W"]).astype(np.complex128)[0]
    k1 = np.arange(1, L + 1, dtype=np.float64)
    pw = np.exp(k1[:, None, None] * loglam[0][None])  # [L, H, N]: lambda^(k+1)
    ref = np.einsum("khn,hn,bhn->bhk", pw, w, x0).real
    ref_state = pw[-1][None] * x0
    return _rel(y, ref) < RTOL and _rel(xl, ref_state) < RTOL


def pin_chunking(impl):
    x, x0 = _case(L=41)
    args = (x["log_re"], x["log_im"], x["W"], x["D"])
    y, xl = impl(x["u"], *args, x0)
    ok = True
    for cut in (1, 13, 40):
        y1, s1 = impl(x["u"][..., :cut], *args, x0)
        y2, s2 = impl(x["u"][..., cut:], *args, s1)
        ok &= _rel(np.concatenate([y1, y2], axis=-1), y) < RTOL and _rel(s2, xl) < RTOL
    return ok


def pin_superposition(impl):
    x, x0 = _case()
    args = (x["log_re"], x["log_im"], x["W"], x["D"])
    y, xl = impl(x["u"], *args, x0)
    ya, sa = impl(x["u"], *args, None)
    yb, sb = impl(np.zeros_like(x["u"]), *args, x0)
    return _rel(y, ya + yb) < RTOL and _rel(xl, sa + sb) < RTOL


PINS = [pin_zero_state_is_plain, pin_free_response, pin_chunking, pin_superposition]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_state_pin(pin):
    assert pin(oracle.dlr_recurrence_state)


def _mutant(kind):
    def impl(u, log_re, log_im, W, D, x0=None):
        u = np.asarray(u, np.float64)
        B, H, L = u.shape
        lam = oracle.dlr_lambda(log_re, log_im)[0]
        w = np.asarray(W).astype(np.complex128)[0]
        N = lam.shape[-1]
        x = np.zeros((B, H, N), np.complex128) if x0 is None else np.asarray(x0, np.complex128)
        if kind == "drop_state":
            x = np.zeros_like(x)
        elif kind == "conj_state":
            x = np.conj(x)
        y = u * np.asarray(D, np.float64)[0][None, :, None]
        prev = x
        for k in range(L):
            prev = x
            if kind == "power_k" and k == 0:
                x = x + u[:, :, 0, None]  # the state enters without its lambda
            else:
                x = lam[None] * x + u[:, :, k, None]
            y[:, :, k] += (x * w[None]).sum(-1).real
        return y, (prev if kind == "stale_state" and L > 0 else x)
    return impl


@pytest.mark.parametrize("kind", ["power_k", "drop_state", "conj_state", "stale_state"])
def test_state_pins_reject_planted_mistake(kind):
    m = _mutant(kind)
    assert [p.__name__ for p in PINS if not p(m)], f"no pin caught '{kind}'"


def test_state_mutant_harness_is_faithful():
    m = _mutant("none")
    assert all(p(m) for p in PINS)
