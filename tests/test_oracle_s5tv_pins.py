"""Pins of the oracle's continuous-time S5 with a per-step step size
(oracle.s5_recurrence_tv; "Simplified State Space Layers for Sequence
Modeling", section 3: zero-order-hold discretisation of a diagonal system with
a timescale per state, and a different timescale supplied at each step for
irregular sampling).

Each pin is a function of an implementation, run on the oracle (must hold) and
on copies with one planted mistake (each must be rejected by a pin).  None of
them re-types the discretisation formula: the reference values come from a
numerical integration of the differential equation x' = Lambda x + B~ u with u
held over each step (classical Runge-Kutta, many substeps), from exact
properties of that integration (two half steps with the same input make one
step; a zero-length step changes nothing; only the product of step and
timescale matters), and from the closed form at Lambda = 0 (an integrator)."""
import types

import numpy as np
import pytest

import oracle
from long_convolution_sequence_amd import inputs


def _small(seed=3, B=2, H=3, P=4, L=7):
    x = inputs.s5_tv_inputs(B, H, P, L, seed=seed)
    # larger timescales than the workload's, so a step moves the state visibly
    x["delta"] = (x["delta"] * 10.0).astype(np.float32)
    return x


def _call(impl, x, **over):
    d = dict(x)
    d.update(over)
    return impl(d["u"], d["lam_c"], d["Bt"], d["C"], d["D"], d["delta"], d["step"])


def _rk4_reference(x, substeps=400):
    """y from integrating x' = Lambda x + B~ u_k over each step of length
    step[b,k] * delta (u held), float64 classical Runge-Kutta."""
    u = x["u"].astype(np.float64)
    lam = x["lam_c"].astype(np.complex128)
    Bt = x["Bt"].astype(np.complex128)
    C = x["C"].astype(np.complex128)
    D = x["D"].astype(np.float64)
    dl = x["delta"].astype(np.float64)
    st = x["step"].astype(np.float64)
    Bsz, H, L = u.shape
    y = np.empty((Bsz, H, L))
    for b in range(Bsz):
        s = np.zeros(lam.shape[0], dtype=np.complex128)
        for k in range(L):
            g = Bt @ u[b, :, k]
            tau = st[b, k] * dl
            h = tau / substeps
            for _ in range(substeps):
                k1 = lam * s + g
                k2 = lam * (s + 0.5 * h * k1) + g
                k3 = lam * (s + 0.5 * h * k2) + g
                k4 = lam * (s + h * k3) + g
                s = s + h / 6.0 * (k1 + 2 * k2 + 2 * k3 + k4)
            y[b, :, k] = (C @ s).real + D * u[b, :, k]
    return y


def _rel(a, b):
    return np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300)


def pin_matches_ode_integration(impl):
    x = _small()
    return _rel(_call(impl, x), _rk4_reference(x)) < 1e-9


def pin_two_half_steps_make_one(impl):
    x = _small(seed=5, L=1)
    one = _call(impl, x)[..., 0]
    u2 = np.repeat(x["u"], 2, axis=2)
    s2 = np.repeat(x["step"] * 0.5, 2, axis=1).astype(np.float32)
    two = _call(impl, x, u=u2, step=s2)[..., 1]
    return _rel(two, one) < 1e-12


def pin_zero_step_changes_nothing(impl):
    x = _small(seed=6)
    st = x["step"].copy()
    st[:, 4] = 0.0
    y = _call(impl, x, step=st)
    Du = x["D"].astype(np.float64)[None, :] * x["u"].astype(np.float64)[:, :, 4]
    Du3 = x["D"].astype(np.float64)[None, :] * x["u"].astype(np.float64)[:, :, 3]
    return _rel(y[:, :, 4] - Du, y[:, :, 3] - Du3) < 1e-12


def pin_only_step_times_timescale_matters(impl):
    x = _small(seed=8)
    a = _call(impl, x)
    b = _call(impl, x, step=(x["step"] * 4.0).astype(np.float32),
              delta=(x["delta"] * 0.25).astype(np.float32))
    c = _call(impl, x, step=(x["step"] * 4.0).astype(np.float32))
    return _rel(b, a) < 1e-12 and _rel(c, a) > 1e-3


def pin_integrator_at_lambda_zero(impl):
    x = _small(seed=9)
    lam0 = np.zeros_like(x["lam_c"])
    y = _call(impl, x, lam_c=lam0)
    u = x["u"].astype(np.float64)
    v = np.einsum("ph,bhl->bpl", x["Bt"].astype(np.complex128), u)
    tau = x["step"].astype(np.float64)[:, None, :] * x["delta"].astype(np.float64)[None, :, None]
    s = np.cumsum(tau * v, axis=2)
    ref = np.einsum("hp,bpl->bhl", x["C"].astype(np.complex128), s).real \
        + x["D"].astype(np.float64)[None, :, None] * u
    return _rel(y, ref) < 1e-12


PINS = [pin_matches_ode_integration, pin_two_half_steps_make_one, pin_zero_step_changes_nothing,
        pin_only_step_times_timescale_matters, pin_integrator_at_lambda_zero]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_tv_pin(pin):
    assert pin(oracle.s5_recurrence_tv)


def _mutant(kind):
    """A copy of the recurrence with one planted mistake."""
    def impl(u, lam_c, Bt, C, D, delta, step):
        u = np.asarray(u).astype(np.float64)
        lam = np.asarray(lam_c).astype(np.complex128)
        Bb = np.asarray(Bt).astype(np.complex128)
        Cc = np.asarray(C).astype(np.complex128)
        D = np.asarray(D).astype(np.float64)
        dl = np.asarray(delta).astype(np.float64)
        st = np.asarray(step).astype(np.float64)
        Bsz, H, L = u.shape
        x = np.zeros((Bsz, lam.shape[0]), dtype=np.complex128)
        y = np.empty((Bsz, H, L))
        for k in range(L):
            sk = np.ones(Bsz) if kind == "no_step" else st[:, k]
            dt = sk[:, None] * dl[None, :]
            z = lam[None, :] * dt
            a = 1.0 + z if kind == "first_order" else np.exp(z)
            if kind == "euler":
                beta = dt
            elif kind == "step_a_only":
                zb = lam[None, :] * dl[None, :]
                beta = np.where(lam == 0, dl[None, :], (np.exp(zb) - 1.0) / np.where(lam == 0, 1.0, lam))
            elif kind == "over_z":
                beta = np.where(z == 0, 1.0, (np.exp(z) - 1.0) / np.where(z == 0, 1.0, z))
            else:
                beta = np.where(lam == 0, dt, (np.exp(z) - 1.0) / np.where(lam == 0, 1.0, lam))
            x = a * x + beta * (u[:, :, k] @ Bb.T)
            y[:, :, k] = (x @ Cc.T).real + D[None, :] * u[:, :, k]
        return y
    return impl


@pytest.mark.parametrize("kind", ["euler", "first_order", "no_step", "step_a_only", "over_z"])
def test_tv_pins_reject_planted_mistake(kind):
    m = _mutant(kind)
    failed = [p.__name__ for p in PINS if not p(m)]
    assert failed, f"no pin caught the planted mistake '{kind}'"


def test_tv_mutant_harness_is_faithful():
    m = _mutant("none")
    assert all(p(m) for p in PINS)


def test_tv_inputs_are_seeded_and_float32():
    a = inputs.s5_tv_inputs(2, 3, 4, 5, seed=11)
    b = inputs.s5_tv_inputs(2, 3, 4, 5, seed=11)
    for k in a:
        assert np.array_equal(a[k], b[k])
    assert a["u"].dtype == np.float32 and a["step"].dtype == np.float32
    assert a["lam_c"].dtype == np.complex64 and a["Bt"].dtype == np.complex64
    assert np.all(a["step"] >= 0.5) and np.all(a["step"] <= 1.5)
