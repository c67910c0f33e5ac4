"""GPU parity of the continuous-time S5 path with a per-step step size
(dssm_s5_forward_tv, through the C ABI) against the float64 oracle
(oracle.s5_recurrence_tv, pinned in test_oracle_s5tv_pins.py).  Same bar as
the other paths: relative L2 <= 1e-5, max |err| <= 1e-4 RMS."""
import numpy as np
import pytest

import oracle
from long_convolution_sequence_amd import binding as bd
from long_convolution_sequence_amd import inputs

from test_gpu_parity import assert_close, say, _torch

pytestmark = pytest.mark.gpu


def run_tv(x):
    torch = _torch()
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in x.items()}
    y = bd.s5_forward_tv(t["u"], t["lam_c"], t["Bt"], t["C"], t["D"], t["delta"], t["step"])
    torch.cuda.synchronize()
    return y.cpu().numpy()


def ref_tv(x):
    return oracle.s5_recurrence_tv(x["u"], x["lam_c"], x["Bt"], x["C"], x["D"], x["delta"],
                                   x["step"])


def test_s5_tv_workload_full_size():
    c = inputs.config("s5_mimo")
    say("case: s5 time-varying, workload shape B=%d H=%d P=%d L=%d" % (c["B"], c["H"], c["P"], c["L"]))
    x = inputs.s5_tv_inputs(c["B"], c["H"], c["P"], c["L"], seed=c["seed"])
    assert_close(run_tv(x), ref_tv(x), "s5tv/full")


TV_EDGE = [
    # (B, H, P, L): one step, ragged tiles, several 4096-step tiles, more than
    # 256 rows of either projection
    (1, 1, 1, 1), (2, 3, 5, 100), (1, 6, 3, 4097), (3, 5, 40, 257), (1, 300, 33, 96),
    (2, 64, 32, 9000),
]


@pytest.mark.parametrize("shape", TV_EDGE, ids=["B%dH%dP%dL%d" % s for s in TV_EDGE])
def test_s5_tv_edge_shapes(shape):
    B, H, P, L = shape
    say("case: s5 time-varying edge B=%d H=%d P=%d L=%d" % shape)
    x = inputs.s5_tv_inputs(B, H, P, L, seed=900 + H + P + L)
    assert_close(run_tv(x), ref_tv(x), "s5tv/edge")


def test_s5_tv_irregular_steps_with_zeros_and_long_gaps():
    say("case: s5 time-varying, steps in [0, 8] with zeros")
    x = inputs.s5_tv_inputs(2, 40, 24, 3000, seed=31)
    rng = np.random.default_rng(5)
    st = rng.uniform(0.0, 8.0, size=x["step"].shape)
    st[rng.random(st.shape) < 0.1] = 0.0
    x["step"] = st.astype(np.float32)
    assert_close(run_tv(x), ref_tv(x), "s5tv/irregular")


def test_s5_tv_integrator_at_lambda_zero():
    say("case: s5 time-varying, lambda_c = 0 for some states")
    x = inputs.s5_tv_inputs(2, 16, 8, 700, seed=32)
    lam = x["lam_c"].copy()
    lam[::2] = 0.0
    x["lam_c"] = lam
    # keep the integrators' states moderate: their sums grow like sqrt(L)
    assert_close(run_tv(x), ref_tv(x), "s5tv/integrator")


def test_s5_tv_constant_step_matches_fixed_layer_on_device():
    """With every step 1 the layer is the fixed-step S5 with the zero-order-hold
    parameters; the two device paths agree on it (within the bar of each)."""
    say("case: s5 time-varying with constant steps vs the fixed-step path")
    torch = _torch()
    x = inputs.s5_tv_inputs(2, 24, 16, 2500, seed=33)
    x["step"] = np.ones_like(x["step"])
    y_tv = run_tv(x)
    lam = x["lam_c"].astype(np.complex128)
    z = lam * x["delta"].astype(np.float64)
    lbar = np.exp(z)
    bbar = ((lbar - 1.0) / lam)[:, None] * x["Bt"].astype(np.complex128)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda()
         for k, v in dict(u=x["u"], lam=lbar.astype(np.complex64), Bbar=bbar.astype(np.complex64),
                          C=x["C"], D=x["D"]).items()}
    y_fixed = bd.s5_forward(t["u"], t["lam"], t["Bbar"], t["C"], t["D"])
    torch.cuda.synchronize()
    ref = ref_tv(x)
    assert_close(y_tv, ref, "s5tv/constant")
    assert_close(y_fixed.cpu().numpy(), ref, "s5/fixed-from-zoh")


def test_s5_tv_is_deterministic():
    x = inputs.s5_tv_inputs(2, 24, 9, 3000, seed=17)
    say("case: s5 time-varying determinism")
    a = run_tv(x)
    b = run_tv(x)
    assert np.array_equal(a, b)
