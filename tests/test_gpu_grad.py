"""GPU parity of the layer gradients (dssm_backward, through the C ABI)
against the float64 oracle (oracle.dlr_backward, itself pinned by finite
differences of the forward map).  Each returned tensor meets the bar of the
forward paths: relative L2 <= 1e-5 and max |err| <= 1e-4 RMS."""
import numpy as np
import pytest

import oracle
from long_convolution_sequence_amd import binding as bd
from long_convolution_sequence_amd import inputs

from test_gpu_parity import assert_close, dev, say, _torch

pytestmark = pytest.mark.gpu


def run_bwd(x, dy, bi):
    torch = _torch()
    t = dev(x)
    g = torch.from_numpy(np.ascontiguousarray(dy)).cuda()
    du, out = bd.backward(t["u"], g, t["log_re"], t["log_im"], t["W"], t["D"], bidirectional=bi)
    torch.cuda.synchronize()
    return du.cpu().numpy(), {k: v.cpu().numpy() for k, v in out.items()}


def check(x, dy, bi, what, hs=None):
    du, g = run_bwd(x, dy, bi)
    if hs is not None:  # channels are independent: the oracle on a subset of them
        x = {k: (v[:, hs] if k in ("u", "log_re", "log_im", "W", "D") else v) for k, v in x.items()}
        dy = dy[:, hs]
        du = du[:, hs]
        g = {k: v[:, hs] for k, v in g.items()}
    r_du, r_lre, r_lim, r_dW, r_dD = oracle.dlr_backward(x["u"], dy, x["log_re"], x["log_im"],
                                                         x["W"], x["D"], bi)
    assert_close(du, r_du, what + " du")
    assert_close(g["dlog_re"], r_lre, what + " dlog_re")
    assert_close(g["dlog_im"], r_lim, what + " dlog_im")
    assert_close(np.stack([g["dW"].real, g["dW"].imag]), np.stack([r_dW.real, r_dW.imag]),
                 what + " dW")
    assert_close(g["dD"], r_dD, what + " dD")


SHAPES = [  # (B, H, N, L, bi)
    (2, 3, 8, 300, 0), (2, 3, 8, 300, 1), (3, 2, 64, 2000, 0), (2, 2, 64, 4097, 1),
    (1, 2, 100, 777, 1), (2, 3, 16, 17, 0), (3, 2, 8, 1, 1), (5, 2, 16, 16384, 0),
    # many batch rows summed in the frequency domain, both directions, ragged L
    (9, 2, 16, 5000, 1), (4, 300, 8, 1024, 1),
]


@pytest.mark.parametrize("shape", SHAPES, ids=["B%dH%dN%dL%dbi%d" % s for s in SHAPES])
def test_backward_against_oracle(shape):
    B, H, N, L, bi = shape
    say("case: backward B=%d H=%d N=%d L=%d bi=%d" % shape)
    x = inputs.dlr_inputs(B, H, N, L, bidirectional=bool(bi), seed=600 + L + N, re_scale=0.5)
    dy = np.random.default_rng(L + 7).normal(size=(B, H, L)).astype(np.float32)
    check(x, dy, bool(bi), "backward")


def test_backward_long_sequence_sampled_channels():
    c = inputs.config("long_sequence")
    say("case: backward on the long-sequence workload, channels 0 and 77")
    x = inputs.inputs_for(c)
    dy = np.random.default_rng(123).normal(size=x["u"].shape).astype(np.float32)
    check(x, dy, False, "backward/long", hs=[0, 77])


def test_backward_empty_batch_zeroes_parameter_gradients():
    torch = _torch()
    x = inputs.dlr_inputs(1, 3, 8, 40, seed=3)
    t = dev(x)
    u = torch.zeros(0, 3, 40, device="cuda")
    du, g = bd.backward(u, u.clone(), t["log_re"], t["log_im"], t["W"], t["D"])
    torch.cuda.synchronize()
    assert du.shape == (0, 3, 40)
    for v in g.values():
        assert torch.count_nonzero(v) == 0


def test_backward_is_deterministic():
    torch = _torch()
    x = inputs.dlr_inputs(2, 3, 16, 1000, bidirectional=True, seed=8)
    dy = np.random.default_rng(5).normal(size=(2, 3, 1000)).astype(np.float32)
    say("case: backward determinism")
    a = run_bwd(x, dy, True)
    b = run_bwd(x, dy, True)
    assert np.array_equal(a[0], b[0])
    for k in a[1]:
        assert np.array_equal(a[1][k], b[1][k])
