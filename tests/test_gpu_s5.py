"""GPU parity of the S5 multi-input multi-output path (C ABI) against the
float64 oracle (sequential recurrence; direct causal sum on small cases).
Same bar as the DLR path: relative L2 <= 1e-5, max |err| <= 1e-4 RMS."""
import numpy as np
import pytest

import oracle
from long_convolution_sequence_amd import binding as bd
from long_convolution_sequence_amd import inputs

from test_gpu_parity import assert_close, say, _torch

pytestmark = pytest.mark.gpu


METHODS = {"scan": bd.S5_SCAN, "fft": bd.S5_FFT, "fused": bd.S5_FUSED}
ALL = ["scan", "fft", "fused"]


def fused_ok(H, P, L):
    """The shapes the fused form takes (P <= 128, H <= 256, H L <= 2^29)."""
    return P <= 128 and H <= 256 and H * L <= 1 << 29


def run_s5(x, method="scan"):
    torch = _torch()
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in x.items()}
    y = bd.s5_forward(t["u"], t["lam"], t["Bbar"], t["C"], t["D"], method=METHODS[method])
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("method", ALL)
def test_s5_workload_full_size(method):
    c = inputs.config("s5_mimo")
    say("case: s5 workload B=%d H=%d P=%d L=%d method=%s" % (c["B"], c["H"], c["P"], c["L"],
                                                            method))
    x = inputs.inputs_for(c)
    y = run_s5(x, method)
    ref = oracle.s5_recurrence(x["u"], x["lam"], x["Bbar"], x["C"], x["D"])
    assert_close(y, ref, "s5/full")
    refp = oracle.s5_direct_prefix(x["u"], x["lam"], x["Bbar"], x["C"], x["D"], 256)
    assert_close(y[..., :256], refp, "s5/prefix-direct")


S5_EDGE = [
    # (B, H, P, L)
    (1, 1, 1, 1), (1, 1, 1, 7), (3, 2, 1, 33), (2, 3, 5, 100), (1, 6, 3, 4096),
    (2, 70, 5, 130), (3, 5, 40, 257), (1, 4, 2, 5000), (2, 64, 32, 1024), (1, 300, 33, 96),
    # contractions over several 256-deep k chunks and several 256-row blocks,
    # ragged row counts inside a wave's 64 rows, ragged time tail
    (1, 600, 140, 3001), (2, 72, 300, 515),
    # more than 1024 input channels: the fragments packed without LDS staging
    (1, 1100, 8, 70),
    # the fused form at its limits (P = 128, H = 256), many segments with a
    # ragged last tile; one segment per row (B >= 256); odd P and H; P not a
    # multiple of 32 (a wave's rows past the packed Bbar); just past the fused
    # limit in P
    (1, 256, 128, 20000), (2, 256, 127, 4099), (260, 6, 5, 150), (4, 17, 128, 300),
    (3, 100, 48, 700), (1, 8, 129, 500),
]


@pytest.mark.parametrize("method", ALL)
@pytest.mark.parametrize("shape", S5_EDGE, ids=["B%dH%dP%dL%d" % s for s in S5_EDGE])
def test_s5_edge_shapes(shape, method):
    B, H, P, L = shape
    say("case: s5 edge B=%d H=%d P=%d L=%d method=%s" % (shape + (method,)))
    x = inputs.s5_inputs(B, H, P, L, seed=500 + H + P + L)
    if method == "fft" and L > 16384:  # past the convolution view's circle
        with pytest.raises(bd.DSSMError, match="L <= 16384"):
            run_s5(x, method)
        return
    if method == "fused" and not fused_ok(H, P, L):  # past the fused form's limits
        with pytest.raises(bd.DSSMError, match="fused S5 form needs"):
            run_s5(x, method)
        return
    y = run_s5(x, method)
    ref = oracle.s5_recurrence(x["u"], x["lam"], x["Bbar"], x["C"], x["D"])
    assert_close(y, ref, "s5/edge")
    if L <= 300:
        refd = oracle.s5_direct_prefix(x["u"], x["lam"], x["Bbar"], x["C"], x["D"], L)
        assert_close(y, refd, "s5/edge/direct")


@pytest.mark.parametrize("method", ALL)
def test_s5_reduces_to_dlr_bank_on_device(method):
    """P = H, Bbar = I, C = diag(w): the S5 layer equals H scalar DLRs; the
    device S5 path must agree with the device DLR paths on it."""
    torch = _torch()
    H, L, B = 4, 3000, 2
    rng = np.random.default_rng(9)
    lam = np.exp(-rng.uniform(0.001, 0.05, H) + 1j * rng.uniform(-3, 3, H)).astype(np.complex64)
    w = (rng.normal(size=H) + 1j * rng.normal(size=H)).astype(np.complex64)
    D = rng.normal(size=H).astype(np.float32)
    u = rng.normal(size=(B, H, L)).astype(np.float32)
    say("case: s5 reduction to DLR bank method=%s" % method)
    y = run_s5(dict(u=u, lam=lam, Bbar=np.eye(H, dtype=np.complex64), C=np.diag(w).astype(np.complex64), D=D),
               method)
    ref = oracle.s5_recurrence(u, lam, np.eye(H), np.diag(w), D)
    assert_close(y, ref, "s5/reduction")


# Magnitudes far from 1.  y is linear in u jointly with nothing else scaled
# apart from D u and C x together, and Bbar -> 2^k Bbar with C -> 2^-k C leaves y
# unchanged; power-of-two factors scale float32 values exactly.
S5_MAGS = [("u", -70), ("u", 60), ("BC", 40), ("BC", -40)]


@pytest.mark.parametrize("method", ALL)
@pytest.mark.parametrize("what,k", S5_MAGS, ids=["%s2^%d" % m for m in S5_MAGS])
def test_s5_magnitudes(what, k, method):
    B, H, P, L = 2, 40, 24, 2000
    say("case: s5 magnitudes %s x 2^%d method=%s" % (what, k, method))
    x = inputs.s5_inputs(B, H, P, L, seed=717)
    ref = oracle.s5_recurrence(x["u"], x["lam"], x["Bbar"], x["C"], x["D"])
    xs = dict(x)
    if what == "u":
        xs["u"] = np.ldexp(x["u"], k).astype(np.float32)
        ref = ref * np.ldexp(1.0, k)
    else:
        xs["Bbar"] = (x["Bbar"] * np.float32(np.ldexp(1.0, k))).astype(np.complex64)
        xs["C"] = (x["C"] * np.float32(np.ldexp(1.0, -k))).astype(np.complex64)
    y = run_s5(xs, method)
    assert np.all(np.isfinite(y))
    assert_close(y, ref, "s5/magnitudes")


@pytest.mark.parametrize("method", ALL)
def test_s5_timed_matches_untimed(method):
    torch = _torch()
    x = inputs.s5_inputs(2, 24, 9, 3000, seed=17)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in x.items()}
    say("case: s5 timed variant B=2 H=24 P=9 L=3000 method=%s" % method)
    m = METHODS[method]
    y0 = bd.s5_forward(t["u"], t["lam"], t["Bbar"], t["C"], t["D"], method=m)
    hip = bd.HipEvents()
    evs = hip.create(8)
    y1 = bd.s5_forward(t["u"], t["lam"], t["Bbar"], t["C"], t["D"], events=evs, method=m)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    for k in range(4):
        assert hip.ms(evs[2 * k], evs[2 * k + 1]) > 0.0
    hip.destroy(evs)


@pytest.mark.parametrize("method", ALL)
def test_s5_empty_is_noop(method):
    torch = _torch()
    x = inputs.s5_inputs(1, 3, 2, 8, seed=1)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in x.items()}
    y = bd.s5_forward(torch.zeros(0, 3, 8, device="cuda"), t["lam"], t["Bbar"], t["C"], t["D"],
                      method=METHODS[method])
    torch.cuda.synchronize()
    assert y.shape == (0, 3, 8)
