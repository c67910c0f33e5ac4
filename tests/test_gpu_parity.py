"""GPU parity of the HIP path against the float64 oracle, through the C ABI.

Bar (fp32 tolerance of the forward map): over the whole output tensor,
relative L2 error <= 1e-5 and max |error| <= 1e-4 * RMS(reference).  The
oracle is the sequential float64 recurrence (and, on small cases, also the
direct O(L^2) sum); the same seeded float32 inputs feed both sides.
"""
import sys

import numpy as np
import pytest

import oracle
from long_convolution_sequence_amd import binding as bd
from long_convolution_sequence_amd import inputs

pytestmark = pytest.mark.gpu

REL_L2 = 1e-5
MAX_VS_RMS = 1e-4


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = got - ref
    rms = np.sqrt(np.mean(ref ** 2))
    rel = np.linalg.norm(d.ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300)
    mx = np.max(np.abs(d)) / max(rms, 1e-300) if d.size else 0.0
    return rel, mx


def assert_close(got, ref, what):
    rel, mx = errors(got, ref)
    say("  %s: rel_l2=%.3e max/rms=%.3e" % (what, rel, mx))
    assert rel <= REL_L2, "%s rel L2 %.3e" % (what, rel)
    assert mx <= MAX_VS_RMS, "%s max/rms %.3e" % (what, mx)


def dev(x):
    torch = _torch()
    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in x.items()}


def run(path, x, bi):
    t = dev(x)
    f = bd.forward_fft if path == "fft" else bd.forward_scan
    y = f(t["u"], t["log_re"], t["log_im"], t["W"], t["D"], bidirectional=bi)
    _torch().cuda.synchronize()
    return y.cpu().numpy()


_ORACLE = {}


def oracle_rec(key, x, bi):
    if key not in _ORACLE:
        _ORACLE[key] = oracle.dlr_recurrence(x["u"], x["log_re"], x["log_im"], x["W"], x["D"], bi)
    return _ORACLE[key]


# ----------------------------------------------------------------------------
# The four DLR workloads at full size, both paths, whole-tensor comparison.
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("idx", [0, 1, 2, 3])
@pytest.mark.parametrize("path", ["fft", "scan"])
def test_workload_full_size(idx, path):
    c = inputs.config(idx)
    say("case: workload %s path=%s B=%d H=%d N=%d L=%d bi=%d" % (
        c["name"], path, c["B"], c["H"], c["N"], c["L"], c["bidirectional"]))
    x = inputs.inputs_for(c)
    y = run(path, x, c["bidirectional"])
    ref = oracle_rec(c["name"], x, c["bidirectional"])
    assert_close(y, ref, "%s/%s" % (c["name"], path))


def test_tiny_workload_against_direct_sum():
    c = inputs.config(0)
    x = inputs.inputs_for(c)
    ref = oracle.dlr_direct(x["u"], x["log_re"], x["log_im"], x["W"], x["D"], False)
    for path in ("fft", "scan"):
        say("case: tiny vs direct, path=%s" % path)
        assert_close(run(path, x, False), ref, "tiny/%s/direct" % path)


# ----------------------------------------------------------------------------
# Kernel generator
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("idx", [0, 1, 2, 3])
def test_generator(idx):
    torch = _torch()
    c = inputs.config(idx)
    say("case: generator %s" % c["name"])
    x = inputs.inputs_for(c)
    t = dev(x)
    K = bd.gen_kernel(t["log_re"], t["log_im"], t["W"], c["L"], complex_out=True)
    Kr = bd.gen_kernel(t["log_re"], t["log_im"], t["W"], c["L"], complex_out=False)
    torch.cuda.synchronize()
    K = K.cpu().numpy()
    Kr = Kr.cpu().numpy()
    ndir, H = x["log_re"].shape[:2]
    hs = sorted(set([0, H // 3, H - 1]))
    for d in range(ndir):
        ref = oracle.dlr_kernel(x["log_re"][d, hs], x["log_im"][d, hs], x["W"][d, hs], c["L"])
        assert_close(K[d, hs].real, ref.real, "K re d=%d" % d)
        assert_close(K[d, hs].imag, ref.imag, "K im d=%d" % d)
        assert np.array_equal(Kr[d, hs], K[d, hs].real)


GEN_EDGE = [  # (H, N, L, W scale exponent): ragged lengths, several mode chunks, magnitudes
    (3, 8, 1, 0), (2, 16, 63, 0), (3, 100, 1001, 0), (2, 64, 4097, 0), (2, 130, 130, 0),
    (2, 64, 3000, -60), (2, 64, 3000, 60),
]


@pytest.mark.parametrize("shape", GEN_EDGE, ids=["H%dN%dL%dW2^%d" % g for g in GEN_EDGE])
def test_generator_edges(shape):
    torch = _torch()
    H, N, L, k = shape
    say("case: generator edge H=%d N=%d L=%d W x 2^%d" % shape)
    x = inputs.dlr_inputs(1, H, N, L, bidirectional=True, seed=900 + L)
    x["W"] = (x["W"] * np.float32(np.ldexp(1.0, k))).astype(np.complex64)
    t = dev(x)
    K = bd.gen_kernel(t["log_re"], t["log_im"], t["W"], L, complex_out=True)
    Kr = bd.gen_kernel(t["log_re"], t["log_im"], t["W"], L, complex_out=False)
    torch.cuda.synchronize()
    K = K.cpu().numpy()
    Kr = Kr.cpu().numpy()
    for d in range(2):
        ref = oracle.dlr_kernel(x["log_re"][d], x["log_im"][d], x["W"][d], L)
        assert_close(K[d].real, ref.real, "K re d=%d" % d)
        assert_close(K[d].imag, ref.imag, "K im d=%d" % d)
        assert np.array_equal(Kr[d], K[d].real)


def test_generator_dft_identity():
    """log_re = 0, log_im = 2 pi n / N, L = N: K = N ifft(W) (DLR page, section 2).

    The device receives float32(2 pi n / N); the map it must reproduce is the
    one those float32 values define, so parity is checked against the oracle
    on the same inputs.  The exact DFT is matched to within the phase error
    the parameter rounding itself causes (|d theta| <= 2.4e-7 rad per mode,
    times k < N), bounded by N * 1e-6 relative."""
    torch = _torch()
    for N in (16, 64, 256):
        say("case: DFT identity N=%d" % N)
        rng = np.random.default_rng(N)
        W = (rng.normal(size=(1, 1, N)) + 1j * rng.normal(size=(1, 1, N))).astype(np.complex64)
        lr = np.zeros((1, 1, N), np.float32)
        li = (2 * np.pi * np.arange(N) / N).astype(np.float32)[None, None, :]
        t = dev(dict(lr=lr, li=li, W=W))
        K = bd.gen_kernel(t["lr"], t["li"], t["W"], N, complex_out=True)
        torch.cuda.synchronize()
        got = K.cpu().numpy()[0, 0]
        ref = oracle.dlr_kernel(lr[0, 0], li[0, 0], W[0, 0], N)
        assert_close(got.real, ref.real, "dft re")
        assert_close(got.imag, ref.imag, "dft im")
        exact = N * np.fft.ifft(W[0, 0].astype(np.complex128))
        rel = np.linalg.norm(got - exact) / np.linalg.norm(exact)
        say("  vs exact DFT: rel_l2=%.3e (bound %.1e)" % (rel, N * 1e-6))
        assert rel <= N * 1e-6


# ----------------------------------------------------------------------------
# Edge cases: ragged and tiny lengths, odd batch, mode counts, long scans.
# ----------------------------------------------------------------------------

EDGE = [
    # (B, H, N, L, bi)
    (1, 3, 8, 1, 0), (1, 3, 8, 1, 1), (3, 2, 8, 2, 0), (2, 2, 8, 15, 1), (3, 3, 8, 16, 0),
    (1, 2, 8, 17, 1), (5, 3, 16, 100, 0), (2, 2, 16, 255, 1), (3, 2, 8, 257, 0),
    (2, 3, 1, 1000, 0), (3, 2, 100, 777, 1), (2, 2, 130, 513, 0), (1, 2, 16, 4097, 1),
    (3, 2, 8, 16383, 0), (2, 1, 4, 16384, 1),
    # one direction at every transform size of the packed spectrum (M = 32 .. 8192)
    (2, 3, 8, 17, 0), (1, 2, 8, 33, 0), (2, 2, 8, 64, 0), (1, 3, 8, 129, 0), (2, 2, 8, 300, 0),
    (1, 2, 8, 2047, 0), (2, 2, 8, 2049, 0), (1, 2, 8, 5000, 0), (2, 1, 8, 8192, 0),
    # three or more row pairs per channel, several mode chunks (N = 100), ragged L
    (4, 3, 8, 1500, 0), (5, 2, 16, 3000, 0), (6, 2, 100, 2048, 0), (3, 3, 64, 9000, 0),
    (4, 2, 64, 16384, 0),
    # the chunked matrix-core scan serves N <= 64: both sides of that limit, a
    # length that leaves a partial chunk and a partial block, reversed too
    (2, 3, 64, 4159, 1), (2, 3, 65, 999, 1), (3, 2, 33, 63, 1),
    # one direction, long transforms: several mode chunks, ragged lengths, one mode
    (2, 2, 100, 6000, 0), (1, 2, 130, 4500, 0), (2, 3, 8, 4097, 0), (1, 2, 1, 16384, 0),
    # more convolution workgroups (one per row pair) than the device holds at once
    (6, 100, 8, 16384, 0), (1, 300, 8, 16384, 0),
]


@pytest.mark.parametrize("shape", EDGE, ids=["B%dH%dN%dL%dbi%d" % s for s in EDGE])
@pytest.mark.parametrize("path", ["fft", "scan"])
def test_edge_shapes(shape, path):
    B, H, N, L, bi = shape
    say("case: edge path=%s B=%d H=%d N=%d L=%d bi=%d" % (path, B, H, N, L, bi))
    x = inputs.dlr_inputs(B, H, N, L, bidirectional=bool(bi), seed=1000 + L + N)
    y = run(path, x, bool(bi))
    ref = oracle_rec(("edge",) + shape, x, bool(bi))
    assert_close(y, ref, "edge/%s" % path)
    if L <= 300:
        refd = oracle.dlr_direct(x["u"], x["log_re"], x["log_im"], x["W"], x["D"], bool(bi))
        assert_close(y, refd, "edge/%s/direct" % path)


@pytest.mark.parametrize("bi", [0, 1])
def test_scan_several_tiles(bi):
    """L beyond one tile of the scan (16384 steps) carries state between tiles."""
    B, H, N, L = 2, 2, 8, 40000
    say("case: scan multi-tile L=%d bi=%d" % (L, bi))
    x = inputs.dlr_inputs(B, H, N, L, bidirectional=bool(bi), seed=77, re_scale=0.05)
    y = run("scan", x, bool(bi))
    ref = oracle_rec(("tiles", bi), x, bool(bi))
    assert_close(y, ref, "scan tiles")


@pytest.mark.parametrize("path", ["fft", "scan"])
def test_shift_pin_no_decay(path):
    """Shift construction (DLR page, section 3.1) with float32 parameters and no
    decay at L = 16384: stresses the phase accuracy of lambda^k."""
    N, L, r = 64, 16384, 5
    n = np.arange(N)
    x = dict(
        u=np.random.default_rng(3).normal(size=(2, 1, L)).astype(np.float32),
        log_re=np.zeros((1, 1, N), np.float32),
        log_im=(2 * np.pi * n / N).astype(np.float32)[None, None, :],
        W=(np.exp(-2j * np.pi * n * r / N) / N).astype(np.complex64)[None, None, :],
        D=np.array([[0.5]], np.float32),
    )
    say("case: shift pin path=%s" % path)
    y = run(path, x, False)
    ref = oracle_rec(("shift",), x, False)
    assert_close(y, ref, "shift/%s" % path)


# Magnitudes far from 1.  The map is linear in u and jointly in (W, D), and a
# power-of-two factor scales float32 values exactly, so the oracle of the
# scaled problem is the scaled oracle.
MAGS = [("u", -100), ("u", -20), ("u", 13), ("u", 100), ("WD", -20), ("WD", 17)]


@pytest.mark.parametrize("what,k", MAGS, ids=["%s2^%d" % m for m in MAGS])
@pytest.mark.parametrize("path", ["fft", "scan"])
def test_magnitudes(path, what, k):
    B, H, N, L = 2, 3, 64, 3000
    say("case: magnitudes path=%s %s x 2^%d" % (path, what, k))
    x = inputs.dlr_inputs(B, H, N, L, bidirectional=True, seed=515)
    ref = oracle_rec(("mag",), x, True) * np.ldexp(1.0, k)
    xs = dict(x)
    if what == "u":
        xs["u"] = np.ldexp(x["u"], k).astype(np.float32)
    else:
        xs["W"] = (x["W"] * np.float32(np.ldexp(1.0, k))).astype(np.complex64)
        xs["D"] = np.ldexp(x["D"], k).astype(np.float32)
    y = run(path, xs, True)
    assert np.all(np.isfinite(y))
    assert_close(y, ref, "magnitudes/%s" % path)


@pytest.mark.parametrize("path", ["fft", "scan"])
def test_large_states(path):
    """A near-undamped mode under a constant input of 1000: its state grows to
    about 8e6, far past the float16 range that the matrix-core operands have
    before they are scaled."""
    B, H, N, L = 1, 2, 64, 8192
    say("case: large states path=%s" % path)
    x = inputs.dlr_inputs(B, H, N, L, seed=616, re_scale=0.01)
    x["u"] = np.full((B, H, L), 1000.0, np.float32)
    ref = oracle_rec(("large",), x, False)
    y = run(path, x, False)
    assert np.all(np.isfinite(y))
    assert_close(y, ref, "large states/%s" % path)


def test_fft_and_scan_agree_and_are_deterministic():
    c = inputs.config(2)
    x = inputs.inputs_for(c)
    say("case: determinism + fft==scan on %s" % c["name"])
    a1 = run("fft", x, True)
    a2 = run("fft", x, True)
    s1 = run("scan", x, True)
    s2 = run("scan", x, True)
    assert np.array_equal(a1, a2)
    assert np.array_equal(s1, s2)
    rel, mx = errors(a1, s1)
    assert rel < 2 * REL_L2 and mx < 2 * MAX_VS_RMS


@pytest.mark.parametrize("path,nk,bi", [("fft", 2, 1), ("fft", 2, 0), ("scan", 2, 1)])
def test_timed_variants_match_and_stamp_each_kernel(path, nk, bi):
    """The timed calls give the untimed calls' bits; each stage's start/stop
    pair is a non-negative duration (the chunked scan's stage 0 has no kernel),
    the main kernel's is positive, and the pairs are ordered in time (both
    directions, and one: the spectrum's packed even/odd form)."""
    torch = _torch()
    c = dict(inputs.config("tiny"), B=3, H=8, N=16, L=2000, bidirectional=bi)
    x = inputs.inputs_for(c)
    t = dev(x)
    f = bd.forward_fft if path == "fft" else bd.forward_scan
    y0 = f(t["u"], t["log_re"], t["log_im"], t["W"], t["D"], bidirectional=bool(bi))
    hip = bd.HipEvents()
    evs = hip.create(2 * nk)
    y1 = bd.forward_timed(path, t["u"], t["log_re"], t["log_im"], t["W"], t["D"], evs,
                          bidirectional=bool(bi))
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    for k in range(nk):
        assert hip.ms(evs[2 * k], evs[2 * k + 1]) >= 0.0
        if k == nk - 1:
            assert hip.ms(evs[2 * k], evs[2 * k + 1]) > 0.0
        if k:
            assert hip.ms(evs[2 * k - 1], evs[2 * k]) >= 0.0
    hip.destroy(evs)


def test_empty_inputs_are_noops():
    torch = _torch()
    say("case: empty inputs")
    for (B, H, L) in ((0, 3, 8), (2, 0, 8), (2, 3, 0)):
        x = inputs.dlr_inputs(max(B, 1), max(H, 1), 4, max(L, 1), seed=5)
        t = dev(x)
        u = torch.zeros(B, H, L, device="cuda")
        lr, li, W, D = (t["log_re"][:, :H], t["log_im"][:, :H], t["W"][:, :H], t["D"][:, :H])
        for f in (bd.forward_fft, bd.forward_scan):
            y = f(u, lr.contiguous(), li.contiguous(), W.contiguous(), D.contiguous())
            assert y.shape == (B, H, L)
    torch.cuda.synchronize()


# ----------------------------------------------------------------------------
# The recurrence view's work split: several batch rows per workgroup (many
# rows), and the sequence cut into segments whose entering states are joined
# from a state-only pass's segment states (few rows, long sequences).
# ----------------------------------------------------------------------------

SPLIT = [  # (B, H, N, L, bi, re_scale): few rows -> segments
    (1, 4, 64, 1 << 20, 0, 0.1),         # 256 blocks of 4096 steps, 128 segments of 2
    (1, 2, 64, 1 << 19, 1, 0.1),         # both directions, 128 segments
    (2, 3, 33, 5 * 4096 * 3 + 77, 1, 1.0),  # ragged last chunk and block, one block per segment
    (1, 1, 16, 4096 * 2 + 1, 0, 1.0),    # the last segment holds one step
    (3, 2, 64, 3 * 4096, 0, 0.1),        # length a whole number of blocks
    (1, 1, 16, 1 << 20, 0, 0.1),         # 256 segments: a join quarter over 32 terms
    (1, 1, 8, 600000, 1, 1.0),           # 147 segments, both directions, ragged
]


@pytest.mark.parametrize("shape", SPLIT, ids=["B%dH%dN%dL%dbi%d" % s[:5] for s in SPLIT])
def test_scan_sequence_split(shape):
    B, H, N, L, bi, rs = shape
    say("case: scan split B=%d H=%d N=%d L=%d bi=%d" % shape[:5])
    x = inputs.dlr_inputs(B, H, N, L, bidirectional=bool(bi), seed=1300 + L % 1000, re_scale=rs)
    y = run("scan", x, bool(bi))
    ref = oracle.dlr_recurrence(x["u"], x["log_re"], x["log_im"], x["W"], x["D"], bool(bi))
    assert_close(y, ref, "scan/split")


ROWS = [  # (B, H, N, L, bi): many rows -> several batch rows per workgroup, ragged groups;
    # rows of at most 16 chunks (L <= 1024) four to a block, of at most 32 two to a block,
    # with empty row slots, both directions, and lengths off the 16-byte grid
    (7, 300, 16, 500, 0), (9, 130, 64, 4096, 1), (16, 80, 8, 1000, 1), (5, 230, 64, 70, 0),
    (7, 160, 32, 2000, 0), (6, 200, 64, 1537, 1),
]


@pytest.mark.parametrize("shape", ROWS, ids=["B%dH%dN%dL%dbi%d" % s for s in ROWS])
def test_scan_rows_per_workgroup(shape):
    B, H, N, L, bi = shape
    say("case: scan rows per workgroup B=%d H=%d N=%d L=%d bi=%d" % shape)
    x = inputs.dlr_inputs(B, H, N, L, bidirectional=bool(bi), seed=1400 + H)
    y = run("scan", x, bool(bi))
    ref = oracle.dlr_recurrence(x["u"], x["log_re"], x["log_im"], x["W"], x["D"], bool(bi))
    assert_close(y, ref, "scan/rows")
    assert_close(run("fft", x, bool(bi)), ref, "fft/rows")
