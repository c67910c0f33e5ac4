"""Seeded synthetic inputs for the diagonal-SSM forward map.

This module only draws random numbers and lays them out; it holds none of the
forward map's arithmetic.  It is the one module that both the float64 oracle's
tests and the HIP path's tests, smoke check and benchmark use, so that both
sides consume bit-identical float32 inputs.

Recipe (every value is drawn in float64 from numpy's PCG64 with the stated
seed, in the stated order, and cast once to float32 / complex64):

DLR workloads -- the initialisation of "Simplifying and Understanding State
Space Models with Diagonal Linear RNNs", section 2: for each direction d:
  1. r ~ U(ln 5e-4, ln 0.5) over [H, N];  log_re = sqrt(e^r / 2) * re_scale
  2. log_im = 2*pi*n/N for n = 0..N-1, the same for every channel
  3. W.real ~ N(0, 1/N^2) over [H, N], then W.imag likewise
  4. D ~ N(0, 1) over [H]
then u ~ N(0, 1) over [B, H, L].

S5 workload -- "Simplified State Space Layers for Sequence Modeling", section 3
parameter shapes; timescales log-uniform in [1e-3, 1e-1] as in the step
initialiser of "The Annotated S4", Part 1, "An SSM neural network":
  1. ln dt ~ U(ln 1e-3, ln 1e-1) over [P];  lam_p = exp(dt_p (-0.5 + i pi p))
  2. Bbar.real, then Bbar.imag, each ~ N(0, 1/(2H)) over [P, H]
  3. C.real, then C.imag, each ~ N(0, 1/(2H)) over [H, P]
  4. D ~ N(0, 1) over [H]
  5. u ~ N(0, 1) over [B, H, L].

Synthetic N(0, 1) sequences stand in for the pages' datasets (Long Range
Arena, Speech Commands, PG-19, the synthetic tasks), which are not used.
"""

import numpy as np

# The five workloads: the lengths follow the pages' workloads (1024 = the
# image-length LRA size, 4096 and 16K = the synthetic-task lengths, 16K = the
# Path-X scale).
CONFIGS = [
    dict(name="tiny", kind="dlr", B=1, H=4, N=16, L=256, bidirectional=False,
         re_scale=1.0, seed=0),
    dict(name="image_length", kind="dlr", B=16, H=256, N=64, L=1024,
         bidirectional=False, re_scale=1.0, seed=1),
    dict(name="bidirectional", kind="dlr", B=8, H=256, N=64, L=4096,
         bidirectional=True, re_scale=1.0, seed=2),
    dict(name="long_sequence", kind="dlr", B=4, H=128, N=64, L=16384,
         bidirectional=False, re_scale=0.1, seed=3),
    dict(name="s5_mimo", kind="s5", B=4, H=256, P=128, L=16384, seed=4),
]


def config(name_or_index):
    """Return a copy of a workload description by name or index."""
    if isinstance(name_or_index, int):
        return dict(CONFIGS[name_or_index])
    for c in CONFIGS:
        if c["name"] == name_or_index:
            return dict(c)
    raise KeyError(name_or_index)


def dlr_inputs(B, H, N, L, bidirectional=False, seed=0, re_scale=1.0):
    """Seeded DLR parameters and input, float32 / complex64 numpy arrays.

    Returns a dict with u [B,H,L] f32, log_re [ndir,H,N] f32,
    log_im [ndir,H,N] f32, W [ndir,H,N] c64, D [ndir,H] f32.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    ndir = 2 if bidirectional else 1
    log_re = np.empty((ndir, H, N))
    log_im = np.empty((ndir, H, N))
    W = np.empty((ndir, H, N), dtype=np.complex128)
    D = np.empty((ndir, H))
    im_row = 2.0 * np.pi * np.arange(N) / N
    for d in range(ndir):
        r = rng.uniform(np.log(5e-4), np.log(0.5), size=(H, N))
        log_re[d] = np.sqrt(np.exp(r) / 2.0) * re_scale
        log_im[d] = im_row[None, :]
        w_re = rng.normal(0.0, 1.0 / N, size=(H, N))
        w_im = rng.normal(0.0, 1.0 / N, size=(H, N))
        W[d] = w_re + 1j * w_im
        D[d] = rng.normal(0.0, 1.0, size=H)
    u = rng.normal(0.0, 1.0, size=(B, H, L))
    return dict(
        u=u.astype(np.float32),
        log_re=log_re.astype(np.float32),
        log_im=log_im.astype(np.float32),
        W=W.astype(np.complex64),
        D=D.astype(np.float32),
    )


def s5_inputs(B, H, P, L, seed=4):
    """Seeded S5 parameters and input.

    Returns a dict with u [B,H,L] f32, lam [P] c64, Bbar [P,H] c64,
    C [H,P] c64, D [H] f32.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    log_dt = rng.uniform(np.log(1e-3), np.log(1e-1), size=P)
    dt = np.exp(log_dt)
    lam = np.exp(dt * (-0.5 + 1j * np.pi * np.arange(P)))
    s = np.sqrt(1.0 / (2.0 * H))
    b_re = rng.normal(0.0, s, size=(P, H))
    b_im = rng.normal(0.0, s, size=(P, H))
    c_re = rng.normal(0.0, s, size=(H, P))
    c_im = rng.normal(0.0, s, size=(H, P))
    D = rng.normal(0.0, 1.0, size=H)
    u = rng.normal(0.0, 1.0, size=(B, H, L))
    return dict(
        u=u.astype(np.float32),
        lam=lam.astype(np.complex64),
        Bbar=(b_re + 1j * b_im).astype(np.complex64),
        C=(c_re + 1j * c_im).astype(np.complex64),
        D=D.astype(np.float32),
    )


def inputs_for(cfg):
    """Inputs for a workload dict from CONFIGS (or one shaped like it)."""
    if cfg["kind"] == "dlr":
        return dlr_inputs(cfg["B"], cfg["H"], cfg["N"], cfg["L"],
                          cfg.get("bidirectional", False), cfg.get("seed", 0),
                          cfg.get("re_scale", 1.0))
    return s5_inputs(cfg["B"], cfg["H"], cfg["P"], cfg["L"], cfg.get("seed", 4))


def dlr_state(B, H, N, seed=0, scale=3.0):
    """Seeded initial state for the stateful (streaming) forward: x [B,H,N]
    complex64, real then imaginary parts ~ N(0, scale^2 / 2) (|x|^2 has mean
    scale^2, the order of the states a N(0,1) input drives)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    sd = scale / np.sqrt(2.0)
    re = rng.normal(0.0, sd, size=(B, H, N))
    im = rng.normal(0.0, sd, size=(B, H, N))
    return (re + 1j * im).astype(np.complex64)


def s5_tv_inputs(B, H, P, L, seed=4, step_range=(0.5, 1.5)):
    """Seeded continuous-time S5 parameters, per-step step sizes and input.

    Returns a dict with u [B,H,L] f32, lam_c [P] c64 (-0.5 + i pi p),
    delta [P] f32 (log-uniform in [1e-3, 1e-1]), Bt [P,H] c64, C [H,P] c64,
    D [H] f32 and step [B,L] f32 (uniform in step_range: irregular sampling
    around the nominal step).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    log_dt = rng.uniform(np.log(1e-3), np.log(1e-1), size=P)
    lam_c = -0.5 + 1j * np.pi * np.arange(P)
    s = np.sqrt(1.0 / (2.0 * H))
    b_re = rng.normal(0.0, s, size=(P, H))
    b_im = rng.normal(0.0, s, size=(P, H))
    c_re = rng.normal(0.0, s, size=(H, P))
    c_im = rng.normal(0.0, s, size=(H, P))
    D = rng.normal(0.0, 1.0, size=H)
    u = rng.normal(0.0, 1.0, size=(B, H, L))
    step = rng.uniform(step_range[0], step_range[1], size=(B, L))
    return dict(
        u=u.astype(np.float32),
        lam_c=lam_c.astype(np.complex64),
        delta=np.exp(log_dt).astype(np.float32),
        Bt=(b_re + 1j * b_im).astype(np.complex64),
        C=(c_re + 1j * c_im).astype(np.complex64),
        D=D.astype(np.float32),
        step=step.astype(np.float32),
    )
