"""Float64 oracle for the S5-style multi-input multi-output diagonal SSM.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Source: "Simplified State Space Layers for Sequence Modeling", section 2.2 (the
linear recurrence x_k = A_bar x_{k-1} + B_bar u_k computed by a scan) and
section 3 (the S5 layer: one diagonal state of size P shared by all H inputs,
learnable B~ in C^{PxH}, C~ in C^{HxP}, diagonal real D).

Readings where the page is silent: the discrete
diagonal Lambda_bar and B_bar are given directly (no discretisation is applied
here), the initial state is zero, and the real output is Re(C~ x_k) + D * u_k
with no factor of two.

Layouts: u [B, H, L] real; lam [P] complex; Bbar [P, H] complex;
C [H, P] complex; D [H] real.  Output [B, H, L] float64.
"""

import numpy as np


def s5_recurrence(u, lam, Bbar, C, D):
    """Sequential recurrence: v_k = Bbar u_k, x_k = lam * x_{k-1} + v_k,
    y_k = Re(C x_k) + D * u_k, with x_{-1} = 0."""
    u = np.asarray(u).astype(np.float64)
    lam = np.asarray(lam).astype(np.complex128)
    Bb = np.asarray(Bbar).astype(np.complex128)
    Cc = np.asarray(C).astype(np.complex128)
    D = np.asarray(D).astype(np.float64)
    Bsz, H, L = u.shape
    P = lam.shape[0]
    x = np.zeros((Bsz, P), dtype=np.complex128)
    y = np.empty((Bsz, H, L), dtype=np.float64)
    BbT = Bb.T.copy()
    CT = Cc.T.copy()
    for k in range(L):
        uk = u[:, :, k]
        x = lam[None, :] * x + uk @ BbT
        y[:, :, k] = (x @ CT).real + D[None, :] * uk
    return y


def s5_direct_prefix(u, lam, Bbar, C, D, Lp):
    """The first Lp outputs by direct causal sums.

    x_p[k] = sum_{j=0}^{k} lam_p^j v_p[k-j] with v = Bbar u, evaluated by
    numpy.convolve on each (b, p) with the explicit powers lam_p^j =
    exp(j log lam_p); y = Re(C x) + D u.  By causality the first Lp outputs
    depend only on the first Lp inputs, so a prefix is exact.
    """
    u = np.asarray(u).astype(np.float64)[:, :, :Lp]
    lam = np.asarray(lam).astype(np.complex128)
    Bb = np.asarray(Bbar).astype(np.complex128)
    Cc = np.asarray(C).astype(np.complex128)
    D = np.asarray(D).astype(np.float64)
    Bsz, H, L = u.shape
    P = lam.shape[0]
    v = np.einsum("ph,bhl->bpl", Bb, u)
    j = np.arange(L, dtype=np.float64)
    x = np.empty((Bsz, P, L), dtype=np.complex128)
    for p in range(P):
        powers = np.exp(j * np.log(lam[p]))
        for b in range(Bsz):
            x[b, p] = np.convolve(v[b, p], powers)[:L]
    return np.einsum("hp,bpl->bhl", Cc, x).real + D[None, :, None] * u


def _expm1c(z):
    """exp(z) - 1 for complex z without cancellation near z = 0:
    (expm1(a) cos b - 2 sin^2(b/2)) + i exp(a) sin b, z = a + ib."""
    a, b = z.real, z.imag
    return (np.expm1(a) * np.cos(b) - 2.0 * np.sin(0.5 * b) ** 2) + 1j * (np.exp(a) * np.sin(b))


def s5_recurrence_tv(u, lam_c, Bt, C, D, delta, step):
    """S5 with continuous-time parameters and a step size that changes from step
    to step ("Simplified State Space Layers for Sequence Modeling", section 3:
    a diagonal continuous-time system with a learnable timescale per state,
    discretised by zero-order hold; irregularly sampled sequences are handled by
    supplying a different timescale to the discretisation at each step).

    Reading where the page is silent (its discretisation equations were lost):
    the timescale of state p at step k of batch row b is step[b, k] * delta[p]
    (a per-step time increment relative to the nominal step, scaling the
    learnt per-state timescale), and zero-order hold gives, with
    z = lam_c[p] * step[b, k] * delta[p],
        Lambda_bar = exp(z),   B_bar row p = (exp(z) - 1) / lam_c[p] * Bt[p, :]
    ((exp(z) - 1) / lam_c -> step * delta as lam_c -> 0); then
        x_k = Lambda_bar x_{k-1} + B_bar u_k,  y_k = Re(C x_k) + D * u_k,  x_{-1} = 0.

    Layouts: u [B, H, L] real; lam_c [P] complex; Bt [P, H] complex;
    C [H, P] complex; D [H] real; delta [P] real; step [B, L] real.
    """
    u = np.asarray(u).astype(np.float64)
    lam = np.asarray(lam_c).astype(np.complex128)
    Bb = np.asarray(Bt).astype(np.complex128)
    Cc = np.asarray(C).astype(np.complex128)
    D = np.asarray(D).astype(np.float64)
    dl = np.asarray(delta).astype(np.float64)
    st = np.asarray(step).astype(np.float64)
    Bsz, H, L = u.shape
    P = lam.shape[0]
    x = np.zeros((Bsz, P), dtype=np.complex128)
    y = np.empty((Bsz, H, L), dtype=np.float64)
    BbT = Bb.T.copy()
    CT = Cc.T.copy()
    zero = lam == 0
    inv = np.where(zero, 0.0, 1.0 / np.where(zero, 1.0, lam))
    for k in range(L):
        uk = u[:, :, k]
        dt = st[:, k][:, None] * dl[None, :]  # [B, P]
        z = lam[None, :] * dt
        a = np.exp(z)
        beta = np.where(zero[None, :], dt, _expm1c(z) * inv[None, :])
        x = a * x + beta * (uk @ BbT)
        y[:, :, k] = (x @ CT).real + D[None, :] * uk
    return y
