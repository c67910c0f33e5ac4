"""Float64 oracle for the gradients of the DLR layer map (vector-Jacobian
product at an output cotangent dy).

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

The map is the one of ``oracle.dlr`` (DLR page, section 2):
  y[b,h,k] = sum_{j<=k} Re K_f[h,j] u[b,h,k-j]
           (+ sum_{j<=L-1-k} Re K_b[h,j] u[b,h,k+j])  +  (D_f + D_b)[h] u[b,h,k],
  K_d[h,j] = sum_n W[d,h,n] lambda[d,h,n]^j,  lambda = exp(-log_re^2 + i log_im).
For the scalar f = sum(dy * y) the gradients follow from the chain rule on
these definitions (the DLR page prints the derivative of K with respect to
lambda in its vanishing-gradient paragraph, dK_j / dlambda = j W lambda^(j-1)):

* du: the transposed Toeplitz operator applied to dy,
  du[k] = sum_j Re K_f[j] dy[k+j] + sum_j Re K_b[j] dy[k-j] + (D_f + D_b) dy[k];
* the kernel cotangents  G_f[h,j] = sum_{b,k} dy[b,h,k] u[b,h,k-j],
  G_b[h,j] = sum_{b,k} dy[b,h,k] u[b,h,k+j]  (d f / d Re K_d[h,j]);
* dW = d f / d Re W + i d f / d Im W = sum_j G_j conj(lambda^j);
* with Z = sum_j j G_j W lambda^j:  d f / d log_re = -2 log_re Re Z,
  d f / d log_im = -Im Z  (d lambda^j / d log_re = -2 log_re j lambda^j,
  d lambda^j / d log_im = i j lambda^j);
* dD_d = sum_{b,k} dy u  (the same for both directions).
All inputs are promoted exactly to float64 / complex128.
"""

import numpy as np

from .dlr import dlr_kernel


def dlr_backward(u, dy, log_re, log_im, W, D, bidirectional=False):
    """Returns (du [B,H,L], dlog_re [ndir,H,N], dlog_im [ndir,H,N],
    dW [ndir,H,N] complex, dD [ndir,H]) for f = sum(dy * y)."""
    u = np.asarray(u).astype(np.float64)
    dy = np.asarray(dy).astype(np.float64)
    re = np.asarray(log_re).astype(np.float64)
    im = np.asarray(log_im).astype(np.float64)
    w = np.asarray(W).astype(np.complex128)
    Dd = np.asarray(D).astype(np.float64)
    Bsz, H, L = u.shape
    ndir = 2 if bidirectional else 1
    if re.shape[0] != ndir:
        raise ValueError("parameter leading dimension must be ndir")
    N = re.shape[-1]
    du = dy * Dd.sum(axis=0)[None, :, None]
    dlre = np.zeros((ndir, H, N))
    dlim = np.zeros((ndir, H, N))
    dW = np.zeros((ndir, H, N), dtype=np.complex128)
    dD = np.zeros((ndir, H))
    j = np.arange(L, dtype=np.float64)
    for d in range(ndir):
        for h in range(H):
            K = dlr_kernel(re[d, h], im[d, h], w[d, h], L).real
            G = np.zeros(L)
            for b in range(Bsz):
                if d == 0:
                    # du[k] += sum_j K[j] dy[k+j];  G[j] += sum_k dy[k] u[k-j]
                    du[b, h] += np.correlate(dy[b, h], K, mode="full")[L - 1:]
                    G += np.correlate(dy[b, h], u[b, h], mode="full")[L - 1:]
                else:
                    # du[k] += sum_j K[j] dy[k-j];  G[j] += sum_k dy[k] u[k+j]
                    du[b, h] += np.convolve(dy[b, h], K)[:L]
                    G += np.correlate(u[b, h], dy[b, h], mode="full")[L - 1:]
                dD[d, h] += float(np.dot(dy[b, h], u[b, h]))
            powers = np.exp(j[:, None] * (-re[d, h] * re[d, h] + 1j * im[d, h])[None, :])  # [L, N]
            dW[d, h] = (G[:, None] * np.conj(powers)).sum(axis=0)
            Z = w[d, h] * ((j * G)[:, None] * powers).sum(axis=0)
            dlre[d, h] = -2.0 * re[d, h] * Z.real
            dlim[d, h] = -Z.imag
    return du, dlre, dlim, dW, dD
