"""Float64 oracle for the diagonal linear RNN (DLR) forward map.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Source: "Simplifying and Understanding State Space Models with Diagonal Linear
RNNs", section 2.  The page's display equations were lost in extraction; what
survives, and what this module follows, is:

* the parameterisation  Lambda = exp(-(log Lambda)_re^2 + i (log Lambda)_im)
  (section 2, paragraph on parameterising Lambda);
* the kernel  K_j = sum_{i} w_i lambda_i^j  and the convolution view
  y_k = sum_{j=0}^{k} K_j u_{k-j}  (section 2, the vanishing-gradient paragraph
  and the DFT remark  K = (<w, Lambda^k>)_{0<=k<L});
* the real cast  y_k = sum_{j=0}^{k} Re(K_j) u_{k-j}  (section 2, first
  paragraph);
* the bidirectional form as the sum of two independent DLRs, one per direction
  (section 2, bidirectionality paragraph).

Readings where the page is silent:

* the recurrence is  x_k = Lambda x_{k-1} + 1 u_k,  x_{-1} = 0,
  y_k = Re <w, x_k>  -- the only recurrence with unit input weights whose
  impulse response is the printed K_j; the zero initial state follows "The
  Annotated S4", Part 1, "Training SSMs: the convolutional representation";
* <w, Lambda^k> is the plain (non-conjugating) sum sum_i w_i lambda_i^k;
* a real feed-through  D u_k  is added, as in the SSM layer of "The Annotated
  S4", Part 1, "An SSM neural network" (convolution plus D times the input);
* each direction of the bidirectional form is a complete DLR with its own j=0
  tap and its own D; the backward DLR runs on the time-reversed input and its
  output is reversed back.

Layouts (last index fastest):
  u            [B, H, L]   real
  log_re       [ndir, H, N] real      (ndir = 2 if bidirectional else 1)
  log_im       [ndir, H, N] real
  W            [ndir, H, N] complex
  D            [ndir, H]    real
All inputs are promoted exactly to float64 / complex128 before any arithmetic.
"""

import numpy as np


def _real64(x):
    return np.asarray(x).astype(np.float64)


def _cplx128(x):
    return np.asarray(x).astype(np.complex128)


def dlr_lambda(log_re, log_im):
    """lambda = exp(-(log_re)^2 + i*log_im), elementwise, in complex128.

    DLR page, section 2 (parameterisation of Lambda): |lambda| = exp(-re^2) <= 1
    and lambda is periodic in the imaginary log with period 2*pi.
    """
    re = _real64(log_re)
    im = _real64(log_im)
    return np.exp(-re * re + 1j * im)


def dlr_kernel(log_re, log_im, W, L):
    """K_j = sum_n W_n lambda_n^j for 0 <= j < L (complex128).

    DLR page, section 2: K = (<w, Lambda^k>)_{0<=k<L}.  The power lambda^j is
    taken as exp(j * log lambda) with log lambda = -re^2 + i*im, so no error
    accumulates along j.

    Shapes: log_re, log_im, W are [..., N]; the result is [..., L].
    """
    re = _real64(log_re)
    im = _real64(log_im)
    w = _cplx128(W)
    lead = re.shape[:-1]
    n = re.shape[-1]
    log_lam = (-re * re + 1j * im).reshape(-1, n)
    w = w.reshape(-1, n)
    j = np.arange(L, dtype=np.float64)
    out = np.empty((log_lam.shape[0], L), dtype=np.complex128)
    for c in range(log_lam.shape[0]):
        powers = np.exp(j[:, None] * log_lam[c][None, :])  # [L, N]: lambda_n^j
        out[c] = powers @ w[c]
    return out.reshape(lead + (L,))


def dlr_kernel_cast(log_re, log_im, W, L, cast="re"):
    """The real kernel the convolution applies, from K = dlr_kernel(...):

    * cast "re":   Re K_j  (DLR page, section 2: the real cast of the kernel);
    * cast "prod": Re K_j * Im K_j  (DLR page, section 2.1: the DLR-prod cast,
      used in the Shift experiments of section 3).

    Shapes as dlr_kernel; the result is real [..., L].
    """
    K = dlr_kernel(log_re, log_im, W, L)
    if cast == "re":
        return K.real
    if cast == "prod":
        return K.real * K.imag
    raise ValueError("cast must be 're' or 'prod'")


def dlr_direct(u, log_re, log_im, W, D, bidirectional=False, cast="re"):
    """DLR layer output by the direct O(L^2) causal sum, float64.

    y[b,h,k] = sum_{j=0}^{k} Kc_f[h,j] u[b,h,k-j]
             (+ sum_{j=0}^{L-1-k} Kc_b[h,j] u[b,h,k+j]   if bidirectional)
             + (D_f[h] (+ D_b[h])) u[b,h,k],
    with Kc the cast kernel of dlr_kernel_cast (Re K by default).

    The sums are done by numpy.convolve (a direct, non-FFT method) on each
    channel and truncated to the first L outputs; the backward term convolves
    the reversed input and reverses the result.
    """
    u = _real64(u)
    Bsz, H, L = u.shape
    ndir = 2 if bidirectional else 1
    re = _real64(log_re)
    if re.shape[0] != ndir:
        raise ValueError("parameter leading dimension must be ndir")
    D = _real64(D)
    y = u * D.sum(axis=0)[None, :, None]
    for d in range(ndir):
        for h in range(H):
            k = dlr_kernel_cast(re[d, h], _real64(log_im)[d, h], _cplx128(W)[d, h], L, cast)
            for b in range(Bsz):
                if d == 0:
                    y[b, h] += np.convolve(u[b, h], k)[:L]
                else:
                    y[b, h] += np.convolve(u[b, h][::-1], k)[:L][::-1]
    return y


def dlr_recurrence(u, log_re, log_im, W, D, bidirectional=False):
    """DLR layer output by the sequential recurrence, float64.

    x_k = lambda * x_{k-1} + u_k (every mode gets the input), x_{-1} = 0,
    y_k = Re(sum_n W_n x_{k,n}) + D u_k.  The backward direction of the
    bidirectional form runs the same recurrence over k = L-1, ..., 0.
    """
    u = _real64(u)
    Bsz, H, L = u.shape
    ndir = 2 if bidirectional else 1
    lam = dlr_lambda(log_re, log_im)  # [ndir, H, N]
    if lam.shape[0] != ndir:
        raise ValueError("parameter leading dimension must be ndir")
    w = _cplx128(W)
    D = _real64(D)
    y = u * D.sum(axis=0)[None, :, None]
    for d in range(ndir):
        x = np.zeros((Bsz, H, lam.shape[-1]), dtype=np.complex128)
        order = range(L) if d == 0 else range(L - 1, -1, -1)
        for k in order:
            x = lam[d][None] * x + u[:, :, k, None]
            y[:, :, k] += (x * w[d][None]).sum(axis=-1).real
    return y


def dlr_recurrence_state(u, log_re, log_im, W, D, x0=None):
    """One-direction DLR forward from a given initial state, float64.

    The recurrence of dlr_recurrence with x_{-1} = x0 instead of zero:
      x_k = lambda * x_{k-1} + u_k,  y_k = Re(sum_n W_n x_{k,n}) + D u_k,
    returning (y [B,H,L], x_{L-1} [B,H,N] complex) -- the state a later call
    continues from.  This is the recurrent (RNN) view run in chunks ("The
    Annotated S4", Part 1, "Discrete-time SSM: the recurrent representation":
    the state carries everything the past contributes), and with x0 = 0 it
    is dlr_recurrence.  With L = 0 the state passes through unchanged.
    x0 is [B, H, N] complex (None = zero).
    """
    u = _real64(u)
    Bsz, H, L = u.shape
    lam = dlr_lambda(log_re, log_im)
    if lam.shape[0] != 1:
        raise ValueError("the stateful form has one direction")
    w = _cplx128(W)[0]
    N = lam.shape[-1]
    x = np.zeros((Bsz, H, N), dtype=np.complex128) if x0 is None else _cplx128(x0).copy()
    y = u * _real64(D)[0][None, :, None]
    for k in range(L):
        x = lam[0][None] * x + u[:, :, k, None]
        y[:, :, k] += (x * w[None]).sum(axis=-1).real
    return y, x
