/*
 * dssm.h -- C ABI of libdssm.so: the forward map of a bank of H independent
 * diagonal linear RNN / diagonal state-space channels on AMD MI355X (gfx950).
 *
 * The map (DLR = "Simplifying and Understanding State Space Models with
 * Diagonal Linear RNNs", section 2):
 *
 *   lambda[h,n] = exp(-log_re[h,n]^2 + i*log_im[h,n])        (parameterisation)
 *   K[h,j]      = sum_n W[h,n] * lambda[h,n]^j,  0 <= j < L    (kernel)
 *   y[b,h,k]    = sum_{j=0}^{k} Re(K[h,j]) u[b,h,k-j] + D[h] u[b,h,k]
 *
 * The real cast of the kernel is the DLR page's (section 2, first paragraph);
 * the D feed-through is the SSM layer of "The Annotated S4" (Part 1, "An SSM
 * neural network").  With bidirectional = 1 a second, independent DLR runs on
 * the time-reversed input and its reversed output is added (DLR page,
 * section 2, bidirectional paragraph):
 *
 *   y[b,h,k] += sum_{j=0}^{L-1-k} Re(K_b[h,j]) u[b,h,k+j] + D_b[h] u[b,h,k]
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Layouts are row-major, last index fastest.  ndir = 1 + bidirectional.
 * - Every array argument is a DEVICE pointer (memory of the current HIP
 *   device), float32, 16-byte aligned.  Complex values are interleaved
 *   (re, im) float32 pairs, i.e. torch.complex64 / view_as_real layout.
 * - `stream` is a hipStream_t (NULL = the legacy default stream).  Every call
 *   only enqueues kernels on `stream` and returns; it never synchronises.
 * - Ownership: the caller allocates and owns every buffer, including the
 *   workspace `ws` of at least the size reported by dssm_workspace_size().
 *   The library allocates no device memory and keeps no pointer after return
 *   (the one exception: the fixed per-device scratch array of
 *   dssm_forward_fft_noalloc, part of the library's device image).
 *   Outputs must not alias inputs.  The workspace may be reused by later calls
 *   on the same stream; concurrent calls need distinct workspaces.
 * - Errors: every call returns a dssm_status.  Arguments are validated on the
 *   host before anything is launched, so an error return means nothing was
 *   enqueued (except DSSM_ERR_HIP, reported by the launch itself).  No call
 *   aborts or throws.  dssm_last_error() gives a per-thread message.
 * - Thread safety: calls may be made from several threads; the only mutable
 *   library state is the per-thread last-error message and the per-device
 *   scratch address of dssm_forward_fft_noalloc (looked up once under a
 *   lock; see that call for the race between overlapping calls). 
 */
#ifndef DSSM_H
#define DSSM_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSSM_VERSION 10300 /* major*10000 + minor*100 + patch */

/* Status codes. */
typedef enum {
  DSSM_OK = 0,
  DSSM_ERR_INVALID_ARG = -1,  /* null pointer, bad dimension or flag, misaligned pointer */
  DSSM_ERR_UNSUPPORTED = -2,  /* valid but outside what this library computes */
  DSSM_ERR_WORKSPACE = -3,    /* ws_bytes smaller than dssm_workspace_size() */
  DSSM_ERR_HIP = -4           /* a HIP launch reported an error */
} dssm_status;

/* Operations, for dssm_workspace_size(). */
typedef enum {
  DSSM_OP_GEN = 0,     /* dssm_gen_kernel */
  DSSM_OP_FFT = 1,     /* dssm_forward_fft */
  DSSM_OP_SCAN = 2,    /* dssm_forward_scan */
  DSSM_OP_BWD = 3,     /* dssm_backward */
  DSSM_OP_S5_SCAN = 4,  /* dssm_s5_forward, method DSSM_S5_SCAN (shape N = state size P) */
  DSSM_OP_S5_FFT = 5,   /* dssm_s5_forward, method DSSM_S5_FFT (shape N = state size P) */
  DSSM_OP_S5_FUSED = 6  /* dssm_s5_forward, method DSSM_S5_FUSED (shape N = state size P) */
} dssm_op;

/* How dssm_s5_forward runs the state recurrence ("Simplified State Space
 * Layers for Sequence Modeling", section 2.3: the recurrent mode and the
 * convolution mode of a linear time-invariant system give the same map). */
typedef enum {
  DSSM_S5_SCAN = 0, /* the recurrence as a parallel scan over time */
  DSSM_S5_FFT = 1,  /* per state, the convolution with lambda_p^j by FFT */
  DSSM_S5_FUSED = 2 /* projections and recurrence in one pass over u (v, x on chip) */
} dssm_s5_method;

/* How the complex kernel K is cast to the real kernel the convolution applies
 * (DLR page, section 2 for the real cast; section 2.1 for DLR-prod). */
typedef enum {
  DSSM_CAST_RE = 0,    /* Re K_j */
  DSSM_CAST_RE_IM = 1  /* Re K_j * Im K_j (DLR-prod) */
} dssm_cast;

/* Shape of a DLR bank: batch B, channels H, modes N, length L. */
typedef struct {
  int B, H, N, L;
  int bidirectional; /* 0 or 1 */
} dssm_shape;

/* DLR parameters (device pointers, float32).
 *   log_re [ndir, H, N]      (log Lambda)_re
 *   log_im [ndir, H, N]      (log Lambda)_im
 *   W      [ndir, H, N, 2]   complex output weights w
 *   D      [ndir, H]         real feed-through
 * Direction 0 is left-to-right, direction 1 (if bidirectional) right-to-left. */
typedef struct {
  const float* log_re;
  const float* log_im;
  const float* W;
  const float* D;
} dssm_dlr_params;

/* Gradients of the DLR parameters (device pointers, float32, 16-byte
 * aligned), laid out as the parameters of dssm_dlr_params:
 *   dlog_re [ndir, H, N], dlog_im [ndir, H, N], dW [ndir, H, N, 2]
 *   (d f / d Re W, d f / d Im W), dD [ndir, H]. */
typedef struct {
  float* dlog_re;
  float* dlog_im;
  float* dW;
  float* dD;
} dssm_dlr_grads;

/* Library version (DSSM_VERSION of the build). */
int dssm_version(void);

/* Static text for a status code. */
const char* dssm_status_string(int status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* dssm_last_error(void);

/* Bytes of workspace needed by `op` for shape `s` (host only; launches
 * nothing).  Returns DSSM_ERR_INVALID_ARG / DSSM_ERR_UNSUPPORTED exactly
 * when the corresponding compute call would.  Limits common to the DLR calls:
 * 1 <= N <= 4096, H (1 + bidirectional) <= 65535, B H L <= 2^40 and
 * B H (1 + bidirectional) <= 2^31 - 1.  For DSSM_OP_S5_SCAN / _FFT / _FUSED
 * the shape is read as the S5 shape {B, H, P = N, L, bidirectional} and the
 * result is dssm_s5_workspace_size() of that method. */
int dssm_workspace_size(int op, const dssm_shape* s, size_t* bytes);

/* Kernel generation: K[d,h,j] = sum_n W[d,h,n] lambda[d,h,n]^j for 0 <= j < L
 * (DLR page, section 2: K = (<w, Lambda^k>)_{0<=k<L}).
 *   complex_out = 0: K is [ndir, H, L] float32 holding Re K.
 *   complex_out = 1: K is [ndir, H, L, 2] float32 holding K (re, im).
 * Powers are formed from lambda^r (r < 64) and anchors W lambda^(64q) that
 * are computed in float64 and rounded once to float32; the sum over modes is
 * a matrix-core contraction on split operands (fp16 hi + lo, three products,
 * float32 accumulation; the anchors scaled by a power of two first), ~22
 * significant bits per operand.  B and p->D are ignored (D may be NULL); the
 * workspace size is 0 (ws may be NULL).
 * Requires 1 <= N <= 4096, 1 <= L <= 2^24. */
int dssm_gen_kernel(const dssm_dlr_params* p, const dssm_shape* s, int complex_out,
                    float* K, void* ws, size_t ws_bytes, void* stream);

/* The real kernel a cast applies: K [ndir, H, L] float32 holding Re K_j
 * (cast = DSSM_CAST_RE, as dssm_gen_kernel with complex_out = 0) or
 * Re K_j * Im K_j (cast = DSSM_CAST_RE_IM, the DLR-prod kernel of the DLR page,
 * section 2.1), K as in dssm_gen_kernel.  Any other cast returns
 * DSSM_ERR_INVALID_ARG.  Other arguments and limits as dssm_gen_kernel. */
int dssm_gen_kernel_cast(const dssm_dlr_params* p, const dssm_shape* s, int cast, float* K,
                         void* ws, size_t ws_bytes, void* stream);

/* Layer forward by the convolution view: y [B, H, L] from u [B, H, L].
 * Generates Re K, takes its spectrum on a zero-padded circle of length 2M
 * (M = the smallest power of two >= max(L, 16)), and for each channel forms
 * y = first L samples of IFFT(FFT(pad(u)) * spectrum) + D u -- the Toeplitz
 * product computed as a circulant product of size 2M (DLR page, section 2;
 * "The Annotated S4", Part 1, "Training SSMs: the convolutional
 * representation").  For bidirectional = 1 the backward kernel enters as the
 * conjugate spectrum (a correlation) and D_f + D_b multiplies u.
 * Requires L <= 16384 (the FFT is staged in one compute unit's LDS); longer L
 * returns DSSM_ERR_UNSUPPORTED (use dssm_forward_scan). */
int dssm_forward_fft(const float* u, const dssm_dlr_params* p, const dssm_shape* s,
                     float* y, void* ws, size_t ws_bytes, void* stream);

/* dssm_forward_fft without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace of dssm_forward_fft (the
 * real kernel rows and the spectrum table) lives in a device array inside the
 * library, 64 MiB per device, held by each device from the library's first
 * call on it until the process ends; the call itself allocates and frees
 * nothing.  Shapes whose workspace, dssm_workspace_size(DSSM_OP_FFT, s), is
 * larger than 64 MiB return DSSM_ERR_UNSUPPORTED before anything is
 * enqueued (for example B=4, H=128, L=16384 needs 42 MB; H=256, L=16384 needs
 * 84 MB and is refused).  Every call on one device uses that device's one
 * array: calls that overlap in time on the same device (different streams,
 * or threads) race and give wrong results; serialise them.  Results are the
 * same as dssm_forward_fft's.  Other arguments, conventions and limits as
 * dssm_forward_fft. */
int dssm_forward_fft_noalloc(const float* u, const dssm_dlr_params* p, const dssm_shape* s,
                             float* y, void* stream);

/* dssm_forward_fft with the kernel cast `cast` in place of Re K: with
 * DSSM_CAST_RE_IM each direction's convolution applies Re K_j * Im K_j (the
 * DLR-prod layer of the DLR page, sections 2.1 and 3); DSSM_CAST_RE is
 * dssm_forward_fft.  Any other cast returns DSSM_ERR_INVALID_ARG.  The
 * workspace is dssm_workspace_size(DSSM_OP_FFT, s).  DLR-prod has no
 * recurrence entry point: as a recurrence it is a DLR of N^2 modes
 * lambda_n lambda_m. */
int dssm_forward_fft_cast(const float* u, const dssm_dlr_params* p, const dssm_shape* s,
                          int cast, float* y, void* ws, size_t ws_bytes, void* stream);

/* Gradients of the layer map (the map of dssm_forward_fft / dssm_forward_scan,
 * which is the same map) for the scalar f = sum(dy * y): the input gradient
 * du [B, H, L] and the parameter gradients g (DLR page, section 2: K_j =
 * sum_n W_n lambda_n^j, lambda = exp(-log_re^2 + i log_im), dK_j / dlambda =
 * j W lambda^(j-1)).  With the kernel cotangents
 *   G_f[h,j] = sum_{b,k} dy[b,h,k] u[b,h,k-j],  G_b[h,j] = sum_{b,k} dy[b,h,k] u[b,h,k+j]:
 *   du     = the transposed layer operator applied to dy (the convolution with
 *            the conjugate spectrum: correlation with Re K_f, convolution with
 *            Re K_b, plus (D_f + D_b) dy);
 *   dW     = sum_j G_j conj(lambda^j);   with Z = sum_j j G_j W lambda^j:
 *   dlog_re = -2 log_re Re Z,  dlog_im = -Im Z;   dD_d = sum_{b,k} dy u.
 * The cotangents are lagged correlations summed over the batch in the
 * frequency domain (one transform per pair (u_b, dy_b) and half of the 2L
 * circle, one inverse per channel and half, both directions from the same
 * inverse); the sums over j run on float32 matrix products over 64-tap
 * blocks combined with float64 powers lambda^(64 q).
 * u, dy, du: [B, H, L] float32, 16-byte aligned; du must not alias u or dy.
 * Workspace: dssm_workspace_size(DSSM_OP_BWD, s).  Requires L <= 16384 (as
 * dssm_forward_fft) and B H <= 2^26.  With B = 0 or L = 0 the parameter
 * gradients are set to zero (u, dy, du, ws unused); with H = 0 nothing is
 * done. */
int dssm_backward(const float* u, const float* dy, const dssm_dlr_params* p,
                  const dssm_shape* s, float* du, const dssm_dlr_grads* g, void* ws,
                  size_t ws_bytes, void* stream);

/* Layer forward by the recurrence view: x_k = lambda x_{k-1} + u_k (x_{-1} = 0,
 * every mode driven by u), y_k = Re(sum_n W_n x_{k,n}) + D u_k; the backward
 * direction runs over k = L-1 .. 0 and is added ("The Annotated S4", Part 1,
 * "Discrete-time SSM: the recurrent representation"; the diagonal parallel
 * scan of "Simplified State Space Layers for Sequence Modeling", section 2.2).
 * For N <= 64 (and B H <= 2^24) the map is computed by chunks of 64 steps:
 * within a chunk as dense contractions on the matrix cores (the Toeplitz
 * product of the taps plus the contribution of the carried state, on split
 * fp16 operands scaled by powers of two), across chunks by the state
 * recurrence; otherwise time is split into segments, one per lane, whose
 * carries are combined with powers of lambda computed in float64.  Accepts
 * any L >= 1. */
int dssm_forward_scan(const float* u, const dssm_dlr_params* p, const dssm_shape* s,
                      float* y, void* ws, size_t ws_bytes, void* stream);

/* Streaming (stateful) forward by the recurrence view, one direction: the
 * recurrence of dssm_forward_scan continued from a given state instead of
 * zero ("The Annotated S4", Part 1, "Discrete-time SSM: the recurrent
 * representation": the state carries everything the past contributes, so a
 * sequence processed in consecutive chunks gives the outputs of the whole):
 *   x_{-1} = x (on entry),  x_k = lambda x_{k-1} + u_k,
 *   y_k = Re(sum_n W_n x_{k,n}) + D u_k,  x = x_{L-1} (on exit).
 *   x [B, H, N] complex (float32 pairs), read and then overwritten in place;
 *   it must not alias u or y.  u, y [B, H, L] as for dssm_forward_scan.
 * Requires bidirectional = 0 (a right-to-left direction needs the future:
 * DSSM_ERR_UNSUPPORTED).  L = 0 leaves x unchanged.  Workspace: the size
 * dssm_workspace_size(DSSM_OP_SCAN, s) reports.  Chunks of a long sequence
 * agree with the unsplit call within float32 rounding (the segment carries
 * are combined in a different order). */
int dssm_forward_scan_state(const float* u, const dssm_dlr_params* p, const dssm_shape* s,
                            float* x, float* y, void* ws, size_t ws_bytes, void* stream);

/* One decode step for every (b, h), the recurrent view advanced by one token
 * (the constant work per generated token that the DLR page's PG-19
 * language-modelling paragraph contrasts with attention; "The Annotated S4",
 * Part 3, "Sampling and caching": the recurrent state is the cache):
 *   x <- lambda x + u_t,  y_t = Re(sum_n W_n x_n) + D u_t.
 *   u_t, y_t [B, H] float32; x [B, H, N] complex, updated in place (no alias).
 * s->L must be 1 and s->bidirectional 0.  lambda is formed in float64 and
 * rounded once to float32 per call; a run of k steps is the float32 chain of
 * k products, so its error grows with k like any float32 recurrence.  No
 * workspace.  Requires B H <= 262140 (one wave per (b, h), four per
 * workgroup, at most 65535 workgroups); larger B H returns
 * DSSM_ERR_UNSUPPORTED. */
int dssm_step(const float* u_t, const dssm_dlr_params* p, const dssm_shape* s, float* x,
              float* y_t, void* stream);

/* ------------------------------------------------------------------------
 * S5-style multi-input multi-output diagonal SSM ("Simplified State Space
 * Layers for Sequence Modeling", section 3): one diagonal state of size P
 * shared by all H inputs,
 *   v_k = Bbar u_k,  x_k = lambda * x_{k-1} + v_k  (x_{-1} = 0),
 *   y_k = Re(C x_k) + D * u_k,
 * with the discrete lambda and Bbar given directly (no discretisation is
 * applied) and no factor 2 on the real part.  Layouts:
 *   u, y   [B, H, L] float32
 *   lambda [P, 2]    complex
 *   Bbar   [P, H, 2] complex
 *   C      [H, P, 2] complex
 *   D      [H]       float32
 * The projections are dense contractions (over H, and over 2P) on the
 * matrix cores with split operands: each float32 operand is written as an
 * fp16 hi part plus an fp16 lo part after a power-of-two scale per row (or
 * per time step), and three fp16 products (hi.hi + hi.lo + lo.hi) are
 * accumulated in float32, about 22 significant bits per operand.  The
 * state recurrence runs by `method`:
 *   DSSM_S5_SCAN: v and x in the workspace, a segmented complex scan
 *     between the projections whose carries use powers of lambda computed in
 *     float64 (section 2.2, the parallel scan);
 *   DSSM_S5_FUSED: the same recurrence with v and x never written to memory:
 *     per 64-step tile of a batch row, v = Bbar u, the tile's recurrence and
 *     y = Re(C x) + D u in one kernel; the sequence of a row is cut into
 *     segments whose entering states come from a state-only pass (the state
 *     each segment leaves from zero), joined with powers of lambda in
 *     float64.  Requires P <= 128, H <= 256 and H L <= 2^29 (otherwise
 *     DSSM_ERR_UNSUPPORTED);
 *   DSSM_S5_FFT: per state p and batch row b, the causal convolution
 *     x_p = (lambda_p^j)_j * v_p (section 2.3, the convolution mode), by a
 *     complex FFT on a zero-padded circle of length 2M (M = the smallest
 *     power of two >= max(L, 16)); the spectrum of the powers,
 *     (1 - (lambda w^m)^M) / (1 - lambda w^m) with w = exp(-i pi / M), is
 *     evaluated in float64 and rounded once.  Requires L <= 16384 (longer L:
 *     DSSM_ERR_UNSUPPORTED); its workspace adds P x 2M complex values.
 * Any other method returns DSSM_ERR_INVALID_ARG.  bidirectional = 1 is
 * DSSM_ERR_UNSUPPORTED (the pages define no bidirectional S5).
 * Requires 1 <= P <= 4096, L <= 2^24, B <= 65535.
 * ------------------------------------------------------------------------ */
typedef struct {
  int B, H, P, L;
  int bidirectional; /* must be 0 */
} dssm_s5_shape;

typedef struct {
  const float* lambda;
  const float* Bbar;
  const float* C;
  const float* D;
} dssm_s5_params;

/* Bytes of workspace dssm_s5_forward needs with `method` (host only).
 * DSSM_S5_FUSED needs only the packed projections, the segment states and
 * powers of lambda; the other methods add v and x (2 x B P L complex
 * float32). */
int dssm_s5_workspace_size(const dssm_s5_shape* s, int method, size_t* bytes);

/* Bytes of workspace dssm_s5_forward_tv needs (host only): the packed
 * projections, v and x.  Errors as dssm_s5_workspace_size. */
int dssm_s5_tv_workspace_size(const dssm_s5_shape* s, size_t* bytes);

/* y [B, H, L] from u [B, H, L] by `method` (a dssm_s5_method); same
 * conventions as the DLR calls. */
int dssm_s5_forward(const float* u, const dssm_s5_params* p, const dssm_s5_shape* s, int method,
                    float* y, void* ws, size_t ws_bytes, void* stream);

/* S5 in continuous time with a step size that changes from step to step
 * ("Simplified State Space Layers for Sequence Modeling", section 3: a
 * diagonal continuous-time system with a learnable timescale per state,
 * discretised by zero-order hold; irregularly sampled sequences are handled
 * by supplying a different timescale to the discretisation at each step).
 * The timescale of state p at step k of batch row b is step[b, k] * delta[p];
 * with z = lambda_c[p] step[b, k] delta[p]:
 *   x_k = exp(z) x_{k-1} + (exp(z) - 1) / lambda_c[p] (Btilde u_k)_p,
 *   y_k = Re(C x_k) + D u_k,   x_{-1} = 0
 * ((exp(z) - 1) / lambda_c is step delta where lambda_c = 0).  Layouts:
 *   lambda_c [P, 2] complex (continuous-time), Btilde [P, H, 2] complex,
 *   C [H, P, 2] complex, D [H] float32, delta [P] float32,
 *   step [B, L] float32 (the caller's time increments over the nominal step;
 *   0 is allowed: the state is then carried over unchanged).
 * The projections are those of dssm_s5_forward (Btilde in place of Bbar);
 * the scan forms z in float64 and the discretised values in float32.  Same
 * shape limits and conventions as dssm_s5_forward, workspace
 * dssm_s5_tv_workspace_size; step must be 16-byte aligned. */
typedef struct {
  const float* lambda_c;
  const float* Btilde;
  const float* C;
  const float* D;
  const float* delta;
} dssm_s5_tv_params;

int dssm_s5_forward_tv(const float* u, const dssm_s5_tv_params* p, const dssm_s5_shape* s,
                       const float* step, float* y, void* ws, size_t ws_bytes, void* stream);

/* Timing variant of dssm_s5_forward (n_events = 8): start/stop pairs of the
 * four stages, in order: packing of Bbar and C, input projection, the state
 * recurrence (the scan kernel, or the spectrum and convolution kernels of
 * DSSM_S5_FFT), output projection (same event conventions as the DLR timing
 * variants).  For DSSM_S5_FUSED the last three pairs stamp the state-only
 * pass, the kernel that forms the powers of lambda, and the output pass
 * (which also joins the segment states); with one segment per row there is
 * no state-only pass and its pair is recorded back to back. */
int dssm_s5_forward_timed(const float* u, const dssm_s5_params* p, const dssm_s5_shape* s,
                          int method, float* y, void* ws, size_t ws_bytes, void* stream,
                          void* const* events, int n_events);

/* Timing variants: identical results to dssm_forward_fft / dssm_forward_scan;
 * the kernels of stage k are launched with hipExtLaunchKernel so that the GPU
 * itself stamps events[2k] when the stage's first kernel starts and
 * events[2k+1] when its last kernel ends (hipEventElapsedTime of a pair is
 * the stage's duration, without the dispatch gap before it).  A pair of NULL
 * handles leaves that stage untimed (plain launches: an event-stamped launch
 * costs more host time).  n_events = 4 for both:
 *   fft:  [0,1] parameters -> kernel spectrum (generator and spectrum
 *         kernels), [2,3] convolution.
 *   scan: [0,1] per-mode constants of the segmented scan (with the chunked
 *         matrix-core form, used for N <= 64, there is no such kernel and the
 *         pair is recorded back to back: a duration of ~0), [2,3] scan.
 * The events are owned by the caller and must have timing enabled; a NULL
 * array, a pair with one NULL handle, or a wrong n_events returns
 * DSSM_ERR_INVALID_ARG before anything is enqueued. */
int dssm_forward_fft_timed(const float* u, const dssm_dlr_params* p, const dssm_shape* s,
                           float* y, void* ws, size_t ws_bytes, void* stream,
                           void* const* events, int n_events);
int dssm_forward_scan_timed(const float* u, const dssm_dlr_params* p, const dssm_shape* s,
                            float* y, void* ws, size_t ws_bytes, void* stream,
                            void* const* events, int n_events);

#ifdef __cplusplus
}
#endif

#endif /* DSSM_H */
