"""ctypes binding of libdssm.so (C ABI in include/dssm.h).

Argument marshalling only: every step of the forward map runs in the library's
HIP kernels.  Torch supplies device memory and the current stream.  If the
library is missing or a call fails, an exception is raised -- there is no
fallback path.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdssm.so")

DSSM_OK = 0
DSSM_ERR_INVALID_ARG = -1
DSSM_ERR_UNSUPPORTED = -2
DSSM_ERR_WORKSPACE = -3
DSSM_ERR_HIP = -4

OP_GEN, OP_FFT, OP_SCAN, OP_BWD, OP_S5_SCAN, OP_S5_FFT, OP_S5_FUSED = 0, 1, 2, 3, 4, 5, 6
# how the S5 state recurrence runs: scan between the projections, per-state FFT
# convolution, or fused with both projections (v and x on chip)
S5_SCAN, S5_FFT, S5_FUSED = 0, 1, 2
CAST_RE, CAST_RE_IM = 0, 1  # Re K, or Re K * Im K (DLR-prod)

# Every function the header declares (checked by the ABI tests).
EXPORTS = [
    "dssm_version", "dssm_status_string", "dssm_last_error", "dssm_workspace_size",
    "dssm_gen_kernel", "dssm_gen_kernel_cast", "dssm_forward_fft", "dssm_forward_fft_noalloc",
    "dssm_forward_fft_cast",
    "dssm_forward_scan", "dssm_backward",
    "dssm_forward_fft_timed", "dssm_forward_scan_timed",
    "dssm_forward_scan_state", "dssm_step",
    "dssm_s5_workspace_size", "dssm_s5_tv_workspace_size", "dssm_s5_forward",
    "dssm_s5_forward_timed", "dssm_s5_forward_tv",
]


class Grads(ctypes.Structure):
    _fields_ = [("dlog_re", ctypes.c_void_p), ("dlog_im", ctypes.c_void_p),
                ("dW", ctypes.c_void_p), ("dD", ctypes.c_void_p)]


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("N", ctypes.c_int),
                ("L", ctypes.c_int), ("bidirectional", ctypes.c_int)]


class DLRParams(ctypes.Structure):
    _fields_ = [("log_re", ctypes.c_void_p), ("log_im", ctypes.c_void_p),
                ("W", ctypes.c_void_p), ("D", ctypes.c_void_p)]


class S5Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("P", ctypes.c_int),
                ("L", ctypes.c_int), ("bidirectional", ctypes.c_int)]


class S5Params(ctypes.Structure):
    _fields_ = [("lam", ctypes.c_void_p), ("Bbar", ctypes.c_void_p), ("C", ctypes.c_void_p),
                ("D", ctypes.c_void_p)]


class S5TVParams(ctypes.Structure):
    _fields_ = [("lam_c", ctypes.c_void_p), ("Bt", ctypes.c_void_p), ("C", ctypes.c_void_p),
                ("D", ctypes.c_void_p), ("delta", ctypes.c_void_p)]


class DSSMError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("dssm status %d: %s" % (status, message))
        self.status = status


_lib = None


def lib():
    """Load libdssm.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libdssm.so is not built; run `python -m long_convolution_sequence_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    L.dssm_version.restype = ctypes.c_int
    L.dssm_version.argtypes = []
    L.dssm_status_string.restype = ctypes.c_char_p
    L.dssm_status_string.argtypes = [ctypes.c_int]
    L.dssm_last_error.restype = ctypes.c_char_p
    L.dssm_last_error.argtypes = []
    L.dssm_workspace_size.restype = ctypes.c_int
    L.dssm_workspace_size.argtypes = [ctypes.c_int, ctypes.POINTER(Shape), ctypes.POINTER(sz)]
    L.dssm_gen_kernel.restype = ctypes.c_int
    L.dssm_gen_kernel.argtypes = [ctypes.POINTER(DLRParams), ctypes.POINTER(Shape), ctypes.c_int,
                                  vp, vp, sz, vp]
    L.dssm_gen_kernel_cast.restype = ctypes.c_int
    L.dssm_gen_kernel_cast.argtypes = [ctypes.POINTER(DLRParams), ctypes.POINTER(Shape),
                                       ctypes.c_int, vp, vp, sz, vp]
    L.dssm_backward.restype = ctypes.c_int
    L.dssm_backward.argtypes = [vp, vp, ctypes.POINTER(DLRParams), ctypes.POINTER(Shape), vp,
                                ctypes.POINTER(Grads), vp, sz, vp]
    L.dssm_forward_fft_cast.restype = ctypes.c_int
    L.dssm_forward_fft_cast.argtypes = [vp, ctypes.POINTER(DLRParams), ctypes.POINTER(Shape),
                                        ctypes.c_int, vp, vp, sz, vp]
    for name in ("dssm_forward_fft", "dssm_forward_scan"):
        f = getattr(L, name)
        f.restype = ctypes.c_int
        f.argtypes = [vp, ctypes.POINTER(DLRParams), ctypes.POINTER(Shape), vp, vp, sz, vp]
    for name in ("dssm_forward_fft_timed", "dssm_forward_scan_timed"):
        f = getattr(L, name)
        f.restype = ctypes.c_int
        f.argtypes = [vp, ctypes.POINTER(DLRParams), ctypes.POINTER(Shape), vp, vp, sz, vp,
                      ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
    L.dssm_forward_fft_noalloc.restype = ctypes.c_int
    L.dssm_forward_fft_noalloc.argtypes = [vp, ctypes.POINTER(DLRParams), ctypes.POINTER(Shape),
                                           vp, vp]
    L.dssm_forward_scan_state.restype = ctypes.c_int
    L.dssm_forward_scan_state.argtypes = [vp, ctypes.POINTER(DLRParams), ctypes.POINTER(Shape),
                                          vp, vp, vp, sz, vp]
    L.dssm_step.restype = ctypes.c_int
    L.dssm_step.argtypes = [vp, ctypes.POINTER(DLRParams), ctypes.POINTER(Shape), vp, vp, vp]
    L.dssm_s5_tv_workspace_size.restype = ctypes.c_int
    L.dssm_s5_tv_workspace_size.argtypes = [ctypes.POINTER(S5Shape), ctypes.POINTER(ctypes.c_size_t)]
    L.dssm_s5_workspace_size.restype = ctypes.c_int
    L.dssm_s5_workspace_size.argtypes = [ctypes.POINTER(S5Shape), ctypes.c_int,
                                         ctypes.POINTER(sz)]
    L.dssm_s5_forward.restype = ctypes.c_int
    L.dssm_s5_forward.argtypes = [vp, ctypes.POINTER(S5Params), ctypes.POINTER(S5Shape),
                                  ctypes.c_int, vp, vp, sz, vp]
    L.dssm_s5_forward_timed.restype = ctypes.c_int
    L.dssm_s5_forward_timed.argtypes = [vp, ctypes.POINTER(S5Params), ctypes.POINTER(S5Shape),
                                        ctypes.c_int, vp, vp, sz, vp,
                                        ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
    L.dssm_s5_forward_tv.restype = ctypes.c_int
    L.dssm_s5_forward_tv.argtypes = [vp, ctypes.POINTER(S5TVParams), ctypes.POINTER(S5Shape), vp,
                                     vp, vp, sz, vp]
    _lib = L
    return L


def check(status):
    if status != DSSM_OK:
        raise DSSMError(status, lib().dssm_last_error().decode())


def workspace_size(op, B, H, N, L, bidirectional=False):
    shape = Shape(B, H, N, L, int(bool(bidirectional)))
    out = ctypes.c_size_t(0)
    check(lib().dssm_workspace_size(op, ctypes.byref(shape), ctypes.byref(out)))
    return out.value


# ----------------------------------------------------------------------------
# torch-facing wrappers
# ----------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dev_f32(t, name, numel=None, device=None):
    """t as a contiguous float32 device tensor (complex64 viewed as pairs),
    with `numel` float32 elements and on `device` when those are given."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.dtype == torch.complex64:
        t = torch.view_as_real(t)
    if t.dtype != torch.float32:
        raise TypeError("%s must be float32 (or complex64), got %s" % (name, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if numel is not None and t.numel() != numel:
        raise ValueError("%s has %d float32 elements, expected %d" % (name, t.numel(), numel))
    return t


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(stream):
    """Context for the binding's own allocations (workspace, default outputs):
    made on the stream the kernels run on, so the caching allocator does not
    hand their memory to another stream's allocation while those kernels may
    still use it."""
    import contextlib

    torch = _torch()
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _workspace(op, shape, workspace, device, stream=None):
    torch = _torch()
    need = ctypes.c_size_t(0)
    check(lib().dssm_workspace_size(op, ctypes.byref(shape), ctypes.byref(need)))
    if workspace is None:
        with _on_stream(stream):
            workspace = torch.empty(max(need.value, 256), dtype=torch.uint8, device=device)
    elif workspace.device != device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on %s" % device)
    return workspace, workspace.numel() * workspace.element_size()


def _empty(shape, dtype, device, stream):
    torch = _torch()
    with _on_stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def _params(log_re, log_im, W, D, ndir, H, N, device):
    n = ndir * H * N
    lr = _dev_f32(log_re, "log_re", n, device)
    li = _dev_f32(log_im, "log_im", n, device)
    w = _dev_f32(W, "W", 2 * n, device)
    if D is None:  # generator only
        return DLRParams(lr.data_ptr(), li.data_ptr(), w.data_ptr(), None), (lr, li, w)
    d = _dev_f32(D, "D", ndir * H, device)
    keep = (lr, li, w, d)
    return DLRParams(lr.data_ptr(), li.data_ptr(), w.data_ptr(), d.data_ptr()), keep


def gen_kernel(log_re, log_im, W, L, complex_out=False, out=None, workspace=None, stream=None):
    """K[d,h,j] = sum_n W lambda^j for j < L.  log_re/log_im [ndir,H,N] f32,
    W [ndir,H,N] c64.  Returns Re K [ndir,H,L] f32 or K [ndir,H,L] c64."""
    torch = _torch()
    ndir, H, N = log_re.shape
    dev = log_re.device
    shape = Shape(1, H, N, L, ndir - 1)
    p, keep = _params(log_re, log_im, W, None, ndir, H, N, dev)
    if out is None:
        out = _empty((ndir, H, L), torch.complex64 if complex_out else torch.float32, dev, stream)
    o = _dev_f32(out, "out", ndir * H * L * (2 if complex_out else 1), dev)
    ws, nbytes = _workspace(OP_GEN, shape, workspace, dev, stream)
    check(lib().dssm_gen_kernel(ctypes.byref(p), ctypes.byref(shape), int(bool(complex_out)),
                                o.data_ptr(), ws.data_ptr(), nbytes, _stream(stream)))
    del keep
    return out


def gen_kernel_cast(log_re, log_im, W, L, cast=CAST_RE, out=None, workspace=None, stream=None):
    """The real kernel of a cast: Re K (CAST_RE) or Re K * Im K (CAST_RE_IM,
    DLR-prod), [ndir,H,L] f32."""
    torch = _torch()
    ndir, H, N = log_re.shape
    dev = log_re.device
    shape = Shape(1, H, N, L, ndir - 1)
    p, keep = _params(log_re, log_im, W, None, ndir, H, N, dev)
    if out is None:
        out = _empty((ndir, H, L), torch.float32, dev, stream)
    o = _dev_f32(out, "out", ndir * H * L, dev)
    ws, nbytes = _workspace(OP_GEN, shape, workspace, dev, stream)
    check(lib().dssm_gen_kernel_cast(ctypes.byref(p), ctypes.byref(shape), int(cast),
                                     o.data_ptr(), ws.data_ptr(), nbytes, _stream(stream)))
    del keep
    return out


def _rows(u, name="u"):
    uu = _dev_f32(u, name)
    if uu.dim() != 3:
        raise ValueError("%s must be [B, H, L]" % name)
    return uu


def _forward(fn, op, u, log_re, log_im, W, D, bidirectional, y, workspace, stream, events=None,
             cast=None):
    torch = _torch()
    uu = _rows(u)
    B, H, L = uu.shape
    dev = uu.device
    ndir = 2 if bidirectional else 1
    N = log_re.shape[-1]
    shape = Shape(B, H, N, L, int(bool(bidirectional)))
    p, keep = _params(log_re, log_im, W, D, ndir, H, N, dev)
    if y is None:
        y = _empty(uu.shape, torch.float32, dev, stream)
    yy = _dev_f32(y, "y", uu.numel(), dev)
    ws, nbytes = _workspace(op, shape, workspace, dev, stream)
    args = [uu.data_ptr(), ctypes.byref(p), ctypes.byref(shape)]
    if cast is not None:
        args.append(int(cast))
    args += [yy.data_ptr(), ws.data_ptr(), nbytes, _stream(stream)]
    if events is not None:
        arr = (ctypes.c_void_p * len(events))(*events)
        args += [arr, len(events)]
    check(fn(*args))
    del keep
    return y


def forward_fft(u, log_re, log_im, W, D, bidirectional=False, y=None, workspace=None, stream=None):
    """Layer forward by the FFT convolution view.  u [B,H,L] f32 -> y [B,H,L]."""
    return _forward(lib().dssm_forward_fft, OP_FFT, u, log_re, log_im, W, D, bidirectional, y,
                    workspace, stream)


def forward_fft_noalloc(u, log_re, log_im, W, D, y, bidirectional=False, stream=None):
    """forward_fft into the caller's y with the library's fixed per-device
    scratch array as workspace: nothing is allocated, here or in the library.
    Calls that overlap in time on one device race on that array."""
    uu = _rows(u)
    B, H, L = uu.shape
    dev = uu.device
    ndir = 2 if bidirectional else 1
    N = log_re.shape[-1]
    shape = Shape(B, H, N, L, int(bool(bidirectional)))
    p, keep = _params(log_re, log_im, W, D, ndir, H, N, dev)
    yy = _dev_f32(y, "y", uu.numel(), dev)
    check(lib().dssm_forward_fft_noalloc(uu.data_ptr(), ctypes.byref(p), ctypes.byref(shape),
                                         yy.data_ptr(), _stream(stream)))
    del keep
    return y


def forward_fft_cast(u, log_re, log_im, W, D, cast, bidirectional=False, y=None, workspace=None,
                     stream=None):
    """Layer forward by the FFT convolution view with the kernel cast `cast`
    (CAST_RE: as forward_fft; CAST_RE_IM: DLR-prod)."""
    return _forward(lib().dssm_forward_fft_cast, OP_FFT, u, log_re, log_im, W, D, bidirectional, y,
                    workspace, stream, cast=cast)


def backward(u, dy, log_re, log_im, W, D, bidirectional=False, du=None, workspace=None,
             stream=None):
    """Gradients of f = sum(dy * y) for the layer map: returns du [B,H,L] f32
    and a dict dlog_re, dlog_im [ndir,H,N] f32, dW [ndir,H,N] c64
    (d/d Re W + i d/d Im W), dD [ndir,H] f32."""
    torch = _torch()
    uu = _rows(u)
    dev = uu.device
    gg = _dev_f32(dy, "dy", uu.numel(), dev)
    B, H, L = uu.shape
    ndir = 2 if bidirectional else 1
    N = log_re.shape[-1]
    shape = Shape(B, H, N, L, int(bool(bidirectional)))
    p, keep = _params(log_re, log_im, W, D, ndir, H, N, dev)
    if du is None:
        du = _empty(uu.shape, torch.float32, dev, stream)
    dd = _dev_f32(du, "du", uu.numel(), dev)
    out = dict(dlog_re=_empty((ndir, H, N), torch.float32, dev, stream),
               dlog_im=_empty((ndir, H, N), torch.float32, dev, stream),
               dW=_empty((ndir, H, N), torch.complex64, dev, stream),
               dD=_empty((ndir, H), torch.float32, dev, stream))
    g = Grads(out["dlog_re"].data_ptr(), out["dlog_im"].data_ptr(), out["dW"].data_ptr(),
              out["dD"].data_ptr())
    ws, nbytes = _workspace(OP_BWD, shape, workspace, dev, stream)
    check(lib().dssm_backward(uu.data_ptr(), gg.data_ptr(), ctypes.byref(p), ctypes.byref(shape),
                              dd.data_ptr(), ctypes.byref(g), ws.data_ptr(), nbytes,
                              _stream(stream)))
    del keep
    return du, out


def forward_scan(u, log_re, log_im, W, D, bidirectional=False, y=None, workspace=None, stream=None):
    """Layer forward by the recurrence (scan) view.  u [B,H,L] f32 -> y [B,H,L]."""
    return _forward(lib().dssm_forward_scan, OP_SCAN, u, log_re, log_im, W, D, bidirectional, y,
                    workspace, stream)


def forward_scan_state(u, log_re, log_im, W, D, x, y=None, workspace=None, stream=None):
    """Streaming forward, one direction: continues the recurrence from the
    state x [B,H,N] c64 (updated in place to the state after the last step).
    u [B,H,L] f32 -> y [B,H,L]."""
    torch = _torch()
    uu = _rows(u)
    B, H, L = uu.shape
    dev = uu.device
    N = log_re.shape[-1]
    shape = Shape(B, H, N, L, 0)
    p, keep = _params(log_re, log_im, W, D, 1, H, N, dev)
    xx = _dev_f32(x, "x", 2 * B * H * N, dev)
    if y is None:
        y = _empty(uu.shape, torch.float32, dev, stream)
    yy = _dev_f32(y, "y", uu.numel(), dev)
    ws, nbytes = _workspace(OP_SCAN, shape, workspace, dev, stream)
    check(lib().dssm_forward_scan_state(uu.data_ptr(), ctypes.byref(p), ctypes.byref(shape),
                                        xx.data_ptr(), yy.data_ptr(), ws.data_ptr(), nbytes,
                                        _stream(stream)))
    del keep
    return y


def step(u_t, log_re, log_im, W, D, x, y=None, stream=None):
    """One decode step: u_t [B,H] f32 -> y_t [B,H]; x [B,H,N] c64 updated in
    place."""
    torch = _torch()
    uu = _dev_f32(u_t, "u_t")
    if uu.dim() != 2:
        raise ValueError("u_t must be [B, H]")
    B, H = uu.shape
    dev = uu.device
    N = log_re.shape[-1]
    shape = Shape(B, H, N, 1, 0)
    p, keep = _params(log_re, log_im, W, D, 1, H, N, dev)
    xx = _dev_f32(x, "x", 2 * B * H * N, dev)
    if y is None:
        y = _empty(uu.shape, torch.float32, dev, stream)
    yy = _dev_f32(y, "y", uu.numel(), dev)
    check(lib().dssm_step(uu.data_ptr(), ctypes.byref(p), ctypes.byref(shape), xx.data_ptr(),
                          yy.data_ptr(), _stream(stream)))
    del keep
    return y


def forward_timed(path, u, log_re, log_im, W, D, events, bidirectional=False, y=None,
                  workspace=None, stream=None):
    """forward_fft / forward_scan whose stages the GPU brackets with the given
    raw hipEvent_t handles (ints, None for an untimed stage): a start/stop pair
    per stage, 4 in all -- fft: kernel spectrum (from the parameters),
    convolution; scan: constants, scan."""
    if path == "fft":
        fn, op = lib().dssm_forward_fft_timed, OP_FFT
    else:
        fn, op = lib().dssm_forward_scan_timed, OP_SCAN
    return _forward(fn, op, u, log_re, log_im, W, D, bidirectional, y, workspace, stream,
                    events=list(events))


def s5_workspace_size(B, H, P, L, method=S5_SCAN):
    shape = S5Shape(B, H, P, L, 0)
    out = ctypes.c_size_t(0)
    check(lib().dssm_s5_workspace_size(ctypes.byref(shape), int(method), ctypes.byref(out)))
    return out.value


def s5_tv_workspace_size(B, H, P, L):
    shape = S5Shape(B, H, P, L, 0)
    out = ctypes.c_size_t(0)
    check(lib().dssm_s5_tv_workspace_size(ctypes.byref(shape), ctypes.byref(out)))
    return out.value


def _s5_workspace(shape, workspace, device, stream, method=S5_SCAN):
    """method None: the size dssm_s5_forward_tv needs."""
    torch = _torch()
    need = ctypes.c_size_t(0)
    if method is None:
        check(lib().dssm_s5_tv_workspace_size(ctypes.byref(shape), ctypes.byref(need)))
    else:
        check(lib().dssm_s5_workspace_size(ctypes.byref(shape), int(method), ctypes.byref(need)))
    if workspace is None:
        with _on_stream(stream):
            workspace = torch.empty(max(need.value, 256), dtype=torch.uint8, device=device)
    elif workspace.device != device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on %s" % device)
    return workspace, workspace.numel() * workspace.element_size()


def s5_forward(u, lam, Bbar, C, D, y=None, workspace=None, stream=None, events=None,
               method=S5_SCAN):
    """S5 layer forward.  u [B,H,L] f32, lam [P] c64, Bbar [P,H] c64,
    C [H,P] c64, D [H] f32 -> y [B,H,L] f32.  method: S5_SCAN (the
    recurrence as a scan between the projections), S5_FFT (per state, the
    convolution with lambda^j by FFT) or S5_FUSED (projections and
    recurrence in one pass, v and x on chip).  events: optional 8 raw
    hipEvent_t handles, a start/stop pair per stage (pack, proj_in,
    recurrence, proj_out; for S5_FUSED: pack, state-only pass, powers of
    lambda, output pass)."""
    torch = _torch()
    uu = _rows(u)
    B, H, L = uu.shape
    dev = uu.device
    lm = _dev_f32(lam, "lam", device=dev)
    P = lm.numel() // 2
    bb = _dev_f32(Bbar, "Bbar", 2 * P * H, dev)
    cc = _dev_f32(C, "C", 2 * H * P, dev)
    dd = _dev_f32(D, "D", H, dev)
    shape = S5Shape(B, H, P, L, 0)
    prm = S5Params(lm.data_ptr(), bb.data_ptr(), cc.data_ptr(), dd.data_ptr())
    if y is None:
        y = _empty(uu.shape, torch.float32, dev, stream)
    yy = _dev_f32(y, "y", uu.numel(), dev)
    ws, nbytes = _s5_workspace(shape, workspace, dev, stream, method)
    args = [uu.data_ptr(), ctypes.byref(prm), ctypes.byref(shape), int(method), yy.data_ptr(),
            ws.data_ptr(), nbytes, _stream(stream)]
    if events is None:
        check(lib().dssm_s5_forward(*args))
    else:
        arr = (ctypes.c_void_p * len(events))(*events)
        check(lib().dssm_s5_forward_timed(*(args + [arr, len(events)])))
    return y


def s5_forward_tv(u, lam_c, Bt, C, D, delta, step, y=None, workspace=None, stream=None):
    """Continuous-time S5 layer forward with a step size per (b, k).  u [B,H,L]
    f32, lam_c [P] c64, Bt [P,H] c64, C [H,P] c64, D [H] f32, delta [P] f32,
    step [B,L] f32 -> y [B,H,L] f32."""
    torch = _torch()
    uu = _rows(u)
    B, H, L = uu.shape
    dev = uu.device
    lm = _dev_f32(lam_c, "lam_c", device=dev)
    P = lm.numel() // 2
    bb = _dev_f32(Bt, "Bt", 2 * P * H, dev)
    cc = _dev_f32(C, "C", 2 * H * P, dev)
    dd = _dev_f32(D, "D", H, dev)
    dl = _dev_f32(delta, "delta", P, dev)
    ss = _dev_f32(step, "step", B * L, dev)
    shape = S5Shape(B, H, P, L, 0)
    prm = S5TVParams(lm.data_ptr(), bb.data_ptr(), cc.data_ptr(), dd.data_ptr(), dl.data_ptr())
    if y is None:
        y = _empty(uu.shape, torch.float32, dev, stream)
    yy = _dev_f32(y, "y", uu.numel(), dev)
    ws, nbytes = _s5_workspace(shape, workspace, dev, stream, None)
    check(lib().dssm_s5_forward_tv(uu.data_ptr(), ctypes.byref(prm), ctypes.byref(shape),
                                   ss.data_ptr(), yy.data_ptr(), ws.data_ptr(), nbytes,
                                   _stream(stream)))
    return y


class HipEvents:
    """Raw hipEvent_t handles through libamdhip64, for the timing variants
    (plumbing only: create, elapsed time, destroy)."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.h.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError("hipEventCreate failed: %d" % rc)
            out.append(e.value)
        return out

    def ms(self, a, b):
        t = ctypes.c_float()
        rc = self.h.hipEventElapsedTime(ctypes.byref(t), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return t.value

    def record(self, e, stream):
        rc = self.h.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError("hipEventRecord failed: %d" % rc)

    def destroy(self, evs):
        for e in evs:
            self.h.hipEventDestroy(ctypes.c_void_p(e))
