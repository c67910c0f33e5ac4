// Host entry points of libdssm.so (C ABI declared in include/dssm.h):
// argument validation, workspace carving and kernel launches on the caller's
// stream.  No device memory is allocated here.
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/dssm.h"
#include "dssm_internal.h"

using namespace dssm;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return DSSM_OK;
}

int hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DSSM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return DSSM_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kMaxN = 4096;
constexpr int kMaxLScan = 1 << 24;
constexpr int kMaxFFTL = 1 << kMaxLog2M;
constexpr int kMaxGrid = 65535;

// Validate a shape for `op`; on success *empty tells whether there is no work.
int check_shape(int op, const dssm_shape* s, bool* empty) {
  if (!s) return fail(DSSM_ERR_INVALID_ARG, "shape is NULL");
  if (s->B < 0 || s->H < 0 || s->L < 0)
    return fail(DSSM_ERR_INVALID_ARG, "negative dimension (B=%d H=%d L=%d)", s->B, s->H, s->L);
  if (s->N < 1) return fail(DSSM_ERR_INVALID_ARG, "N must be >= 1 (got %d)", s->N);
  if (s->bidirectional != 0 && s->bidirectional != 1)
    return fail(DSSM_ERR_INVALID_ARG, "bidirectional must be 0 or 1 (got %d)", s->bidirectional);
  if (op != DSSM_OP_GEN && op != DSSM_OP_FFT && op != DSSM_OP_SCAN && op != DSSM_OP_BWD)
    return fail(DSSM_ERR_INVALID_ARG, "unknown op %d", op);
  const int ndir = 1 + s->bidirectional;
  if (s->N > kMaxN) return fail(DSSM_ERR_UNSUPPORTED, "N=%d exceeds %d", s->N, kMaxN);
  if ((long)s->H * ndir > kMaxGrid)
    return fail(DSSM_ERR_UNSUPPORTED, "H*ndir=%ld exceeds %d", (long)s->H * ndir, kMaxGrid);
  if (s->L > kMaxLScan) return fail(DSSM_ERR_UNSUPPORTED, "L=%d exceeds %d", s->L, kMaxLScan);
  if (op == DSSM_OP_FFT && s->L > kMaxFFTL)
    return fail(DSSM_ERR_UNSUPPORTED, "FFT path needs L <= %d (got %d); use the scan path",
                kMaxFFTL, s->L);
  if (op == DSSM_OP_BWD && s->L > kMaxFFTL)
    return fail(DSSM_ERR_UNSUPPORTED, "the backward pass needs L <= %d (got %d)", kMaxFFTL, s->L);
  if (op == DSSM_OP_BWD && (long)s->B * s->H > (1L << 26))
    return fail(DSSM_ERR_UNSUPPORTED, "B*H=%ld too large for the backward pass",
                (long)s->B * s->H);
  if ((long)s->B * s->H * s->L > (1L << 40))
    return fail(DSSM_ERR_UNSUPPORTED, "B*H*L too large");
  // rows (and the workgroups of the per-row kernels) are counted in int
  if ((long)s->B * s->H * ndir > (long)INT32_MAX)
    return fail(DSSM_ERR_UNSUPPORTED, "B*H*ndir=%ld exceeds 2^31 - 1",
                (long)s->B * s->H * ndir);
  const bool no_rows = (op == DSSM_OP_GEN) ? false : (s->B == 0);
  *empty = no_rows || s->H == 0 || s->L == 0;
  return DSSM_OK;
}

// D is read by the forward calls only (dssm_gen_kernel ignores it).
int check_params(const dssm_dlr_params* p, bool need_d) {
  if (!p) return fail(DSSM_ERR_INVALID_ARG, "params is NULL");
  if (!p->log_re || !p->log_im || !p->W || (need_d && !p->D))
    return fail(DSSM_ERR_INVALID_ARG, "a parameter pointer is NULL");
  if (!aligned16(p->log_re) || !aligned16(p->log_im) || !aligned16(p->W) ||
      (need_d && !aligned16(p->D)))
    return fail(DSSM_ERR_INVALID_ARG, "parameter pointers must be 16-byte aligned");
  return DSSM_OK;
}

// The recurrence view runs in the chunked state-space form on the matrix
// cores for up to 64 modes (one workgroup per (b, h)); otherwise in the
// segmented scan.
bool use_chunk(const dssm_shape* s) {
  return chunk_supported(s->N) && (long)s->B * s->H <= (1L << 24);
}

// Workspace layout, every region aligned to 256 bytes.
struct Layout {
  size_t reK = 0, spec = 0, consts = 0, carry = 0, corr = 0, parts = 0, chunk = 0, total = 0;
};

Layout layout(int op, const dssm_shape* s) {
  Layout l;
  const size_t ndh = (size_t)(1 + s->bidirectional) * s->H;
  const size_t N = s->N, L = s->L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  if (op == DSSM_OP_FFT) {
    const int log2m = fft_log2m(s->L);
    const size_t M = (size_t)1 << log2m;
    l.reK = take(ndh * L * sizeof(float));
    l.spec = take((size_t)s->H * 2 * M * sizeof(float2));
  }
  if (op == DSSM_OP_BWD) {
    // the layer's (conjugate) spectrum for du, the two halves of the
    // batch-summed lagged correlations, then the partial parameter sums
    const int log2m = fft_log2m(s->L);
    const size_t M = (size_t)1 << log2m;
    l.reK = take(ndh * L * sizeof(float));
    l.spec = take((size_t)s->H * 2 * M * sizeof(float2));
    l.corr = take((size_t)corr_groups(s->B, s->H) * s->H * 2 * M * sizeof(float));
    l.parts = take(ndh * (size_t)grad_splits(s->L) * N * 2 * 2 * sizeof(double));
  }
  if (op == DSSM_OP_SCAN && use_chunk(s)) {
    // segment states of the chunked form (none unless the sequence is split)
    l.chunk = take(chunk_workspace(s->B, s->H, s->N, s->L, 1 + s->bidirectional));
  } else if (op == DSSM_OP_SCAN) {
    const ScanPlan plan = scan_plan(s->B, s->L);
    l.consts = take(ndh * N * plan.nconst * sizeof(float));
    l.carry = take((size_t)s->B * s->H * N * sizeof(float2));
  }
  l.total = off;
  return l;
}

int check_ws(int op, const dssm_shape* s, void* ws, size_t ws_bytes, Layout* l) {
  *l = layout(op, s);
  if (ws_bytes < l->total)
    return fail(DSSM_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                ws_bytes, l->total);
  if (l->total > 0 && !ws) return fail(DSSM_ERR_INVALID_ARG, "workspace is NULL");
  if (ws && (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(DSSM_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return DSSM_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

}  // namespace

extern "C" {

int dssm_version(void) { return DSSM_VERSION; }

const char* dssm_status_string(int status) {
  switch (status) {
    case DSSM_OK: return "ok";
    case DSSM_ERR_INVALID_ARG: return "invalid argument";
    case DSSM_ERR_UNSUPPORTED: return "unsupported";
    case DSSM_ERR_WORKSPACE: return "workspace too small";
    case DSSM_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* dssm_last_error(void) { return g_last_error.c_str(); }

static int s5_workspace(const dssm_s5_shape* s, int method, size_t* bytes);

int dssm_workspace_size(int op, const dssm_shape* s, size_t* bytes) {
  if (!bytes) return fail(DSSM_ERR_INVALID_ARG, "bytes is NULL");
  if (op == DSSM_OP_S5_SCAN || op == DSSM_OP_S5_FFT || op == DSSM_OP_S5_FUSED) {
    // N is the state size P
    if (!s) return fail(DSSM_ERR_INVALID_ARG, "shape is NULL");
    const dssm_s5_shape s5{s->B, s->H, s->N, s->L, s->bidirectional};
    return s5_workspace(&s5,
                        op == DSSM_OP_S5_FFT     ? DSSM_S5_FFT
                        : op == DSSM_OP_S5_FUSED ? DSSM_S5_FUSED
                                                 : DSSM_S5_SCAN,
                        bytes);
  }
  bool empty = false;
  int rc = check_shape(op, s, &empty);
  if (rc) return rc;
  *bytes = empty ? 0 : layout(op, s).total;
  return ok();
}

static int gen_impl(const dssm_dlr_params* p, const dssm_shape* s, int out, float* K, void* ws,
                    size_t ws_bytes, void* stream) {
  bool empty = false;
  int rc = check_shape(DSSM_OP_GEN, s, &empty);
  if (rc) return rc;
  if (empty) return ok();
  if ((rc = check_params(p, false))) return rc;
  if (!K || !aligned16(K)) return fail(DSSM_ERR_INVALID_ARG, "K is NULL or not 16-byte aligned");
  Layout l;
  if ((rc = check_ws(DSSM_OP_GEN, s, ws, ws_bytes, &l))) return rc;
  if ((rc = hip_check(launch_gen(p->log_re, p->log_im, p->W, (1 + s->bidirectional) * s->H, s->N,
                                 s->L, out, K, static_cast<hipStream_t>(stream)),
                      "gen launch")))
    return rc;
  return ok();
}

int dssm_gen_kernel(const dssm_dlr_params* p, const dssm_shape* s, int complex_out, float* K,
                    void* ws, size_t ws_bytes, void* stream) {
  if (complex_out != 0 && complex_out != 1) {
    bool empty = false;
    const int rc = check_shape(DSSM_OP_GEN, s, &empty);
    if (rc) return rc;
    return fail(DSSM_ERR_INVALID_ARG, "complex_out must be 0 or 1");
  }
  return gen_impl(p, s, complex_out ? kGenComplex : kGenRe, K, ws, ws_bytes, stream);
}

static int check_cast(int cast) {
  if (cast != DSSM_CAST_RE && cast != DSSM_CAST_RE_IM)
    return fail(DSSM_ERR_INVALID_ARG, "cast must be DSSM_CAST_RE (0) or DSSM_CAST_RE_IM (1), got %d",
                cast);
  return DSSM_OK;
}

int dssm_gen_kernel_cast(const dssm_dlr_params* p, const dssm_shape* s, int cast, float* K,
                         void* ws, size_t ws_bytes, void* stream) {
  bool empty = false;
  int rc = check_shape(DSSM_OP_GEN, s, &empty);
  if (rc) return rc;
  if ((rc = check_cast(cast))) return rc;
  return gen_impl(p, s, cast == DSSM_CAST_RE_IM ? kGenReIm : kGenRe, K, ws, ws_bytes, stream);
}

// A kernel's start/stop pair is both handles or neither (kernel untimed).
static int check_events(void* const* events, int n_events) {
  if (!events) return DSSM_OK;
  for (int k = 0; 2 * k < n_events; ++k)
    if (!events[2 * k] != !events[2 * k + 1])
      return fail(DSSM_ERR_INVALID_ARG, "events[%d] and events[%d] must both be set or both NULL",
                  2 * k, 2 * k + 1);
  return DSSM_OK;
}

// Start/stop event pair of kernel k of a timed call (none when untimed).
static KEvents kev(void* const* events, int k) {
  KEvents e;
  if (events) {
    e.start = static_cast<hipEvent_t>(events[2 * k]);
    e.stop = static_cast<hipEvent_t>(events[2 * k + 1]);
  }
  return e;
}

// Shared body of the forward calls.  events (optional) are hipEvent_t pairs
// that the GPU stamps at the start and the end of each kernel.
static int forward_impl(int op, const float* u, const dssm_dlr_params* p, const dssm_shape* s,
                        float* y, void* ws, size_t ws_bytes, void* stream, void* const* events,
                        int n_events, int cast = DSSM_CAST_RE) {
  bool empty = false;
  int rc = check_shape(op, s, &empty);
  if (rc) return rc;
  if ((rc = check_cast(cast))) return rc;
  const int want = 4;
  if (events && n_events != want)
    return fail(DSSM_ERR_INVALID_ARG, "n_events must be %d (got %d)", want, n_events);
  if (empty) return ok();
  if ((rc = check_params(p, true))) return rc;
  if (!u || !y || !aligned16(u) || !aligned16(y))
    return fail(DSSM_ERR_INVALID_ARG, "u or y is NULL or not 16-byte aligned");
  if (u == y) return fail(DSSM_ERR_INVALID_ARG, "y must not alias u");
  if ((rc = check_events(events, n_events))) return rc;
  Layout l;
  if ((rc = check_ws(op, s, ws, ws_bytes, &l))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int ndir = 1 + s->bidirectional;
  if (op == DSSM_OP_FFT) {
    const int log2m = fft_log2m(s->L);
    float2* spec = at<float2>(ws, l.spec);
    const KEvents e0 = kev(events, 0);  // parameters -> spectrum: generator + spectrum
    float* reK = at<float>(ws, l.reK);
    const int gen_out = cast == DSSM_CAST_RE_IM ? kGenReIm : kGenRe;
    if ((rc = hip_check(launch_gen(p->log_re, p->log_im, p->W, ndir * s->H, s->N, s->L, gen_out,
                                   reK, st, KEvents{e0.start, nullptr}),
                        "gen launch")))
      return rc;
    if ((rc = hip_check(launch_spectrum(reK, p->D, ndir, s->H, s->L, log2m, spec, st,
                                        KEvents{nullptr, e0.stop}),
                        "spectrum launch")))
      return rc;
    if ((rc = hip_check(launch_conv(u, spec, s->B, s->H, s->L, log2m, y, st, kev(events, 1)),
                        "conv launch")))
      return rc;
  } else if (use_chunk(s)) {
    // chunked state-space form on the matrix cores (operands formed in the
    // kernel): stage 0 has no kernel, its pair is recorded back to back
    const KEvents e0 = kev(events, 0);
    if (e0.start && (rc = hip_check(hipEventRecord(e0.start, st), "event record"))) return rc;
    if (e0.stop && (rc = hip_check(hipEventRecord(e0.stop, st), "event record"))) return rc;
    if ((rc = hip_check(launch_chunk(u, p->log_re, p->log_im, p->W, p->D, s->B, s->H, s->N, s->L,
                                     ndir, y, nullptr, nullptr, at<void>(ws, l.chunk), st,
                                     kev(events, 1)),
                        "chunk launch")))
      return rc;
  } else {
    const ScanPlan plan = scan_plan(s->B, s->L);
    float* consts = at<float>(ws, l.consts);
    if ((rc = hip_check(launch_scan_consts(p->log_re, p->log_im, p->W, ndir * s->H, s->N, plan,
                                           consts, st, kev(events, 0)),
                        "scan consts launch")))
      return rc;
    if ((rc = hip_check(launch_scan(u, consts, p->D, s->B, s->H, s->N, s->L, ndir, plan, y, st,
                                    at<float2>(ws, l.carry), kev(events, 1)),
                        "scan launch")))
      return rc;
  }
  return ok();
}

int dssm_forward_fft(const float* u, const dssm_dlr_params* p, const dssm_shape* s, float* y,
                     void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(DSSM_OP_FFT, u, p, s, y, ws, ws_bytes, stream, nullptr, 0);
}

// Scratch memory of dssm_forward_fft_noalloc: the workspace of the FFT view
// (the real kernel rows and the spectrum table) as a file-scope device array.
// Each device holds its own copy, from the library's first use on it until
// the process ends.  Host code never passes the symbol itself to a kernel:
// the device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the
// first call per device, then cached).
int scratch_address(void** out) {
  int dev = -1;
  if (int rc = hip_check(hipGetDevice(&dev), "hipGetDevice")) return rc;
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DSSM_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (int rc = hip_check(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress"))
      return rc;
    if (!ptr) return fail(DSSM_ERR_HIP, "hipGetSymbolAddress returned NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DSSM_OK;
}
}  // namespace

int dssm_forward_fft_noalloc(const float* u, const dssm_dlr_params* p, const dssm_shape* s,
                             float* y, void* stream) {
  bool empty = false;
  int rc = check_shape(DSSM_OP_FFT, s, &empty);
  if (rc) return rc;
  if (empty) return ok();
  const size_t need = layout(DSSM_OP_FFT, s).total;
  if (need > kScratchBytes)
    return fail(DSSM_ERR_UNSUPPORTED,
                "the allocation-free forward needs %zu bytes of scratch for this shape; its "
                "maximum is %zu (use dssm_forward_fft with a caller workspace)",
                need, kScratchBytes);
  // argument errors are reported before the device is touched
  if ((rc = check_params(p, true))) return rc;
  if (!u || !y || !aligned16(u) || !aligned16(y))
    return fail(DSSM_ERR_INVALID_ARG, "u or y is NULL or not 16-byte aligned");
  if (u == y) return fail(DSSM_ERR_INVALID_ARG, "y must not alias u");
  void* ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  return forward_impl(DSSM_OP_FFT, u, p, s, y, ws, kScratchBytes, stream, nullptr, 0);
}

int dssm_forward_fft_cast(const float* u, const dssm_dlr_params* p, const dssm_shape* s,
                          int cast, float* y, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(DSSM_OP_FFT, u, p, s, y, ws, ws_bytes, stream, nullptr, 0, cast);
}

int dssm_backward(const float* u, const float* dy, const dssm_dlr_params* p, const dssm_shape* s,
                  float* du, const dssm_dlr_grads* g, void* ws, size_t ws_bytes, void* stream) {
  bool empty = false;
  int rc = check_shape(DSSM_OP_BWD, s, &empty);
  if (rc) return rc;
  if (s->H == 0) return ok();
  if ((rc = check_params(p, true))) return rc;
  if (!g) return fail(DSSM_ERR_INVALID_ARG, "grads is NULL");
  if (!g->dlog_re || !g->dlog_im || !g->dW || !g->dD)
    return fail(DSSM_ERR_INVALID_ARG, "a gradient pointer is NULL");
  if (!aligned16(g->dlog_re) || !aligned16(g->dlog_im) || !aligned16(g->dW) || !aligned16(g->dD))
    return fail(DSSM_ERR_INVALID_ARG, "gradient pointers must be 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int ndir = 1 + s->bidirectional;
  if (empty) {  // no rows or no steps: the parameter gradients are zero
    if ((rc = hip_check(launch_zero_grads(g->dlog_re, g->dlog_im, g->dW, g->dD, ndir * s->H, s->N,
                                          st),
                        "zero launch")))
      return rc;
    return ok();
  }
  if (!u || !dy || !du || !aligned16(u) || !aligned16(dy) || !aligned16(du))
    return fail(DSSM_ERR_INVALID_ARG, "u, dy or du is NULL or not 16-byte aligned");
  if (du == u || du == dy) return fail(DSSM_ERR_INVALID_ARG, "du must not alias u or dy");
  Layout l;
  if ((rc = check_ws(DSSM_OP_BWD, s, ws, ws_bytes, &l))) return rc;
  const int log2m = fft_log2m(s->L);
  float* reK = at<float>(ws, l.reK);
  float2* spec = at<float2>(ws, l.spec);
  float* corr = at<float>(ws, l.corr);
  // du: the transposed operator, i.e. the layer's spectrum conjugated
  if ((rc = hip_check(launch_gen(p->log_re, p->log_im, p->W, ndir * s->H, s->N, s->L, kGenRe, reK,
                                 st),
                      "gen launch")))
    return rc;
  if ((rc = hip_check(launch_spectrum(reK, p->D, ndir, s->H, s->L, log2m, spec, st, {}, 1),
                      "spectrum launch")))
    return rc;
  if ((rc = hip_check(launch_conv(dy, spec, s->B, s->H, s->L, log2m, du, st), "conv launch")))
    return rc;
  // kernel cotangents of both directions: the lagged correlations of u and
  // dy, summed over the batch in the frequency domain
  if ((rc = hip_check(launch_corr(u, dy, s->B, s->H, s->L, log2m, corr, st), "corr launch")))
    return rc;
  if ((rc = hip_check(launch_grad_params(corr, 1 << log2m, corr_groups(s->B, s->H), s->H, s->L,
                                         p->log_re, p->log_im, p->W,
                                         s->N, ndir, at<void>(ws, l.parts), g->dlog_re,
                                         g->dlog_im, g->dW, g->dD, st),
                      "gradient launch")))
    return rc;
  return ok();
}

int dssm_forward_scan(const float* u, const dssm_dlr_params* p, const dssm_shape* s, float* y,
                      void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(DSSM_OP_SCAN, u, p, s, y, ws, ws_bytes, stream, nullptr, 0);
}

int dssm_forward_scan_state(const float* u, const dssm_dlr_params* p, const dssm_shape* s,
                            float* x, float* y, void* ws, size_t ws_bytes, void* stream) {
  bool empty = false;
  int rc = check_shape(DSSM_OP_SCAN, s, &empty);
  if (rc) return rc;
  if (s->bidirectional)
    return fail(DSSM_ERR_UNSUPPORTED, "the stateful forward runs one direction (bidirectional=0)");
  if (empty) return ok();  // L = 0: the state passes through unchanged
  if ((rc = check_params(p, true))) return rc;
  if (!u || !y || !aligned16(u) || !aligned16(y))
    return fail(DSSM_ERR_INVALID_ARG, "u or y is NULL or not 16-byte aligned");
  if (!x || !aligned16(x)) return fail(DSSM_ERR_INVALID_ARG, "x is NULL or not 16-byte aligned");
  if (u == y || x == u || x == y) return fail(DSSM_ERR_INVALID_ARG, "u, x and y must not alias");
  Layout l;
  if ((rc = check_ws(DSSM_OP_SCAN, s, ws, ws_bytes, &l))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (use_chunk(s)) {  // the chunked form, from the state in x and back into it
    if ((rc = hip_check(launch_chunk(u, p->log_re, p->log_im, p->W, p->D, s->B, s->H, s->N, s->L,
                                     1, y, x, x, at<void>(ws, l.chunk), st),
                        "chunk launch")))
      return rc;
    return ok();
  }
  const ScanPlan plan = scan_plan(s->B, s->L);
  float* consts = at<float>(ws, l.consts);
  if ((rc = hip_check(launch_scan_consts(p->log_re, p->log_im, p->W, s->H, s->N, plan, consts, st),
                      "scan consts launch")))
    return rc;
  if ((rc = hip_check(launch_scan(u, consts, p->D, s->B, s->H, s->N, s->L, 1, plan, y, st,
                                  reinterpret_cast<float2*>(x), KEvents{}, true),
                      "scan launch")))
    return rc;
  return ok();
}

int dssm_step(const float* u_t, const dssm_dlr_params* p, const dssm_shape* s, float* x,
              float* y_t, void* stream) {
  bool empty = false;
  int rc = check_shape(DSSM_OP_SCAN, s, &empty);
  if (rc) return rc;
  if (s->L != 1) return fail(DSSM_ERR_INVALID_ARG, "dssm_step takes one time step (L must be 1, got %d)", s->L);
  if (s->bidirectional)
    return fail(DSSM_ERR_UNSUPPORTED, "a decode step runs one direction (bidirectional=0)");
  if (empty) return ok();
  if ((rc = check_params(p, true))) return rc;
  if (!u_t || !y_t || !x || !aligned16(u_t) || !aligned16(y_t) || !aligned16(x))
    return fail(DSSM_ERR_INVALID_ARG, "u_t, x or y_t is NULL or not 16-byte aligned");
  if (u_t == y_t || x == u_t || x == y_t)
    return fail(DSSM_ERR_INVALID_ARG, "u_t, x and y_t must not alias");
  if ((long)s->B * s->H > (long)kMaxGrid * 4)
    return fail(DSSM_ERR_UNSUPPORTED, "B*H=%ld exceeds %ld", (long)s->B * s->H, (long)kMaxGrid * 4);
  if ((rc = hip_check(launch_step(u_t, p->log_re, p->log_im, p->W, p->D, s->B, s->H, s->N, x, y_t,
                                  static_cast<hipStream_t>(stream)),
                      "step launch")))
    return rc;
  return ok();
}

int dssm_forward_fft_timed(const float* u, const dssm_dlr_params* p, const dssm_shape* s,
                           float* y, void* ws, size_t ws_bytes, void* stream,
                           void* const* events, int n_events) {
  if (!events) return fail(DSSM_ERR_INVALID_ARG, "events is NULL");
  return forward_impl(DSSM_OP_FFT, u, p, s, y, ws, ws_bytes, stream, events, n_events);
}

int dssm_forward_scan_timed(const float* u, const dssm_dlr_params* p, const dssm_shape* s,
                            float* y, void* ws, size_t ws_bytes, void* stream,
                            void* const* events, int n_events) {
  if (!events) return fail(DSSM_ERR_INVALID_ARG, "events is NULL");
  return forward_impl(DSSM_OP_SCAN, u, p, s, y, ws, ws_bytes, stream, events, n_events);
}

// ---------------------------------------------------------------------------
// S5
// ---------------------------------------------------------------------------
static int s5_check_shape(const dssm_s5_shape* s, bool* empty) {
  if (!s) return fail(DSSM_ERR_INVALID_ARG, "shape is NULL");
  if (s->B < 0 || s->H < 0 || s->L < 0)
    return fail(DSSM_ERR_INVALID_ARG, "negative dimension (B=%d H=%d L=%d)", s->B, s->H, s->L);
  if (s->P < 1) return fail(DSSM_ERR_INVALID_ARG, "P must be >= 1 (got %d)", s->P);
  if (s->bidirectional != 0 && s->bidirectional != 1)
    return fail(DSSM_ERR_INVALID_ARG, "bidirectional must be 0 or 1 (got %d)", s->bidirectional);
  if (s->bidirectional)
    return fail(DSSM_ERR_UNSUPPORTED, "the S5 layer has no bidirectional form here");
  if (s->P > kMaxN) return fail(DSSM_ERR_UNSUPPORTED, "P=%d exceeds %d", s->P, kMaxN);
  if (s->H > kMaxGrid * 64) return fail(DSSM_ERR_UNSUPPORTED, "H=%d too large", s->H);
  if (s->B > kMaxGrid) return fail(DSSM_ERR_UNSUPPORTED, "B=%d exceeds %d", s->B, kMaxGrid);
  if (s->L > kMaxLScan) return fail(DSSM_ERR_UNSUPPORTED, "L=%d exceeds %d", s->L, kMaxLScan);
  if ((long)s->B * s->P > (1L << 31) - 1) return fail(DSSM_ERR_UNSUPPORTED, "B*P too large");
  if ((long)s->B * (s->H > 2 * s->P ? s->H : 2 * s->P) * s->L > (1L << 40))
    return fail(DSSM_ERR_UNSUPPORTED, "problem too large");
  *empty = s->B == 0 || s->H == 0 || s->L == 0;
  return DSSM_OK;
}

static S5Form s5_form(int method) {
  return method == DSSM_S5_FFT ? kS5Conv : method == DSSM_S5_FUSED ? kS5Fused : kS5Unfused;
}

static int s5_check_method(int method, const dssm_s5_shape* s) {
  if (method != DSSM_S5_SCAN && method != DSSM_S5_FFT && method != DSSM_S5_FUSED)
    return fail(DSSM_ERR_INVALID_ARG,
                "method must be DSSM_S5_SCAN (0), DSSM_S5_FFT (1) or DSSM_S5_FUSED (2), got %d",
                method);
  if (method == DSSM_S5_FUSED && !s5_fused_supported(s->H, s->P, s->L))
    return fail(DSSM_ERR_UNSUPPORTED,
                "the fused S5 form needs P <= 128, H <= 256 and H L <= 2^29 (got P=%d H=%d L=%d); "
                "use DSSM_S5_SCAN",
                s->P, s->H, s->L);
  if (method == DSSM_S5_FFT && s->L > kMaxFFTL)
    return fail(DSSM_ERR_UNSUPPORTED,
                "the S5 convolution view needs L <= %d (got %d); use DSSM_S5_SCAN", kMaxFFTL, s->L);
  return DSSM_OK;
}

static int s5_workspace(const dssm_s5_shape* s, int method, size_t* bytes) {
  bool empty = false;
  int rc = s5_check_shape(s, &empty);
  if (rc) return rc;
  if ((rc = s5_check_method(method, s))) return rc;
  *bytes = empty ? 0 : s5_layout(s->B, s->H, s->P, s->L, s5_form(method)).total;
  return ok();
}

static int s5_impl(const float* u, const dssm_s5_params* p, const dssm_s5_shape* s, int method,
                   float* y, void* ws, size_t ws_bytes, void* stream, void* const* events,
                   int n_events) {
  bool empty = false;
  int rc = s5_check_shape(s, &empty);
  if (rc) return rc;
  if ((rc = s5_check_method(method, s))) return rc;
  if (events && n_events != 8)
    return fail(DSSM_ERR_INVALID_ARG, "n_events must be 8 (got %d)", n_events);
  if (empty) return ok();
  if (!p) return fail(DSSM_ERR_INVALID_ARG, "params is NULL");
  if (!p->lambda || !p->Bbar || !p->C || !p->D)
    return fail(DSSM_ERR_INVALID_ARG, "a parameter pointer is NULL");
  if (!aligned16(p->lambda) || !aligned16(p->Bbar) || !aligned16(p->C) || !aligned16(p->D))
    return fail(DSSM_ERR_INVALID_ARG, "parameter pointers must be 16-byte aligned");
  if (!u || !y || !aligned16(u) || !aligned16(y))
    return fail(DSSM_ERR_INVALID_ARG, "u or y is NULL or not 16-byte aligned");
  if (u == y) return fail(DSSM_ERR_INVALID_ARG, "y must not alias u");
  if ((rc = check_events(events, n_events))) return rc;
  const bool fft = method == DSSM_S5_FFT;
  const S5Layout l = s5_layout(s->B, s->H, s->P, s->L, s5_form(method));
  if (ws_bytes < l.total)
    return fail(DSSM_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                ws_bytes, l.total);
  if (!ws) return fail(DSSM_ERR_INVALID_ARG, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(DSSM_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* apk_in = at<unsigned char>(ws, l.apk_in);
  void* apk_out = at<unsigned char>(ws, l.apk_out);
  int* rexp_in = at<int>(ws, l.rexp_in);
  int* rexp_out = at<int>(ws, l.rexp_out);
  float* v = at<float>(ws, l.v);
  float* x = at<float>(ws, l.x);
  const bool fused = method == DSSM_S5_FUSED;
  if ((rc = hip_check(launch_s5_pack(p->Bbar, p->C, s->H, s->P, apk_in, rexp_in, apk_out,
                                     rexp_out, st, kev(events, 0), fused),
                      "s5 pack")))
    return rc;
  if (fused) {
    // v and x on chip: the powers of lambda, the state-only pass, then the
    // output pass (which joins the segment states)
    if ((rc = hip_check(launch_s5_fused(apk_in, rexp_in, apk_out, rexp_out, p->lambda, p->D, u,
                                        s->B, s->H, s->P, s->L, y, at<float2>(ws, l.sout),
                                        at<unsigned char>(ws, l.fconst), st, kev(events, 2),
                                        kev(events, 1), kev(events, 3)),
                        "s5 fused")))
      return rc;
    return ok();
  }
  if ((rc = hip_check(
           launch_s5_proj_in(apk_in, rexp_in, u, s->B, s->H, s->P, s->L, v, st, kev(events, 1)),
           "s5 proj_in")))
    return rc;
  if (fft) {
    // x_p = (lambda_p^j) * v_p: the spectrum of the powers, then the
    // convolution of every complex row (stage 2 spans both kernels)
    const KEvents e2 = kev(events, 2);
    const int log2m = fft_log2m(s->L);
    float2* spec = at<float2>(ws, l.spec);
    if ((rc = hip_check(launch_s5_spectrum(p->lambda, s->P, log2m, spec, st,
                                           KEvents{e2.start, nullptr}),
                        "s5 spectrum")))
      return rc;
    if ((rc = hip_check(launch_s5_conv(v, spec, s->B, s->P, s->L, log2m, x, st,
                                       KEvents{nullptr, e2.stop}),
                        "s5 conv")))
      return rc;
  } else if ((rc = hip_check(launch_s5_scan(p->lambda, v, s->B, s->P, s->L, x, st, kev(events, 2)),
                             "s5 scan"))) {
    return rc;
  }
  if ((rc = hip_check(launch_s5_proj_out(apk_out, rexp_out, x, p->D, u, s->B, s->H, s->P, s->L,
                                         y, st, kev(events, 3)),
                      "s5 proj_out")))
    return rc;
  return ok();
}

int dssm_s5_forward_tv(const float* u, const dssm_s5_tv_params* p, const dssm_s5_shape* s,
                       const float* step, float* y, void* ws, size_t ws_bytes, void* stream) {
  bool empty = false;
  int rc = s5_check_shape(s, &empty);
  if (rc) return rc;
  if (empty) return ok();
  if (!p) return fail(DSSM_ERR_INVALID_ARG, "params is NULL");
  if (!p->lambda_c || !p->Btilde || !p->C || !p->D || !p->delta)
    return fail(DSSM_ERR_INVALID_ARG, "a parameter pointer is NULL");
  if (!aligned16(p->lambda_c) || !aligned16(p->Btilde) || !aligned16(p->C) || !aligned16(p->D) ||
      !aligned16(p->delta))
    return fail(DSSM_ERR_INVALID_ARG, "parameter pointers must be 16-byte aligned");
  if (!u || !y || !step || !aligned16(u) || !aligned16(y) || !aligned16(step))
    return fail(DSSM_ERR_INVALID_ARG, "u, step or y is NULL or not 16-byte aligned");
  if (u == y || step == y) return fail(DSSM_ERR_INVALID_ARG, "y must not alias u or step");
  const S5Layout l = s5_layout(s->B, s->H, s->P, s->L, kS5Unfused);
  if (ws_bytes < l.total)
    return fail(DSSM_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                ws_bytes, l.total);
  if (!ws) return fail(DSSM_ERR_INVALID_ARG, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(DSSM_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* apk_in = at<unsigned char>(ws, l.apk_in);
  void* apk_out = at<unsigned char>(ws, l.apk_out);
  int* rexp_in = at<int>(ws, l.rexp_in);
  int* rexp_out = at<int>(ws, l.rexp_out);
  float* v = at<float>(ws, l.v);
  float* x = at<float>(ws, l.x);
  if ((rc = hip_check(launch_s5_pack(p->Btilde, p->C, s->H, s->P, apk_in, rexp_in, apk_out,
                                     rexp_out, st),
                      "s5 pack")))
    return rc;
  if ((rc = hip_check(launch_s5_proj_in(apk_in, rexp_in, u, s->B, s->H, s->P, s->L, v, st),
                      "s5 proj_in")))
    return rc;
  if ((rc = hip_check(launch_s5_scan_tv(p->lambda_c, p->delta, step, v, s->B, s->P, s->L, x, st),
                      "s5 scan")))
    return rc;
  if ((rc = hip_check(launch_s5_proj_out(apk_out, rexp_out, x, p->D, u, s->B, s->H, s->P, s->L,
                                         y, st),
                      "s5 proj_out")))
    return rc;
  return ok();
}

int dssm_s5_workspace_size(const dssm_s5_shape* s, int method, size_t* bytes) {
  if (!bytes) return fail(DSSM_ERR_INVALID_ARG, "bytes is NULL");
  return s5_workspace(s, method, bytes);
}

int dssm_s5_tv_workspace_size(const dssm_s5_shape* s, size_t* bytes) {
  if (!bytes) return fail(DSSM_ERR_INVALID_ARG, "bytes is NULL");
  bool empty = false;
  const int rc = s5_check_shape(s, &empty);
  if (rc) return rc;
  *bytes = empty ? 0 : s5_layout(s->B, s->H, s->P, s->L, kS5Unfused).total;
  return ok();
}

int dssm_s5_forward(const float* u, const dssm_s5_params* p, const dssm_s5_shape* s, int method,
                    float* y, void* ws, size_t ws_bytes, void* stream) {
  return s5_impl(u, p, s, method, y, ws, ws_bytes, stream, nullptr, 0);
}

int dssm_s5_forward_timed(const float* u, const dssm_s5_params* p, const dssm_s5_shape* s,
                          int method, float* y, void* ws, size_t ws_bytes, void* stream,
                          void* const* events, int n_events) {
  if (!events) return fail(DSSM_ERR_INVALID_ARG, "events is NULL");
  return s5_impl(u, p, s, method, y, ws, ws_bytes, stream, events, n_events);
}

}  // extern "C"
