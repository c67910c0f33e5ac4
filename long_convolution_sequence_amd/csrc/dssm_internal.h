// Internal declarations shared by the host entry points (api.hip) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dssm {

// Optional pair of caller-owned events that the GPU stamps at the start and
// the end of one kernel (hipExtLaunchKernel): timing of that kernel alone,
// without the dispatch gap before it.
struct KEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Launch `k` on `st`, stamping `ev` around it when given (a plain launch
// otherwise).
template <typename... KArgs, typename... Args>
inline void launch_k(void (*k)(KArgs...), dim3 grid, dim3 block, hipStream_t st, KEvents ev,
                     Args... args) {
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(k, grid, block, 0, st, ev.start, ev.stop, 0,
                          static_cast<KArgs>(args)...);
  else
    hipLaunchKernelGGL(k, grid, block, 0, st, static_cast<KArgs>(args)...);
}

// Anchor spacing of the kernel generator: K[64 q + r] is built from
// lambda^r (r < 64) and the anchor W lambda^(64 q).
constexpr int kAnchor = 64;
// Largest FFT half-length: the circle has length 2M <= 32768, the complex
// half-length transform holds M <= 16384 points in one workgroup's LDS.
constexpr int kMaxLog2M = 14;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// Phase cycle stamps, compiled in only by `build.py --phase-stamps` (which
// defines DSSM_PHASE_STAMPS and writes libdssm_stamps.so beside the library;
// the library proper has none).  A kernel reads the shader-clock counter
// (s_memtime) at its phase boundaries and adds each phase's cycles to a
// register slot; at its end lane 0 of every wave writes the slots to the
// buffer set for that source file (dssm_phase_stamps_fft / _chunk / _gen):
//   buf[(workgroup * waves + wave) * kPhaseSlots + slot], workgroups numbered
//   x fastest.
// Nothing is stored before the end, so the stamps add no memory waits to the
// phases they time.
// ---------------------------------------------------------------------------
constexpr int kPhaseSlots = 16;
#ifdef DSSM_PHASE_STAMPS
static __device__ unsigned long long* g_phase_buf = nullptr;
struct PhaseClock {
  unsigned long long acc[kPhaseSlots];
  unsigned long long last;
  __device__ PhaseClock() : last(__builtin_amdgcn_s_memtime()) {
    for (int k = 0; k < kPhaseSlots; ++k) acc[k] = 0;
  }
  __device__ void mark(int k) {
    const unsigned long long now = __builtin_amdgcn_s_memtime();
    acc[k] += now - last;
    last = now;
  }
  __device__ void write() const {
    if (g_phase_buf && (threadIdx.x & 63) == 0) {
      const size_t wg = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
      const size_t base = (wg * (blockDim.x >> 6) + (threadIdx.x >> 6)) * kPhaseSlots;
      for (int k = 0; k < kPhaseSlots; ++k) g_phase_buf[base + k] = acc[k];
    }
  }
};
#else
struct PhaseClock {
  __device__ void mark(int) {}
  __device__ void write() const {}
};
#endif

// ---------------------------------------------------------------------------
// Kernel generation (eig_gen.hip)
// ---------------------------------------------------------------------------
// K[dh, j] = sum_n W[dh,n] lambda[dh,n]^j for j < L, from the parameters
// directly (float64 powers, split-fp16 matrix-core contraction over the modes).
// out = kGenRe: Re K into float [ndh, L]; kGenComplex: (Re, Im) into float2
// [ndh, L]; kGenReIm: Re K * Im K into float [ndh, L].
constexpr int kGenRe = 0, kGenComplex = 1, kGenReIm = 2;
hipError_t launch_gen(const float* log_re, const float* log_im, const float* W, int ndh, int N,
                      int L, int out, float* K, hipStream_t st, KEvents ev = {});

// ---------------------------------------------------------------------------
// FFT convolution (fft.hip)
// ---------------------------------------------------------------------------
// Spectrum tables: spec[h, half, M] float2 in transform order (the order the
// in-place decimation-in-frequency passes leave the bins in; the bin at
// position 16 t + r is stored at r M/16 + t), scaled by 1/(2M).  half 0 holds
// the even bins of the 2M-point transform of the zero-padded real kernel,
// half 1 the odd bins.  For ndir = 2 the backward kernel enters conjugated.
// sum_d D[d,h] is added to every bin (the feed-through as tap 0); D may be
// NULL.  conj != 0 writes the conjugate table (the transposed operator).
hipError_t launch_spectrum(const float* reK, const float* D, int ndir, int H, int L, int log2m,
                           float2* spec, hipStream_t st, KEvents ev = {}, int conj = 0);

// y[b,h,:L] = first L samples of the 2M-circular convolution of u[b,h,:] with
// the kernel whose spectrum is spec[h] (D u included through tap 0).
hipError_t launch_conv(const float* u, const float2* spec, int B, int H, int L, int log2m, float* y,
                       hipStream_t st, KEvents ev = {});

int fft_log2m(int L);  // log2 of M = max(16, next power of two >= L)

// S5 convolution view: spec [P][2][M] float2 (full storage, the bin at
// position 16 t + r of half `half` at slot r M/16 + t) holds the spectrum of
// lambda_p^j (j < M) on the 2M circle, scaled by 1/(2M), in float64 rounded
// once.  launch_s5_conv: x [B][P][2][L] (real row, imaginary row) = the
// causal convolution of v [B][P][2][L] with lambda_p^j.
hipError_t launch_s5_spectrum(const float* lambda, int P, int log2m, float2* spec,
                              hipStream_t st, KEvents ev = {});
hipError_t launch_s5_conv(const float* v, const float2* spec, int B, int P, int L, int log2m,
                          float* x, hipStream_t st, KEvents ev = {});

// Kernel cotangents for the gradients, summed over the batch: part [G][H][2][M]
// floats (G = corr_groups(B, H) batch groups) such that, for j < L,
//   sum_b sum_i u[b,h,i] dy[b,h,i+j] = sum_g part[g][h][0][j] + part[g][h][1][j],
//   sum_b sum_i dy[b,h,i] u[b,h,i+j] = sum_g part[g][h][0][M-j] - part[g][h][1][M-j] (j >= 1).
int corr_groups(int B, int H);
hipError_t launch_corr(const float* u, const float* dy, int B, int H, int L, int log2m,
                       float* part, hipStream_t st);

// ---------------------------------------------------------------------------
// Parameter gradients from kernel cotangents (grad.hip)
// ---------------------------------------------------------------------------
// part [G][H][2][M]: the halves of the batch-summed lagged correlations
// (launch_corr).  parts: grad_splits(L) * ndir * H * N * 2 double2.
int grad_splits(int L);
hipError_t launch_grad_params(const float* part, int M, int G, int H, int L, const float* log_re,
                              const float* log_im, const float* W, int N, int ndir, void* parts,
                              float* dlog_re, float* dlog_im, float* dW, float* dD,
                              hipStream_t st);
// The four gradient arrays of ndh = ndir H channels set to zero.
hipError_t launch_zero_grads(float* dlog_re, float* dlog_im, float* dW, float* dD, int ndh, int N,
                             hipStream_t st);

// ---------------------------------------------------------------------------
// Recurrence scan (scan.hip)
// ---------------------------------------------------------------------------
struct ScanPlan {
  int seg;        // time steps per lane
  int lpc;        // lanes per channel (power of two, <= 256)
  int cpw;        // channels per wave (64 / lpc when lpc < 64, else 1)
  int waves;      // waves per workgroup
  int tile;       // time steps covered per tile = seg * lpc
  int ntile;      // tiles per channel
  int nconst;     // floats per (d,h,n) in the constant table
};
ScanPlan scan_plan(int B, int L);

// Per-(d,h,n) constants for the scan (float64 arithmetic, rounded once).
hipError_t launch_scan_consts(const float* log_re, const float* log_im, const float* W,
                             int ndh, int N, const ScanPlan& plan, float* consts, hipStream_t st,
                             KEvents ev = {});

// carry: [B, H, N] float2 scratch, used when plan.ntile > 1.  state (one
// direction): carry holds x_{-1} on entry and receives x_{L-1}.
hipError_t launch_scan(const float* u, const float* consts, const float* D, int B, int H, int N,
                       int L, int ndir, const ScanPlan& plan, float* y, hipStream_t st,
                       float2* carry, KEvents ev = {}, bool state = false);

// One token for every (b, h): x [B,H,N] c64 updated in place, y_t [B,H] from
// u_t [B,H].
hipError_t launch_step(const float* u, const float* log_re, const float* log_im, const float* W,
                       const float* D, int B, int H, int N, float* x, float* y, hipStream_t st);

// ---------------------------------------------------------------------------
// Chunked state-space form on the matrix cores (chunk.hip)
// ---------------------------------------------------------------------------
bool chunk_supported(int N);  // N <= 64 modes
// How a launch is organised: rpw batch rows of a channel per workgroup (the
// operands built once), and nseg segments of seg_blocks blocks of 4096 steps
// per row when rows are too few to fill the device.
struct ChunkPlan {
  int rpw = 1, nseg = 1, seg_blocks = 1;
};
ChunkPlan chunk_plan(int B, int H, int L, int ndir);
// Workspace bytes of launch_chunk (0 unless the sequence is split).
size_t chunk_workspace(int B, int H, int N, int L, int ndir);
// y [B,H,L] from u [B,H,L]; the second direction (if any) in reversed time.
// x0 [B,H,N] c64 (may be NULL): the state before step 0 (one direction);
// xend [B,H,N] c64 (may be NULL): receives the state after step L-1 (one
// direction); x0 and xend may be the same array.  ws: chunk_workspace bytes.
hipError_t launch_chunk(const float* u, const float* log_re, const float* log_im, const float* W,
                        const float* D, int B, int H, int N, int L, int ndir, float* y,
                        const float* x0, float* xend, void* ws, hipStream_t st, KEvents ev = {});

// ---------------------------------------------------------------------------
// S5 multi-input multi-output diagonal SSM (s5.hip)
// ---------------------------------------------------------------------------
struct S5Layout {
  size_t apk_in = 0, rexp_in = 0, apk_out = 0, rexp_out = 0, v = 0, x = 0, spec = 0, sout = 0,
         fconst = 0, total = 0;
};
// Which regions a call needs besides the packed fragments:
//   kS5Unfused: v and x (the scan between the projections, also with a step
//     size per step);
//   kS5Conv: v, x and the convolution view's spectrum table [P][2][M] float2;
//   kS5Fused: the fused form's segment states and powers of lambda (the
//     fragments in its layout; requires s5_fused_supported).
enum S5Form { kS5Unfused = 1, kS5Conv = 2, kS5Fused = 3 };
S5Layout s5_layout(int B, int H, int P, int L, S5Form form);

// Bbar [P,H] c64, C [H,P] c64 -> split MFMA fragment tables (16-byte aligned)
// and per-row scale exponents.
// fused: the layout of the fused form: Bbar's rows in its order (per 32
// rows, the real then the imaginary rows of 16 states; 32 ceil(P / 16) rows),
// both kinds zero-padded to 32 s5_fused_ks(H, P) columns.
hipError_t launch_s5_pack(const float* Bbar, const float* C, int H, int P, void* apk_in,
                          int* rexp_in, void* apk_out, int* rexp_out, hipStream_t st,
                          KEvents ev = {}, bool fused = false);
// v [B][P][2][L] = Bbar u
hipError_t launch_s5_proj_in(const void* apk_in, const int* rexp_in, const float* u, int B, int H,
                             int P, int L, float* v, hipStream_t st, KEvents ev = {});
// x [B][P][2][L]: x_k = lambda x_{k-1} + v_k
hipError_t launch_s5_scan(const float* lambda, const float* v, int B, int P, int L, float* x,
                          hipStream_t st, KEvents ev = {});
// x [B][P][2][L] for the continuous-time system with per-step step sizes:
// x_k = exp(z) x_{k-1} + (exp(z) - 1) / lam_c v_k, z = lam_c[p] step[b,k] delta[p]
hipError_t launch_s5_scan_tv(const float* lam_c, const float* delta, const float* step,
                            const float* v, int B, int P, int L, float* x, hipStream_t st,
                            KEvents ev = {});
// The fused form (P <= 128, H <= 256, H L <= 2^29): y from u through the
// packed Bbar (fused row order) and C fragments, v and x kept on chip, the
// sequence of each batch row in nseg segments of seg_tiles 64-step tiles;
// sout: [B][nseg][P] c64 scratch; consts: P (32 + 16 nseg) bytes (powers of
// lambda).  Three launches, each stamped by its own event pair: the powers of
// lambda, a state-only pass, then the output pass that also joins the segment
// states (no state-only pass when nseg == 1: its pair is stamped back to back).
bool s5_fused_supported(int H, int P, int L);
// k steps (of 32) both fused products are padded to: 2, 4 or 8
int s5_fused_ks(int H, int P);
struct S5FusedPlan {
  int nseg = 1, seg_tiles = 1;
};
S5FusedPlan s5_fused_plan(int B, int L);
hipError_t launch_s5_fused(const void* apk_in, const int* rexp_in, const void* apk_out,
                           const int* rexp_out, const float* lambda, const float* D,
                           const float* u, int B, int H, int P, int L, float* y, float2* sout,
                           void* consts, hipStream_t st, KEvents ev_consts = {},
                           KEvents ev_state = {}, KEvents ev_out = {});
// y [B][H][L] = Re(C x) + D u
hipError_t launch_s5_proj_out(const void* apk_out, const int* rexp_out, const float* x,
                              const float* D, const float* u, int B, int H, int P, int L, float* y,
                              hipStream_t st, KEvents ev = {});

}  // namespace dssm
