// Recurrence view of the DLR bank, as a chunked parallel scan.
//
// What is computed ("The Annotated S4", Part 1, "Discrete-time SSM: the
// recurrent representation", with the DLR of "Simplifying and Understanding
// State Space Models with Diagonal Linear RNNs", section 2):
//
//   x_k = lambda x_{k-1} + u_k   (every mode driven by u, x_{-1} = 0)
//   y_k = Re(sum_n W_n x_{k,n}) + D u_k
//
// and, for the bidirectional form, the same recurrence over k = L-1 .. 0 with
// the second parameter set, added.  The linear recurrence is an associative
// scan ("Simplified State Space Layers for Sequence Modeling", section 2.2:
// (a, b) o (a', b') = (a a', a' b + b')); for a diagonal state it runs per mode.
//
// How (MI355X design): one channel's time axis is split into segments of SEG
// steps, one per lane.  All lanes of a workgroup belong to the same channel h,
// so lambda, W and the carry multipliers are wave-uniform scalars, and the
// modes are a sequential loop with the segment's u and y in registers:
//   1. each lane runs its segment from a zero state -> end state;
//   2. a Hillis-Steele scan across the lanes of the channel combines end
//      states with multipliers lambda^(SEG 2^j) (shuffles inside a wave, LDS
//      across waves);
//   3. each lane re-runs its segment from its carry-in and accumulates
//      Re(W x) into y.
// Sequences longer than one tile (SEG x lanes-per-channel steps) carry the
// per-mode state between tiles through the workspace.  Multipliers come from
// float64 arithmetic rounded once, so no float32 power chain is longer than
// SEG steps.
#include <algorithm>

#include "dssm_internal.h"

namespace dssm {
namespace {

constexpr int kScanThreads = 256;
constexpr int kMaxLevels = 8;  // up to 256 lanes per channel
// consts layout per (d,h,n): lam(2) W(2) mu_j = lambda^(SEG 2^j) (2 each, j<8)
constexpr int kNConst = 4 + 2 * kMaxLevels;

__device__ __forceinline__ float2 cmulf(float2 a, float2 b) {
  return make_float2(fmaf(a.x, b.x, -a.y * b.y), fmaf(a.x, b.y, a.y * b.x));
}

__global__ __launch_bounds__(256) void scan_consts_kernel(const float* __restrict__ log_re,
                                                          const float* __restrict__ log_im,
                                                          const float2* __restrict__ W, int ndhn,
                                                          int seg, float* __restrict__ consts) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= ndhn) return;
  const double re = (double)log_re[i];
  const double a = -re * re;
  const double th = (double)log_im[i];
  float* c = consts + (size_t)i * kNConst;
  double s, co;
  sincos(th, &s, &co);
  const double m = exp(a);
  c[0] = (float)(m * co);
  c[1] = (float)(m * s);
  c[2] = W[i].x;
  c[3] = W[i].y;
  for (int j = 0; j < kMaxLevels; ++j) {
    const double k = (double)seg * (double)(1 << j);  // exact; k * th exact in float64
    sincos(k * th, &s, &co);
    const double mk = exp(k * a);
    c[4 + 2 * j] = (float)(mk * co);
    c[5 + 2 * j] = (float)(mk * s);
  }
}

// One direction of one mode over the current tile.
//   uu/yy: this lane's SEG inputs / output accumulators (positions ascending).
//   carry_ptr: per-(channel, mode) state entering the tile (read if
//   use_carry) and leaving it (written by the channel's last lane if
//   write_carry).
// Lanes of a channel are numbered along the scan direction ("virtual" lanes);
// they form blocks of up to 64 inside one wave.  Within a block the scan uses
// shuffles; blocks of a channel spanning several waves are chained through LDS.
template <int SEG, bool REV>
__device__ __forceinline__ void scan_mode(const float* uu, float* yy, const float* __restrict__ cst,
                                          int cl, int lpc, float2* xs, float2* carry_ptr,
                                          bool use_carry, bool write_carry) {
  const float2 lam = make_float2(cst[0], cst[1]);
  const float2 w = make_float2(cst[2], cst[3]);

  // 1. local end state from a zero start
  float2 x = make_float2(0.f, 0.f);
#pragma unroll
  for (int i = 0; i < SEG; ++i) {
    const float uv = uu[REV ? SEG - 1 - i : i];
    x = make_float2(fmaf(lam.x, x.x, fmaf(-lam.y, x.y, uv)), fmaf(lam.x, x.y, lam.y * x.x));
  }
  const int vl = REV ? lpc - 1 - cl : cl;  // virtual lane along the scan
  const int wb = lpc < 64 ? lpc : 64;      // virtual lanes per block
  const int vlw = vl & (wb - 1);           // virtual lane inside its block
  const int lane = threadIdx.x & 63;
  float2 cin = make_float2(0.f, 0.f);
  if (use_carry) {
    cin = *carry_ptr;
    if (vl == 0) {  // the tile's first segment starts from the carried state
      const float2 t = cmulf(make_float2(cst[4], cst[5]), cin);
      x.x += t.x;
      x.y += t.y;
    }
  }
  // 2a. inclusive scan inside the block: X(v) = sum_{v' <= v} mu^(v - v') x(v')
  for (int j = 0; (1 << j) < wb; ++j) {
    const int o = 1 << j;
    const int src = min(max(REV ? lane + o : lane - o, 0), 63);
    float2 p;
    p.x = __shfl(x.x, src);
    p.y = __shfl(x.y, src);
    if (vlw >= o) {
      const float2 t = cmulf(make_float2(cst[4 + 2 * j], cst[5 + 2 * j]), p);
      x.x += t.x;
      x.y += t.y;
    }
  }
  // 2b. blocks of one channel in different waves: carry into block vb is
  //     C = sum_{k < vb} nu^(vb-1-k) X_k(last), nu = lambda^(64 SEG); each lane
  //     adds mu^(vlw+1) C.
  float2 cblk = make_float2(0.f, 0.f);
  if (lpc > 64) {
    const int vb = vl >> 6;
    const int ch = threadIdx.x / lpc;
    __syncthreads();
    if (vlw == 63) xs[ch * 4 + vb] = x;
    __syncthreads();
    const float2 nu = make_float2(cst[4 + 12], cst[5 + 12]);
    for (int k = 0; k < vb; ++k) {
      const float2 t = cmulf(nu, cblk);
      const float2 xk = xs[ch * 4 + k];
      cblk = make_float2(t.x + xk.x, t.y + xk.y);
    }
    float2 pw = make_float2(1.f, 0.f);
    const int e = vlw + 1;
#pragma unroll
    for (int j = 0; j < 7; ++j)
      if ((e >> j) & 1) pw = cmulf(pw, make_float2(cst[4 + 2 * j], cst[5 + 2 * j]));
    const float2 t = cmulf(pw, cblk);
    x.x += t.x;
    x.y += t.y;
  }
  // exclusive carry-in: the previous virtual lane's inclusive state
  float2 xin;
  {
    const int src = min(max(REV ? lane + 1 : lane - 1, 0), 63);
    float2 p;
    p.x = __shfl(x.x, src);
    p.y = __shfl(x.y, src);
    xin = (vl == 0) ? cin : ((vlw == 0) ? cblk : p);
  }
  if (write_carry && vl == lpc - 1) *carry_ptr = x;  // state leaving the tile
  // 3. outputs from the true carry-in
  x = xin;
#pragma unroll
  for (int i = 0; i < SEG; ++i) {
    const int s = REV ? SEG - 1 - i : i;
    const float uv = uu[s];
    x = make_float2(fmaf(lam.x, x.x, fmaf(-lam.y, x.y, uv)), fmaf(lam.x, x.y, lam.y * x.x));
    yy[s] = fmaf(w.x, x.x, fmaf(-w.y, x.y, yy[s]));
  }
}

// Grid: (channel groups of one h) x H.  Workgroup = 256 lanes = cpg channels
// (batch rows b0 .. b0+cpg-1 of channel h) x lpc lanes.
template <int SEG>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(
    const float* __restrict__ u, const float* __restrict__ consts, const float* __restrict__ D,
    float2* __restrict__ carry, int B, int H, int N, int L, int ndir, int lpc, int ntile,
    float* __restrict__ y) {
  __shared__ float2 xs[8];  // block totals: 2 channels x 4 blocks at most
  const int cpg = kScanThreads / lpc;
  const int h = blockIdx.y;
  const int cl = threadIdx.x % lpc;
  const int b = blockIdx.x * cpg + threadIdx.x / lpc;
  const bool active = b < B;
  const int tile = SEG * lpc;
  const float* uc = u + ((size_t)(active ? b : 0) * H + h) * L;
  float* yc = y + ((size_t)(active ? b : 0) * H + h) * L;
  float2* cc = carry + ((size_t)(active ? b : 0) * H + h) * N;
  float deff = 0.f;
  for (int d = 0; d < ndir; ++d) deff += D[(size_t)d * H + h];

  float uu[SEG], yy[SEG];
  auto load_u = [&](int t) {
    const int p0 = t * tile + cl * SEG;
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
      const int p = p0 + i;
      uu[i] = (active && p < L) ? uc[p] : 0.f;
    }
  };
  auto store_y = [&](int t) {
    const int p0 = t * tile + cl * SEG;
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
      const int p = p0 + i;
      if (active && p < L) yc[p] = yy[i];
    }
  };

  if (ntile == 1) {
    load_u(0);
#pragma unroll
    for (int i = 0; i < SEG; ++i) yy[i] = deff * uu[i];
    for (int d = 0; d < ndir; ++d) {
      const float* cst0 = consts + ((size_t)d * H + h) * N * kNConst;
      for (int n = 0; n < N; ++n) {
        if (d == 0)
          scan_mode<SEG, false>(uu, yy, cst0 + (size_t)n * kNConst, cl, lpc, xs, nullptr, false, false);
        else
          scan_mode<SEG, true>(uu, yy, cst0 + (size_t)n * kNConst, cl, lpc, xs, nullptr, false, false);
      }
    }
    store_y(0);
    return;
  }

  // Several tiles: the state of each mode is carried between tiles through
  // `carry`; the backward direction walks the tiles in reverse and adds to y.
  for (int d = 0; d < ndir; ++d) {
    const float* cst0 = consts + ((size_t)d * H + h) * N * kNConst;
    for (int k = 0; k < ntile; ++k) {
      const int t = d == 0 ? k : ntile - 1 - k;
      load_u(t);
      if (d == 0) {
#pragma unroll
        for (int i = 0; i < SEG; ++i) yy[i] = deff * uu[i];
      } else {
        const int p0 = t * tile + cl * SEG;
#pragma unroll
        for (int i = 0; i < SEG; ++i) yy[i] = (active && p0 + i < L) ? yc[p0 + i] : 0.f;
      }
      for (int n = 0; n < N; ++n) {
        // lanes of one channel read the carry written by its last lane in the
        // previous tile; a barrier orders the write and the reads
        __syncthreads();
        if (d == 0)
          scan_mode<SEG, false>(uu, yy, cst0 + (size_t)n * kNConst, cl, lpc, xs, cc + n, k > 0,
                                active);
        else
          scan_mode<SEG, true>(uu, yy, cst0 + (size_t)n * kNConst, cl, lpc, xs, cc + n, k > 0,
                               active);
      }
      store_y(t);
      __syncthreads();
    }
  }
}

template <int SEG>
void scan_launch(const float* u, const float* consts, const float* D, float2* carry, int B, int H,
                 int N, int L, int ndir, const ScanPlan& plan, float* y, hipStream_t st) {
  const int cpg = kScanThreads / plan.lpc;
  const dim3 grid((unsigned)((B + cpg - 1) / cpg), (unsigned)H);
  hipLaunchKernelGGL(scan_kernel<SEG>, grid, dim3(kScanThreads), 0, st, u, consts, D, carry, B, H,
                     N, L, ndir, plan.lpc, plan.ntile, y);
}

}  // namespace

ScanPlan scan_plan(int B, int L) {
  (void)B;
  ScanPlan p;
  // segment length: L/16 rounded up to a power of two, within [4, 64]
  int seg = 4;
  while (seg < 64 && seg * 16 < L) seg *= 2;
  int lpc = 1;
  while (lpc < 256 && lpc * seg < L) lpc *= 2;
  p.seg = seg;
  p.lpc = lpc;
  p.cpw = lpc < 64 ? 64 / lpc : 1;
  p.waves = kScanThreads / 64;
  p.tile = seg * lpc;
  p.ntile = (L + p.tile - 1) / p.tile;
  p.nconst = kNConst;
  return p;
}

hipError_t launch_scan_consts(const float* log_re, const float* log_im, const float* W, int ndh,
                              int N, const ScanPlan& plan, float* consts, hipStream_t st) {
  const int ndhn = ndh * N;
  hipLaunchKernelGGL(scan_consts_kernel, dim3((unsigned)((ndhn + 255) / 256)), dim3(256), 0, st,
                     log_re, log_im, reinterpret_cast<const float2*>(W), ndhn, plan.seg, consts);
  return hipGetLastError();
}

hipError_t launch_scan(const float* u, const float* consts, const float* D, int B, int H, int N,
                       int L, int ndir, const ScanPlan& plan, float* y, hipStream_t st,
                       float2* carry) {
  switch (plan.seg) {
    case 4: scan_launch<4>(u, consts, D, carry, B, H, N, L, ndir, plan, y, st); break;
    case 8: scan_launch<8>(u, consts, D, carry, B, H, N, L, ndir, plan, y, st); break;
    case 16: scan_launch<16>(u, consts, D, carry, B, H, N, L, ndir, plan, y, st); break;
    case 32: scan_launch<32>(u, consts, D, carry, B, H, N, L, ndir, plan, y, st); break;
    case 64: scan_launch<64>(u, consts, D, carry, B, H, N, L, ndir, plan, y, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dssm
