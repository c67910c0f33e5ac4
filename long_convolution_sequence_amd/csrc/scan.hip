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

__device__ __forceinline__ float2 rec_step(float2 lam, float2 x, float u) {
  // lambda * x + u
  return make_float2(fmaf(lam.x, x.x, fmaf(-lam.y, x.y, u)), fmaf(lam.x, x.y, lam.y * x.x));
}

__device__ __forceinline__ float2 cfma(float2 m, float2 p, float2 acc) {  // acc + m p
  return make_float2(fmaf(m.x, p.x, fmaf(-m.y, p.y, acc.x)), fmaf(m.x, p.y, fmaf(m.y, p.x, acc.y)));
}

// Two modes (a, b) of one direction over the current tile: two independent
// recurrences per lane in flight.  uu/yy: this lane's SEG inputs / output
// accumulators (positions ascending); carry_a/b: per-(channel, mode) state
// entering the tile (read if use_carry) and leaving it (written by the
// channel's last lane if write_carry).  Lanes of a channel are numbered along
// the scan direction ("virtual" lanes) in blocks of up to 64 per wave: the
// scan uses shuffles inside a block and LDS between the blocks of a channel.
//
// cap_s >= 0 marks the lane holding the sequence's last position, at index
// cap_s of its segment: it writes the state after that step to the carry (the
// final state of a stateful call; a short last tile runs on past L with zero
// input, so its end state is not it).
template <int SEG, bool REV>
__device__ __forceinline__ void scan_pair(const float* uu, float* yy, const float* __restrict__ ca,
                                          const float* __restrict__ cb, bool has_b, int cl,
                                          int lpc, float4* xs, float2* carry_a, float2* carry_b,
                                          bool use_carry, bool write_carry, int cap_s = -1) {
  const float2 la = make_float2(ca[0], ca[1]);
  const float2 lb = make_float2(cb[0], cb[1]);
  const float2 wa = make_float2(ca[2], ca[3]);
  const float2 wb = has_b ? make_float2(cb[2], cb[3]) : make_float2(0.f, 0.f);

  // 1. local end states from a zero start
  float2 xa = make_float2(0.f, 0.f), xb = xa;
#pragma unroll
  for (int i = 0; i < SEG; ++i) {
    const float uv = uu[REV ? SEG - 1 - i : i];
    xa = rec_step(la, xa, uv);
    xb = rec_step(lb, xb, uv);
  }
  const int vl = REV ? lpc - 1 - cl : cl;
  const int wbk = lpc < 64 ? lpc : 64;
  const int vlw = vl & (wbk - 1);
  const int lane = threadIdx.x & 63;
  float2 cin_a = make_float2(0.f, 0.f), cin_b = cin_a;
  if (use_carry) {
    cin_a = *carry_a;
    if (has_b) cin_b = *carry_b;
    if (vl == 0) {  // the tile's first segment starts from the carried state
      xa = cfma(make_float2(ca[4], ca[5]), cin_a, xa);
      xb = cfma(make_float2(cb[4], cb[5]), cin_b, xb);
    }
  }
  // 2a. inclusive scan inside the block: X(v) = sum_{v' <= v} mu^(v - v') x(v')
  for (int j = 0; (1 << j) < wbk; ++j) {
    const int o = 1 << j;
    const int src = min(max(REV ? lane + o : lane - o, 0), 63);
    float2 pa, pb;
    pa.x = __shfl(xa.x, src);
    pa.y = __shfl(xa.y, src);
    pb.x = __shfl(xb.x, src);
    pb.y = __shfl(xb.y, src);
    if (vlw >= o) {
      xa = cfma(make_float2(ca[4 + 2 * j], ca[5 + 2 * j]), pa, xa);
      xb = cfma(make_float2(cb[4 + 2 * j], cb[5 + 2 * j]), pb, xb);
    }
  }
  // 2b. blocks of one channel in different waves: the carry into block vb is
  //     C = sum_{k < vb} nu^(vb-1-k) X_k(last), nu = lambda^(64 SEG); every
  //     lane adds mu^(vlw+1) C.
  float2 ka = make_float2(0.f, 0.f), kb = ka;
  if (lpc > 64) {
    const int vb = vl >> 6;
    const int ch = threadIdx.x / lpc;
    __syncthreads();
    if (vlw == 63) xs[ch * 4 + vb] = make_float4(xa.x, xa.y, xb.x, xb.y);
    __syncthreads();
    const float2 nua = make_float2(ca[16], ca[17]), nub = make_float2(cb[16], cb[17]);
    for (int k = 0; k < vb; ++k) {
      const float4 t = xs[ch * 4 + k];
      ka = cfma(nua, ka, make_float2(t.x, t.y));
      kb = cfma(nub, kb, make_float2(t.z, t.w));
    }
    float2 pwa = make_float2(1.f, 0.f), pwb = pwa;
    const int e = vlw + 1;
#pragma unroll
    for (int j = 0; j < 7; ++j) {
      if ((e >> j) & 1) {
        pwa = cfma(pwa, make_float2(ca[4 + 2 * j], ca[5 + 2 * j]), make_float2(0.f, 0.f));
        pwb = cfma(pwb, make_float2(cb[4 + 2 * j], cb[5 + 2 * j]), make_float2(0.f, 0.f));
      }
    }
    xa = cfma(pwa, ka, xa);
    xb = cfma(pwb, kb, xb);
  }
  // exclusive carry-in: the previous virtual lane's inclusive state
  float2 ina, inb;
  {
    const int src = min(max(REV ? lane + 1 : lane - 1, 0), 63);
    float2 pa, pb;
    pa.x = __shfl(xa.x, src);
    pa.y = __shfl(xa.y, src);
    pb.x = __shfl(xb.x, src);
    pb.y = __shfl(xb.y, src);
    ina = (vl == 0) ? cin_a : ((vlw == 0) ? ka : pa);
    inb = (vl == 0) ? cin_b : ((vlw == 0) ? kb : pb);
  }
  if (write_carry && vl == lpc - 1) {  // state leaving the tile
    *carry_a = xa;
    if (has_b) *carry_b = xb;
  }
  // 3. outputs from the true carry-in
  xa = ina;
  xb = inb;
  auto out_step = [&](int s) {
    const float uv = uu[s];
    xa = rec_step(la, xa, uv);
    xb = rec_step(lb, xb, uv);
    float acc = yy[s];
    acc = fmaf(wa.x, xa.x, acc);
    acc = fmaf(-wa.y, xa.y, acc);
    acc = fmaf(wb.x, xb.x, acc);
    acc = fmaf(-wb.y, xb.y, acc);
    yy[s] = acc;
  };
  if (__any(cap_s >= 0)) {  // wave-uniform: only the wave holding the last position pays
    float2 fa = xa, fb = xb;
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
      const int s = REV ? SEG - 1 - i : i;
      out_step(s);
      if (s == cap_s) {
        fa = xa;
        fb = xb;
      }
    }
    if (cap_s >= 0) {
      *carry_a = fa;
      if (has_b) *carry_b = fb;
    }
  } else {
#pragma unroll
    for (int i = 0; i < SEG; ++i) out_step(REV ? SEG - 1 - i : i);
  }
}

// All modes of one direction over the current tile, two at a time.
template <int SEG, bool REV>
__device__ __forceinline__ void scan_modes(const float* uu, float* yy,
                                           const float* __restrict__ cst0, int N, int cl, int lpc,
                                           float4* xs, float2* cc, bool use_carry,
                                           bool write_carry, bool sync_each, int cap_s = -1) {
  for (int n = 0; n < N; n += 2) {
    const bool has_b = n + 1 < N;
    if (sync_each) __syncthreads();  // orders the carry write and reads between tiles
    scan_pair<SEG, REV>(uu, yy, cst0 + (size_t)n * kNConst,
                        cst0 + (size_t)(has_b ? n + 1 : n) * kNConst, has_b, cl, lpc, xs,
                        cc + n, cc + (has_b ? n + 1 : n), use_carry, write_carry, cap_s);
  }
}

// Grid: (channel groups of one h) x H.  Workgroup = 256 lanes = cpg channels
// (batch rows b0 .. b0+cpg-1 of channel h) x lpc lanes.  MULTI: the sequence
// spans several tiles and carries cross them through `carry`.  state (MULTI,
// one direction): `carry` holds the state x_{-1} on entry (read by the first
// tile) and receives x_{L-1} on exit, captured at the last position.
template <int SEG, bool MULTI>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(
    const float* __restrict__ u, const float* __restrict__ consts, const float* __restrict__ D,
    float2* __restrict__ carry, int B, int H, int N, int L, int ndir, int lpc, int ntile,
    float* __restrict__ y, int state) {
  __shared__ float4 xs[8];  // block totals (two modes): 2 channels x 4 blocks at most
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
  if (!MULTI) {
    const int p0 = cl * SEG;
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
      const int p = p0 + i;
      uu[i] = (active && p < L) ? uc[p] : 0.f;
      yy[i] = deff * uu[i];
    }
    for (int d = 0; d < ndir; ++d) {
      const float* cst0 = consts + ((size_t)d * H + h) * N * kNConst;
      if (d == 0)
        scan_modes<SEG, false>(uu, yy, cst0, N, cl, lpc, xs, cc, false, false, false);
      else
        scan_modes<SEG, true>(uu, yy, cst0, N, cl, lpc, xs, cc, false, false, false);
    }
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
      const int p = p0 + i;
      if (active && p < L) yc[p] = yy[i];
    }
    return;
  }

  // Several tiles: the backward direction walks the tiles in reverse and adds
  // to the y written by the forward direction.
  for (int d = 0; d < ndir; ++d) {
    const float* cst0 = consts + ((size_t)d * H + h) * N * kNConst;
    for (int k = 0; k < ntile; ++k) {
      const int t = d == 0 ? k : ntile - 1 - k;
      const int p0 = t * tile + cl * SEG;
#pragma unroll
      for (int i = 0; i < SEG; ++i) {
        const int p = p0 + i;
        uu[i] = (active && p < L) ? uc[p] : 0.f;
        if (d == 0) yy[i] = deff * uu[i];
        else yy[i] = (active && p < L) ? yc[p] : 0.f;
      }
      const bool last = k == ntile - 1;
      const int cap_s = (state && last && active && p0 <= L - 1 && L - 1 < p0 + SEG) ? L - 1 - p0
                                                                                   : -1;
      if (d == 0)
        scan_modes<SEG, false>(uu, yy, cst0, N, cl, lpc, xs, cc, k > 0 || state,
                               active && !(state && last), true, cap_s);
      else
        scan_modes<SEG, true>(uu, yy, cst0, N, cl, lpc, xs, cc, k > 0, active, true);
#pragma unroll
      for (int i = 0; i < SEG; ++i) {
        const int p = p0 + i;
        if (active && p < L) yc[p] = yy[i];
      }
      __syncthreads();
    }
  }
}

template <int SEG>
void scan_launch(const float* u, const float* consts, const float* D, float2* carry, int B, int H,
                 int N, int L, int ndir, const ScanPlan& plan, float* y, hipStream_t st,
                 KEvents ev, bool state) {
  const int cpg = kScanThreads / plan.lpc;
  const dim3 grid((unsigned)((B + cpg - 1) / cpg), (unsigned)H);
  if (plan.ntile == 1 && !state)
    launch_k(scan_kernel<SEG, false>, grid, dim3(kScanThreads), st, ev, u, consts, D, carry, B, H, N,
             L, ndir, plan.lpc, plan.ntile, y, 0);
  else
    launch_k(scan_kernel<SEG, true>, grid, dim3(kScanThreads), st, ev, u, consts, D, carry, B, H, N,
             L, ndir, plan.lpc, plan.ntile, y, state ? 1 : 0);
}

// One time step for every (b, h), one wave each (modes across the lanes):
//   x <- lambda x + u_t,  y_t = Re(sum_n W_n x_n) + D u_t,
// the recurrent view advanced by one token ("The Annotated S4", Part 1,
// "Discrete-time SSM: the recurrent representation").  lambda is formed in
// float64 from the exactly promoted parameters and rounded once, as the scan's
// per-step multiplier is.
__global__ __launch_bounds__(256) void step_kernel(const float* __restrict__ u,
                                                   const float* __restrict__ log_re,
                                                   const float* __restrict__ log_im,
                                                   const float2* __restrict__ W,
                                                   const float* __restrict__ D, int B, int H,
                                                   int N, float2* __restrict__ x,
                                                   float* __restrict__ y) {
  const long row = ((long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;  // b H + h
  const int lane = threadIdx.x & 63;
  if (row >= (long)B * H) return;  // whole waves
  const int h = (int)(row % H);
  const float uv = u[row];
  float2* xr = x + (size_t)row * N;
  float acc = 0.f;
  for (int n = lane; n < N; n += 64) {
    const size_t i = (size_t)h * N + n;
    const double re = (double)log_re[i];
    double sn, cs;
    sincos((double)log_im[i], &sn, &cs);
    const double m = exp(-re * re);
    const float2 lam = make_float2((float)(m * cs), (float)(m * sn));
    const float2 xv = rec_step(lam, xr[n], uv);
    xr[n] = xv;
    const float2 w = W[i];
    acc = fmaf(w.x, xv.x, fmaf(-w.y, xv.y, acc));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) y[row] = fmaf(D[h], uv, acc);
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
                              int N, const ScanPlan& plan, float* consts, hipStream_t st,
                              KEvents ev) {
  const int ndhn = ndh * N;
  launch_k(scan_consts_kernel, dim3((unsigned)((ndhn + 255) / 256)), dim3(256), st, ev, log_re,
           log_im, reinterpret_cast<const float2*>(W), ndhn, plan.seg, consts);
  return hipGetLastError();
}

hipError_t launch_scan(const float* u, const float* consts, const float* D, int B, int H, int N,
                       int L, int ndir, const ScanPlan& plan, float* y, hipStream_t st,
                       float2* carry, KEvents ev, bool state) {
  switch (plan.seg) {
    case 4: scan_launch<4>(u, consts, D, carry, B, H, N, L, ndir, plan, y, st, ev, state); break;
    case 8: scan_launch<8>(u, consts, D, carry, B, H, N, L, ndir, plan, y, st, ev, state); break;
    case 16: scan_launch<16>(u, consts, D, carry, B, H, N, L, ndir, plan, y, st, ev, state); break;
    case 32: scan_launch<32>(u, consts, D, carry, B, H, N, L, ndir, plan, y, st, ev, state); break;
    case 64: scan_launch<64>(u, consts, D, carry, B, H, N, L, ndir, plan, y, st, ev, state); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_step(const float* u, const float* log_re, const float* log_im, const float* W,
                       const float* D, int B, int H, int N, float* x, float* y, hipStream_t st) {
  const long waves = (long)B * H;
  const long blocks = (waves + 3) / 4;
  hipLaunchKernelGGL(step_kernel, dim3((unsigned)blocks), dim3(256), 0, st, u, log_re, log_im,
                     reinterpret_cast<const float2*>(W), D, B, H, N, reinterpret_cast<float2*>(x),
                     y);
  return hipGetLastError();
}

}  // namespace dssm
