// Gradients of the DLR layer map with respect to its parameters, from the
// kernel cotangents.
//
// What is computed ("Simplifying and Understanding State Space Models with
// Diagonal Linear RNNs", section 2: K_j = sum_n W_n lambda_n^j and
// lambda = exp(-log_re^2 + i log_im); the page gives dK_j / dlambda =
// j W lambda^(j-1) in its vanishing-gradient paragraph): for the scalar
// f = sum(dy y) and one direction d of channel h, with the kernel cotangent
// G[j] = d f / d Re K_j (the lagged correlation of dy and u summed over the
// batch, computed by the convolution kernels),
//   V0_n = sum_j G[j] lambda_n^j,   V1_n = sum_j j G[j] lambda_n^j,
//   dW_n = conj(V0_n)                     (d f / d Re W + i d f / d Im W),
//   Z_n  = W_n V1_n,  d f / d log_re = -2 log_re Re Z_n,  d f / d log_im = -Im Z_n,
//   d f / d D = G[0]                      (sum over b and k of dy u).
//
// How: j = 64 q + r.  A workgroup takes one (direction, channel) and every
// kSplit-th tile of 64 anchors q; it stages G for a tile in LDS (summing the
// batch rows as it loads them) and the powers lambda^r (r < 64, float64 chains
// rounded once) for a chunk of 64 modes; thread (mode n, part p) sums
// s0 = sum_r G[q][r] lambda^r and s1 = sum_r r G[q][r] lambda^r over its anchors
// q = p, p + 4, ... in float32, and accumulates V0 += mu^q s0 and
// V1 += mu^q (64 q s0 + s1) in float64, with mu^q = lambda^(64 q) by float64
// products.  The parts are combined in LDS and the kSplit partial sums of a
// (direction, channel) by a second kernel, which also forms the gradients.
#include <algorithm>

#include "dssm_internal.h"

namespace dssm {
namespace {

constexpr int kGM = 64;     // modes per chunk
constexpr int kGTile = 64;  // anchors per LDS tile

__device__ __forceinline__ double2 zmul(double2 a, double2 b) {
  return make_double2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}

__device__ __forceinline__ double2 zpow(double2 x, long e) {
  double2 a = make_double2(1.0, 0.0);
  for (; e; e >>= 1) {
    if (e & 1) a = zmul(a, x);
    x = zmul(x, x);
  }
  return a;
}

// Partial sums V0, V1 of (direction d, channel h, split s) for all modes:
// parts[(((d * H + h) * S + s) * N + n) * 2 + {0, 1}].
__global__ __launch_bounds__(256) void grad_vander_kernel(
    const float* __restrict__ corr, int B, int H, int L, const float* __restrict__ log_re,
    const float* __restrict__ log_im, int N, int d, int S, double2* __restrict__ parts) {
  __shared__ float G[kGTile][kAnchor];
  __shared__ float2 P[kAnchor][kGM];
  __shared__ double2 red[4][kGM][2];
  const int t = threadIdx.x, n = t & 63, part = t >> 6;
  const int h = blockIdx.x / S, s = blockIdx.x % S;
  const int Q = (L + kAnchor - 1) / kAnchor;
  const int ntile = (Q + kGTile - 1) / kGTile;

  for (int n0 = 0; n0 < N; n0 += kGM) {
    const int nn = min(kGM, N - n0);
    // lambda of mode n (zero beyond N), its powers r = 16 part .. + 15 into P
    double2 lam = make_double2(0.0, 0.0);
    if (n < nn) {
      const size_t i = ((size_t)d * H + h) * N + n0 + n;
      const double re = (double)log_re[i];
      double sn, cs;
      sincos((double)log_im[i], &sn, &cs);
      const double m = exp(-re * re);
      lam = make_double2(m * cs, m * sn);
    }
    __syncthreads();  // the previous chunk's P and G are read
    {
      double2 x = zpow(lam, 16 * part);
      for (int r = 16 * part; r < 16 * part + 16; ++r) {
        P[r][n] = make_float2((float)x.x, (float)x.y);
        x = zmul(x, lam);
      }
    }
    const double2 mu = zpow(lam, kAnchor);
    const double2 mu4 = zpow(mu, 4);
    const double2 muT = zpow(mu, (long)kGTile * S);  // from one of this workgroup's tiles to the next
    double2 mq0 = zpow(mu, (long)kGTile * s + part);  // mu^q of this thread's first anchor
    double2 v0 = make_double2(0.0, 0.0), v1 = v0;
    for (int tile = s; tile < ntile; tile += S) {
      __syncthreads();  // P written (first tile) / the previous tile's G read
      // stage G[q][r] = sum_b corr[b][h][64 q + r] for the tile's anchors
      for (int e = t; e < kGTile * kAnchor; e += 256) {
        const long j = (long)tile * kGTile * kAnchor + e;
        float g = 0.f;
        if (j < L)
          for (int b = 0; b < B; ++b) g += corr[((size_t)b * H + h) * L + j];
        G[e / kAnchor][e % kAnchor] = g;
      }
      __syncthreads();
      double2 mq = mq0;
      for (int qi = part; qi < kGTile; qi += 4) {
        float2 s0 = make_float2(0.f, 0.f), s1 = s0;
#pragma unroll 8
        for (int r = 0; r < kAnchor; ++r) {
          const float g = G[qi][r];
          const float2 p = P[r][n];
          const float gr = g * (float)r;
          s0.x = fmaf(g, p.x, s0.x);
          s0.y = fmaf(g, p.y, s0.y);
          s1.x = fmaf(gr, p.x, s1.x);
          s1.y = fmaf(gr, p.y, s1.y);
        }
        const double q64 = 64.0 * (double)((long)tile * kGTile + qi);
        const double2 a0 = make_double2((double)s0.x, (double)s0.y);
        const double2 a1 = make_double2(q64 * a0.x + (double)s1.x, q64 * a0.y + (double)s1.y);
        const double2 t0 = zmul(mq, a0), t1 = zmul(mq, a1);
        v0.x += t0.x;
        v0.y += t0.y;
        v1.x += t1.x;
        v1.y += t1.y;
        mq = zmul(mq, mu4);
      }
      mq0 = zmul(mq0, muT);
    }
    red[part][n][0] = v0;
    red[part][n][1] = v1;
    __syncthreads();
    if (part == 0 && n < nn) {
      double2 a = red[0][n][0], c = red[0][n][1];
      for (int p2 = 1; p2 < 4; ++p2) {
        a.x += red[p2][n][0].x;
        a.y += red[p2][n][0].y;
        c.x += red[p2][n][1].x;
        c.y += red[p2][n][1].y;
      }
      double2* o = parts + ((((size_t)d * H + h) * S + s) * N + n0 + n) * 2;
      o[0] = a;
      o[1] = c;
    }
  }
}

// dW, dlog_re, dlog_im per (direction, channel, mode) from the partial sums;
// dD per (direction, channel) from lag 0 of that direction's correlation.
__global__ __launch_bounds__(256) void grad_combine_kernel(
    const double2* __restrict__ parts, int S, int ndir, int H, int N,
    const float* __restrict__ log_re, const float2* __restrict__ W,
    const float* __restrict__ corr, int B, int L, float* __restrict__ dlog_re,
    float* __restrict__ dlog_im, float2* __restrict__ dW, float* __restrict__ dD) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long total = (long)ndir * H * N;
  if (i >= total) return;
  const long dh = i / N;
  const int n = (int)(i % N);
  double2 v0 = make_double2(0.0, 0.0), v1 = v0;
  for (int s = 0; s < S; ++s) {
    const double2* o = parts + ((dh * S + s) * N + n) * 2;
    v0.x += o[0].x;
    v0.y += o[0].y;
    v1.x += o[1].x;
    v1.y += o[1].y;
  }
  const double2 w = make_double2((double)W[i].x, (double)W[i].y);
  const double2 z = zmul(w, v1);
  dW[i] = make_float2((float)v0.x, (float)-v0.y);
  dlog_re[i] = (float)(-2.0 * (double)log_re[i] * z.x);
  dlog_im[i] = (float)(-z.y);
  if (n == 0) {
    const int d = (int)(dh / H), h = (int)(dh % H);
    const float* c = corr + (size_t)d * B * H * L;
    double g = 0.0;
    for (int b = 0; b < B; ++b) g += (double)c[((size_t)b * H + h) * L];
    dD[dh] = (float)g;
  }
}

__global__ void zero_kernel(float* __restrict__ p, long n) {
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

}  // namespace

hipError_t launch_zero_grads(float* dlog_re, float* dlog_im, float* dW, float* dD, int ndh, int N,
                             hipStream_t st) {
  const long nn = (long)ndh * N;
  const unsigned blocks = (unsigned)std::min<long>((2 * nn + 255) / 256, 4096);
  launch_k(zero_kernel, dim3(blocks), dim3(256), st, KEvents{}, dlog_re, nn);
  launch_k(zero_kernel, dim3(blocks), dim3(256), st, KEvents{}, dlog_im, nn);
  launch_k(zero_kernel, dim3(blocks), dim3(256), st, KEvents{}, dW, 2 * nn);
  launch_k(zero_kernel, dim3(blocks), dim3(256), st, KEvents{}, dD, (long)ndh);
  return hipGetLastError();
}

int grad_splits(int L) {
  const int Q = (L + kAnchor - 1) / kAnchor;
  const int ntile = (Q + kGTile - 1) / kGTile;
  return ntile < 4 ? ntile : 4;
}

hipError_t launch_grad_params(const float* corr, int B, int H, int L, const float* log_re,
                              const float* log_im, const float* W, int N, int ndir, void* parts,
                              float* dlog_re, float* dlog_im, float* dW, float* dD,
                              hipStream_t st) {
  const int S = grad_splits(L);
  double2* pp = static_cast<double2*>(parts);
  for (int d = 0; d < ndir; ++d)
    launch_k(grad_vander_kernel, dim3((unsigned)(H * S)), dim3(256), st, KEvents{},
             corr + (size_t)d * B * H * L, B, H, L, log_re, log_im, N, d, S, pp);
  const long total = (long)ndir * H * N;
  launch_k(grad_combine_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), st, KEvents{},
           static_cast<const double2*>(pp), S, ndir, H, N, log_re,
           reinterpret_cast<const float2*>(W), corr, B, L, dlog_re, dlog_im,
           reinterpret_cast<float2*>(dW), dD);
  return hipGetLastError();
}

}  // namespace dssm
