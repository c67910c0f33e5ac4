// Kernel generation for the diagonal linear RNN:
//   K[h, j] = sum_n W[h,n] lambda[h,n]^j,   lambda = exp(-re^2 + i im)
// ("Simplifying and Understanding State Space Models with Diagonal Linear
// RNNs", section 2: the parameterisation of Lambda and K = (<w, Lambda^k>)_k).
//
// One workgroup produces a 64 x 64 block of K for one channel: j = 64 q + r
// with q in a tile of 64 anchors and r < 64, via
//   K[64 q + r] = sum_n (W_n lambda_n^(64 q)) * lambda_n^r.
// Precision: both factors are formed in float64 -- lambda from exp/sincos of
// the exactly promoted parameters, lambda^(16 t) and (lambda^64)^e by binary
// powering, then chains of at most 15 float64 products -- and rounded once to
// float32; no float32 power chain exists.  The contraction over the modes is
// a real product of a (64 x 2N) by a (2N x 64) matrix, done on the matrix
// cores in float32 (v_mfma_f32_16x16x4f32):
//   Re K = sum_n Re A Re P - Im A Im P,   Im K = sum_n Re A Im P + Im A Re P.
#include "dssm_internal.h"

namespace dssm {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double2 zmul(double2 x, double2 y) {
  return make_double2(x.x * y.x - x.y * y.y, x.x * y.y + x.y * y.x);
}

// Row stride (floats) of the LDS operand tables: rows k' = 2n + part (part 0
// = real, 1 = imaginary) of 64 entries; 80 keeps the four rows an MFMA step
// reads in different LDS banks.
constexpr int kRow = 80;
constexpr int kModes = 64;  // modes staged per chunk

template <bool kComplex>
__global__ __launch_bounds__(256) void gen_kernel(const float* __restrict__ log_re,
                                                  const float* __restrict__ log_im,
                                                  const float2* __restrict__ W, int N, int L,
                                                  float* __restrict__ K) {
  __shared__ float sA[2 * kModes * kRow];  // [2n + part][q]: W lambda^(64 q)
  __shared__ float sP[2 * kModes * kRow];  // [2n + part][r]: lambda^r
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int dh = blockIdx.y;
  const int Q = (L + kAnchor - 1) / kAnchor;
  const int q0 = blockIdx.x * 64;

  v4f acc_re[4], acc_im[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    acc_re[c] = v4f{0.f, 0.f, 0.f, 0.f};
    acc_im[c] = v4f{0.f, 0.f, 0.f, 0.f};
  }

  for (int n0 = 0; n0 < N; n0 += kModes) {
    const int nn = min(kModes, N - n0);
    // ---- tables: 4 threads per mode, 16 entries of each table per thread
    {
      const int nl = t >> 2, tq = t & 3;
      double2 lam = make_double2(0.0, 0.0), wv = make_double2(0.0, 0.0);
      if (nl < nn) {
        const int dhn = dh * N + n0 + nl;
        const double re = (double)log_re[dhn];
        double s, c;
        sincos((double)log_im[dhn], &s, &c);
        const double m = exp(-re * re);
        lam = make_double2(m * c, m * s);
        const float2 wf = W[dhn];
        wv = make_double2((double)wf.x, (double)wf.y);
      }
      // lambda^16, lambda^32, lambda^48, lambda^64
      double2 l2 = zmul(lam, lam), l4 = zmul(l2, l2), l8 = zmul(l4, l4), l16 = zmul(l8, l8);
      const double2 l32 = zmul(l16, l16);
      const double2 mu = zmul(l32, l32);  // lambda^64
      double2 x = tq == 0 ? make_double2(1.0, 0.0)
                 : tq == 1 ? l16
                 : tq == 2 ? l32
                           : zmul(l32, l16);
      float* prow = sP + (2 * nl) * kRow + 16 * tq;
#pragma unroll
      for (int i = 0; i < 16; ++i) {  // lambda^r, r = 16 tq + i
        prow[i] = (float)x.x;
        prow[kRow + i] = (float)x.y;
        x = zmul(x, lam);
      }
      // W mu^e, e = q0 + 16 tq, by binary powering of mu, then a chain of 15
      int e = q0 + 16 * tq;
      double2 a = wv, base = mu;
      while (e) {
        if (e & 1) a = zmul(a, base);
        base = zmul(base, base);
        e >>= 1;
      }
      float* arow = sA + (2 * nl) * kRow + 16 * tq;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool in = (q0 + 16 * tq + i) < Q;
        arow[i] = in ? (float)a.x : 0.f;
        arow[kRow + i] = in ? (float)a.y : 0.f;
        a = zmul(a, mu);
      }
    }
    __syncthreads();
    // ---- contraction: wave w owns anchors q0 + 16 w .. +15, all 64 r
    {
      const int kq = lane >> 4;  // k' offset inside a step (0..3)
      const int part = kq & 1;
      const int qa = 16 * w + (lane & 15);
      const int steps = (2 * nn + 3) / 4;
      // operands of one k step: a (A column) and b[c] / bi[c] (B rows)
      auto load = [&](int ks, float& a, float* b, float* bi) {
        const int kk = 4 * ks + kq;  // row 2n + part
        const bool inrow = kk < 2 * nn;
        a = inrow ? sA[kk * kRow + qa] : 0.f;  // A = [Re A, -Im A] along k'
        if (part) a = -a;
        const float* pr = sP + kk * kRow + (lane & 15);
        const float* pr_sw = sP + (kk ^ 1) * kRow + (lane & 15);  // other part of the mode
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          b[c] = inrow ? pr[16 * c] : 0.f;  // [Re P; Im P]
          if (kComplex) {
            const float v = inrow ? pr_sw[16 * c] : 0.f;  // [Im P; -Re P]
            bi[c] = part ? -v : v;
          }
        }
      };
      float a, b[4], bi[4];
      load(0, a, b, bi);
      for (int ks = 0; ks < steps; ++ks) {
        float an, bn[4], bin[4];
        load(min(ks + 1, steps - 1), an, bn, bin);  // prefetch the next step
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc_re[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b[c], acc_re[c], 0, 0, 0);
          if (kComplex)
            acc_im[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bi[c], acc_im[c], 0, 0, 0);
        }
        a = an;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          b[c] = bn[c];
          bi[c] = bin[c];
        }
      }
    }
    __syncthreads();
  }

  // acc[c][v]: q = q0 + 16 w + 4 (lane / 16) + v, r = 16 c + lane % 16
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int q = q0 + 16 * w + 4 * (lane >> 4) + v;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const long j = (long)q * kAnchor + 16 * c + (lane & 15);
      if (q < Q && j < L) {
        if (kComplex)
          reinterpret_cast<float2*>(K)[(size_t)dh * L + j] = make_float2(acc_re[c][v], acc_im[c][v]);
        else
          K[(size_t)dh * L + j] = acc_re[c][v];
      }
    }
  }
}

}  // namespace

hipError_t launch_gen(const float* log_re, const float* log_im, const float* W, int ndh, int N,
                      int L, int complex_out, float* K, hipStream_t st, KEvents ev) {
  const int Q = (L + kAnchor - 1) / kAnchor;
  const dim3 grid((unsigned)((Q + 63) / 64), (unsigned)ndh);
  const float2* w2 = reinterpret_cast<const float2*>(W);
  if (complex_out)
    launch_k(gen_kernel<true>, grid, dim3(256), st, ev, log_re, log_im, w2, N, L, K);
  else
    launch_k(gen_kernel<false>, grid, dim3(256), st, ev, log_re, log_im, w2, N, L, K);
  return hipGetLastError();
}

}  // namespace dssm
