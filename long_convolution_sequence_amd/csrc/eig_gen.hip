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
// Table rows of modes beyond N (up to the chunk of 64) are written too: the
// anchors there are zero, so the contraction runs unpredicated.
#include "dssm_internal.h"
#include "gen_core.h"

namespace dssm {
namespace {

using gen::v4f;

// Row stride (floats) of the LDS operand tables: rows k' = 2n + part of 64
// entries; 80 keeps the four rows an MFMA step reads in different LDS banks.
constexpr int kRow = 80;
constexpr int kModes = 64;  // modes staged per chunk

// One workgroup (4 waves) produces a 64 x 64 block of K for one channel:
// anchors q0 .. q0 + 63 (wave w: 16 of them) by r < 64; 4 threads per mode
// build the tables.
template <bool kComplex>
__global__ __launch_bounds__(256) void gen_kernel(const float* __restrict__ log_re,
                                                  const float* __restrict__ log_im,
                                                  const float2* __restrict__ W, int N, int L,
                                                  float* __restrict__ K) {
  __shared__ float sA[2 * kModes * kRow];
  __shared__ float sP[2 * kModes * kRow];
  __shared__ float sQ[kComplex ? 2 * kModes * kRow : 1];
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
    gen::build_tables<4, 16, 16, kRow, kRow, kComplex>(log_re, log_im, W, dh * N + n0, nn, t >> 2,
                                                       t & 3, q0, Q, sA, sP, sQ);
    __syncthreads();
    gen::contract<kRow, kRow, kComplex>(sA, sP, sQ, 16 * w, 0, (2 * nn + 3) / 4, lane, acc_re,
                                        acc_im);
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
