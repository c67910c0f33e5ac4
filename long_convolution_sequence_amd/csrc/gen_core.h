// Device-side pieces of the kernel generator, shared by the standalone
// generator (eig_gen.hip) and the fused generator + spectrum (fft.hip).
//
// What is computed ("Simplifying and Understanding State Space Models with
// Diagonal Linear RNNs", section 2: lambda = exp(-re^2 + i im) and
// K = (<w, Lambda^k>)_k), for one channel and a chunk of modes:
//   P[n, r] = lambda_n^r                  (r < 64)
//   A[n, q] = W_n lambda_n^(64 q)          (q in the workgroup's anchors)
//   K[64 q + r] = sum_n A[n, q] P[n, r]
// Both tables are formed in float64 -- lambda from exp/sincos of the exactly
// promoted parameters, starting powers by binary powering, then short chains
// of float64 products -- and rounded once to float32.  The contraction is a
// real product over rows k' = 2n + part done on the matrix cores in float32
// (v_mfma_f32_16x16x4f32):
//   Re K = sum_k' A'[k'] P[k'],  A' = [Re A; -Im A],  P = [Re P; Im P]
//   Im K = sum_k' A'[k'] Q[k'],  Q = [Im P; -Re P]  (complex output only).
// Rows of modes beyond N hold zero anchors, so the contraction needs no bounds
// checks.
#pragma once

#include <hip/hip_runtime.h>

namespace dssm {
namespace gen {

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double2 zmul(double2 x, double2 y) {
  return make_double2(x.x * y.x - x.y * y.y, x.x * y.y + x.y * y.x);
}

// x^e, e >= 0, by binary powering.
__device__ __forceinline__ double2 zpow(double2 x, int e) {
  double2 a = make_double2(1.0, 0.0);
  while (e) {
    if (e & 1) a = zmul(a, x);
    x = zmul(x, x);
    e >>= 1;
  }
  return a;
}

// Tables of one chunk of modes [n0, n0 + nn) of channel dh, written by TPM
// threads per mode (thread `sub` of mode `nl`): P entries r = PPT sub .. +PPT-1
// into sP (row stride RP), A entries q = q0 + APT sub .. +APT-1 into sA (row
// stride RA, column q - q0), zero for q >= Q.  With Q_OUT the Q table is also
// written (row stride RP).  Modes nl >= nn write zero anchors.
template <int TPM, int PPT, int APT, int RA, int RP, bool Q_OUT>
__device__ __forceinline__ void build_tables(const float* __restrict__ log_re,
                                             const float* __restrict__ log_im,
                                             const float2* __restrict__ W, int dhn0, int nn,
                                             int nl, int sub, int q0, int Q, float* sA, float* sP,
                                             float* sQ) {
  static_assert(PPT * TPM == 64, "lambda^r table covers r < 64");
  double2 lam = make_double2(0.0, 0.0), wv = make_double2(0.0, 0.0);
  if (nl < nn) {
    const double re = (double)log_re[dhn0 + nl];
    double s, c;
    sincos((double)log_im[dhn0 + nl], &s, &c);
    const double m = exp(-re * re);
    lam = make_double2(m * c, m * s);
    const float2 wf = W[dhn0 + nl];
    wv = make_double2((double)wf.x, (double)wf.y);
  }
  // lambda^r, r = PPT sub + i
  {
    double2 x = zpow(lam, PPT * sub);
    float* prow = sP + (2 * nl) * RP + PPT * sub;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      prow[i] = (float)x.x;
      prow[RP + i] = (float)x.y;
      if (Q_OUT) {
        float* qrow = sQ + (2 * nl) * RP + PPT * sub;
        qrow[i] = (float)x.y;
        qrow[RP + i] = -(float)x.x;
      }
      x = zmul(x, lam);
    }
  }
  // W mu^q, mu = lambda^64, q = q0 + APT sub + i
  {
    const double2 mu = zpow(lam, 64);
    const int qs = q0 + APT * sub;
    double2 a = zmul(wv, zpow(mu, qs));
    float* arow = sA + (2 * nl) * RA + APT * sub;
#pragma unroll
    for (int i = 0; i < APT; ++i) {
      const bool in = qs + i < Q;
      arow[i] = in ? (float)a.x : 0.f;
      arow[RA + i] = in ? -(float)a.y : 0.f;
      a = zmul(a, mu);
    }
  }
}

// Contraction of one chunk for one wave: anchors [qw, qw + 16) (columns of
// sA) by the NC blocks of 16 taps r0 .. r0 + 16 NC - 1, over rows
// 0 .. 4 steps - 1.  acc[c][v] accumulates
// K[64 (qw + 4 (lane / 16) + v) + r0 + 16 c + lane % 16].
template <int RA, int RP, bool Q_OUT, int NC = 4>
__device__ __forceinline__ void contract(const float* sA, const float* sP, const float* sQ, int qw,
                                         int r0, int steps, int lane, v4f* acc_re, v4f* acc_im) {
  const float* pa = sA + (lane >> 4) * RA + qw + (lane & 15);
  const float* pp = sP + (lane >> 4) * RP + r0 + (lane & 15);
  const float* pq = sQ + (Q_OUT ? (lane >> 4) * RP + r0 + (lane & 15) : 0);
  // Two operand sets alternate: the loads of one step are in flight while
  // the previous step multiplies (no register copies between steps).
  float a0, a1, b0[NC], b1[NC], q0v[NC], q1v[NC];
  auto load = [&](int ks, float& a, float* b, float* q) {
    const int ka = 4 * min(ks, steps - 1) * RA;
    const int kp = 4 * min(ks, steps - 1) * RP;
    a = pa[ka];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      b[c] = pp[kp + 16 * c];
      q[c] = Q_OUT ? pq[kp + 16 * c] : 0.f;
    }
  };
  auto mul = [&](float a, const float* b, const float* q) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      acc_re[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b[c], acc_re[c], 0, 0, 0);
      if (Q_OUT) acc_im[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, q[c], acc_im[c], 0, 0, 0);
    }
  };
  load(0, a0, b0, q0v);
  for (int ks = 0; ks < steps; ks += 2) {
    load(ks + 1, a1, b1, q1v);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the products
    mul(a0, b0, q0v);
    if (ks + 1 < steps) {
      load(ks + 2, a0, b0, q0v);
      __builtin_amdgcn_sched_barrier(0);
      mul(a1, b1, q1v);
    }
  }
}

}  // namespace gen
}  // namespace dssm
