// Kernel generation for the diagonal linear RNN:
//   K[h, j] = sum_n W[h,n] lambda[h,n]^j,   lambda = exp(-re^2 + i im)
// ("Simplifying and Understanding State Space Models with Diagonal Linear
// RNNs", section 2: the parameterisation of Lambda and K = (<w, Lambda^k>)_k).
//
// With anchors mu = lambda^64 and j = 64 q + r (r < 64):
//   K[64 q + r] = sum_n lambda_n^r (W_n mu_n^q),
// a real contraction over the rows k' = 2n + part of
//   P[r][k'] = (Re lambda^r, Im lambda^r),   A[q][k'] = (Re W mu^q, -Im W mu^q)
// (Re K = sum_k' P A; Im K uses (Im lambda^r, -Re lambda^r) in place of P).
// Both tables are formed in float64 -- lambda from exp/sincos of the exactly
// promoted parameters, starting powers by binary powering, then chains of 16
// float64 products -- and rounded once to float32.  The contraction runs on
// the matrix cores (v_mfma_f32_16x16x32_f16) on split operands: fp16 hi + lo,
// three products, float32 accumulation.  P (|P| <= 1, no scale needed) is
// stored split, once for all four waves; A is split as it is read, after an
// exact power-of-two scale from its largest entry.
//
// One workgroup (4 waves) produces a 64 x 64 block of K for one channel:
// anchors q0 .. q0 + 63 (wave w: q0 + 16 w .. + 15) by r < 64, over the modes in
// chunks of 64 (thread (n = lane, w) forms table rows 16 w .. 16 w + 15 of mode
// n).  Modes beyond N have zero anchors, so the contraction runs unpredicated.
#include "dssm_internal.h"
#include "mfma_split.h"

namespace dssm {
namespace {

using namespace mx;

constexpr int kModes = 64;           // modes per table chunk
constexpr int kQW = 64;              // anchors per workgroup
// Row strides: the 16 rows of one 16-byte fragment read fall in distinct banks.
constexpr int kTS = 2 * kModes + 4;   // A rows (float)
constexpr int kTSh = 2 * kModes + 8;  // P rows (fp16)
static_assert(kAnchor == 64, "one anchor per 64 taps");

struct GenLds {
  _Float16 Ph[kAnchor][kTSh], Pl[kAnchor][kTSh];  // P[r][k'] split (|P| <= 1: no scale)
  float A[kQW][kTS];                              // A[q - q0][k']
  double2 lam[kModes], wv[kModes];
  float red[4];
};

// x^e, e >= 0, by binary powering.
__device__ __forceinline__ double2 zpow(double2 x, int e) {
  double2 a = make_double2(1.0, 0.0);
  for (; e; e >>= 1) {
    if (e & 1) a = zmul(a, x);
    x = zmul(x, x);
  }
  return a;
}

// Output kOut: 0 = Re K, 1 = K (re, im), 2 = Re K Im K (the DLR-prod cast of
// the DLR page, section 2.1).
template <int kOut>
__global__ __launch_bounds__(256, 2) void gen_kernel(const float* __restrict__ log_re,
                                                     const float* __restrict__ log_im,
                                                     const float2* __restrict__ W, int N, int L,
                                                     float* __restrict__ K) {
  __shared__ GenLds s;
  PhaseClock pc;  // phase stamps (instrumented builds only): slots below
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, g = lane >> 4;
  const int dh = blockIdx.y;
  const int Q = (L + kAnchor - 1) / kAnchor;
  const int q0 = blockIdx.x * kQW;
  constexpr bool kComplex = kOut != 0;  // the imaginary part is formed too

  f4 tot[4], toti[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) tot[rt] = toti[rt] = f4{0.f, 0.f, 0.f, 0.f};

  for (int n0 = 0; n0 < N; n0 += kModes) {
    const int nn = min(kModes, N - n0);
    if (n0) __syncthreads();  // the previous chunk's tables are read
    if (w == 0) {
      double2 lam = make_double2(0.0, 0.0), wv = lam;
      if (lane < nn) {
        const size_t i = (size_t)dh * N + n0 + lane;
        const double re = (double)log_re[i];
        double sn, cs;
        sincos((double)log_im[i], &sn, &cs);
        const double m = exp(-re * re);
        lam = make_double2(m * cs, m * sn);
        wv = make_double2((double)W[i].x, (double)W[i].y);
      }
      s.lam[lane] = lam;
      s.wv[lane] = wv;
    }
    __syncthreads();
    pc.mark(0);  // lambda and W (wave 0, float64), barrier
    float am = 0.f;  // largest |A| entry written by this thread
    {
      const int n = lane;
      const double2 lam = s.lam[n], wv = s.wv[n];
      double2 x = zpow(lam, 16 * w);  // lambda^r, r = 16 w + i
      const double2 mu = zpow(lam, kAnchor);
      const int qs = q0 + 16 * w;
      double2 a = zmul(wv, zpow(mu, qs));  // W mu^q, q = qs + i
#pragma unroll 4
      for (int i = 0; i < 16; ++i) {  // the two chains are independent: their latencies overlap
        half2v hi, lo;
        _Float16 h, l;
        split16(opaquef((float)x.x), h, l);
        hi[0] = h;
        lo[0] = l;
        split16(opaquef((float)x.y), h, l);
        hi[1] = h;
        lo[1] = l;
        *reinterpret_cast<half2v*>(&s.Ph[16 * w + i][2 * n]) = hi;
        *reinterpret_cast<half2v*>(&s.Pl[16 * w + i][2 * n]) = lo;
        const bool in = qs + i < Q;
        const float2 af = make_float2(in ? (float)a.x : 0.f, in ? -(float)a.y : 0.f);
        *reinterpret_cast<float2*>(&s.A[16 * w + i][2 * n]) = af;
        am = fmaxf(am, fmaxf(fabsf(af.x), fabsf(af.y)));
        x = zmul(x, lam);
        a = zmul(a, mu);
      }
    }
    pc.mark(1);  // tables: powers and anchors (float64 chains), split, LDS
    am = wave_max(am);
    if (lane == 0) s.red[w] = am;
    __syncthreads();
    pc.mark(2);  // largest anchor entry, barrier
    const int eA = scale_exp(fmaxf(fmaxf(s.red[0], s.red[1]), fmaxf(s.red[2], s.red[3])));

    // wave w: D[r][q] for r < 64 (4 row tiles) and q = q0 + 16 w + lane % 16
    f4 acc[4], acci[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[rt] = acci[rt] = f4{0.f, 0.f, 0.f, 0.f};
    const int steps = (2 * nn + 31) / 32;  // k-steps of 32 rows holding modes < nn
    for (int ks = 0; ks < steps; ++ks) {
      half8 bh, bl;
      {
        f4 lo4, hi4;
        lds_read8(&s.A[16 * w + (lane & 15)][32 * ks + 8 * g], lo4, hi4);
        const float v[8] = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        split8(v, bh, bl, eA);
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int r = 16 * rt + (lane & 15), k = 32 * ks + 8 * g;
        const half8 ah = *reinterpret_cast<const half8*>(&s.Ph[r][k]);
        const half8 al = *reinterpret_cast<const half8*>(&s.Pl[r][k]);
        acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh, acc[rt], 0, 0, 0);
        acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bl, acc[rt], 0, 0, 0);
        acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bh, acc[rt], 0, 0, 0);
        if (kComplex) {  // (Im lambda^r, -Re lambda^r) per mode: swap and negate (exact)
          half8 qh, ql;
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            qh[e] = ah[e + 1];
            qh[e + 1] = -ah[e];
            ql[e] = al[e + 1];
            ql[e + 1] = -al[e];
          }
          acci[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh, bh, acci[rt], 0, 0, 0);
          acci[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh, bl, acci[rt], 0, 0, 0);
          acci[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql, bh, acci[rt], 0, 0, 0);
        }
      }
    }
    pc.mark(3);  // contraction (matrix cores)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        tot[rt][v] += __builtin_amdgcn_ldexpf(acc[rt][v], -eA);
        if (kComplex) toti[rt][v] += __builtin_amdgcn_ldexpf(acci[rt][v], -eA);
      }
  }

  // tot[rt][v]: r = 16 rt + 4 g + v, q = q0 + 16 w + lane % 16; j = 64 q + r.
  // Positions at or beyond L fall outside the buffer range and are dropped.
  const int q = q0 + 16 * w + (lane & 15);
  if (kOut == 2) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) tot[rt][v] *= toti[rt][v];
  }
  if (kOut == 1) {
    const BufRes kb = buf_res(K + (size_t)dh * L * 2, 8u * (unsigned)L);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = kAnchor * q + 16 * rt + 4 * g + v;
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 o = {__float_as_uint(tot[rt][v]), __float_as_uint(toti[rt][v])};
        __builtin_amdgcn_raw_buffer_store_b64(o, kb, 8 * j, 0, 0);
      }
  } else {
    const BufRes kb = buf_res(K + (size_t)dh * L, 4u * (unsigned)L);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int j = kAnchor * q + 16 * rt + 4 * g;
      if ((L & 3) == 0) {  // the 16-byte group lies wholly inside or outside the row
        const u32x4 o = {__float_as_uint(tot[rt][0]), __float_as_uint(tot[rt][1]),
                         __float_as_uint(tot[rt][2]), __float_as_uint(tot[rt][3])};
        __builtin_amdgcn_raw_buffer_store_b128(o, kb, 4 * j, 0, 0);
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tot[rt][v]), kb, 4 * (j + v), 0, 0);
      }
    }
  }
  pc.mark(4);  // stores issued
  pc.write();
}

}  // namespace

hipError_t launch_gen(const float* log_re, const float* log_im, const float* W, int ndh, int N,
                      int L, int out, float* K, hipStream_t st, KEvents ev) {
  const int Q = (L + kAnchor - 1) / kAnchor;
  const dim3 grid((unsigned)((Q + kQW - 1) / kQW), (unsigned)ndh);
  const float2* w2 = reinterpret_cast<const float2*>(W);
  if (out == kGenComplex)
    launch_k(gen_kernel<1>, grid, dim3(256), st, ev, log_re, log_im, w2, N, L, K);
  else if (out == kGenReIm)
    launch_k(gen_kernel<2>, grid, dim3(256), st, ev, log_re, log_im, w2, N, L, K);
  else
    launch_k(gen_kernel<0>, grid, dim3(256), st, ev, log_re, log_im, w2, N, L, K);
  return hipGetLastError();
}

}  // namespace dssm

#ifdef DSSM_PHASE_STAMPS
// Buffer for the generator's phase stamps (instrumented builds only).
extern "C" int dssm_phase_stamps_gen(void* buf) {
  return (int)hipMemcpyToSymbol(HIP_SYMBOL(dssm::g_phase_buf), &buf, sizeof(buf));
}
#endif
