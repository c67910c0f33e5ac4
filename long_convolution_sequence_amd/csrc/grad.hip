// Gradients of the DLR layer map with respect to its parameters, from the
// kernel cotangents.
//
// What is computed ("Simplifying and Understanding State Space Models with
// Diagonal Linear RNNs", section 2: K_j = sum_n W_n lambda_n^j and
// lambda = exp(-log_re^2 + i log_im); the page gives dK_j / dlambda =
// j W lambda^(j-1) in its vanishing-gradient paragraph): for the scalar
// f = sum(dy y) and one direction d of channel h, with the kernel cotangent
// G[j] = d f / d Re K_j (the lagged correlation of dy and u summed over the
// batch; the correlation kernel leaves its halves in part[h][2][M]:
// G_f[j] = part[h][0][j] + part[h][1][j], and G_b[j] = part[h][0][M - j] -
// part[h][1][M - j] for j >= 1, G_b[0] = G_f[0]),
//   V0_n = sum_j G[j] lambda_n^j,   V1_n = sum_j j G[j] lambda_n^j,
//   dW_n = conj(V0_n)                     (d f / d Re W + i d f / d Im W),
//   Z_n  = W_n V1_n,  d f / d log_re = -2 log_re Re Z_n,  d f / d log_im = -Im Z_n,
//   d f / d D = G[0]                      (sum over b and k of dy u).
//
// How: j = 64 q + r, so V0_n = sum_q mu_n^q S0[q][n] and
// V1_n = sum_q mu_n^q (64 q S0[q][n] + S1[q][n]) with mu = lambda^64 and
//   S0[q][n] = sum_r G[q][r] lambda_n^r,   S1[q][n] = sum_r r G[q][r] lambda_n^r:
// two real products (Q x 64) x (64 x 2N) with the same right operand, run on
// the matrix cores in float32 (v_mfma_f32_16x16x4_f32: exact products,
// float32 sums, as a float32 dot product).  A workgroup takes one (direction,
// channel) and a contiguous range of 16-anchor tiles; it stages G for them in
// LDS (summing the batch rows as it loads them).  Wave w takes modes
// 16 w .. 16 w + 15 of a chunk of 64: its right operands (Re and Im of
// lambda^r, r < 64, float64 chains rounded once) stay in registers, and each
// lane adds its four anchors' mu^q S terms into float64 sums (mu^q by float64
// products).  The kSplit partial sums of a (direction, channel) are combined,
// and the gradients formed, by a second kernel.
#include <algorithm>

#include "dssm_internal.h"

namespace dssm {
namespace {

constexpr int kGM = 64;       // modes per chunk (4 waves x 16)
constexpr int kQT = 16;       // anchors per matrix tile
constexpr int kMaxTiles = 4;  // tiles per workgroup
constexpr int kGS = kAnchor + 4;  // LDS row stride of G (floats)

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t BufRes;

// Raw buffer over `bytes` bytes at `base`: loads at or past the end read zero.
__device__ __forceinline__ BufRes buf_res(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ float buf_load(BufRes r, int voff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}

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

__device__ __forceinline__ double shfl_xor_d(double v, int m) {
  const long long b = __double_as_longlong(v);
  const int lo = __shfl_xor((int)(b & 0xffffffffLL), m), hi = __shfl_xor((int)(b >> 32), m);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// Tiles of 16 anchors, and the workgroups (splits) sharing them, for length L.
__host__ __device__ __forceinline__ int anchor_tiles(int L) {
  const int Q = (L + kAnchor - 1) / kAnchor;
  return (Q + kQT - 1) / kQT;
}

// Partial sums V0, V1 of (direction d, channel h, split s) for all modes:
// parts[(((d * H + h) * S + s) * N + n) * 2 + {0, 1}].
// Matrix layouts of v_mfma_f32_16x16x4_f32 (lane l, i = l % 16, g = l / 16):
// A[i][k = g], B[k = g][j = i], D[i][j]: lane j + 16 (i / 4), element i % 4.
// Instruction ks (< 16) of a tile covers r = 16 g + ks on lane group g.
__global__ __launch_bounds__(256) void grad_vander_kernel(
    const float* __restrict__ part, int M, int NG, int H, int L, const float* __restrict__ log_re,
    const float* __restrict__ log_im, int N, int d, int S, double2* __restrict__ parts) {
  __shared__ float G[kMaxTiles * kQT][kGS];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int j = lane & 15, g = lane >> 4;
  const int h = blockIdx.x / S, s = blockIdx.x % S;
  const int ntile = anchor_tiles(L);
  const int per = (ntile + S - 1) / S;
  const int tile0 = s * per, tiles = max(0, min(per, ntile - tile0));

  // stage G[q][r] = G_d[64 q + r] for this split's anchors from the two
  // correlation halves of every batch group (raw buffers: offsets outside
  // them read zero; the backward direction reads them mirrored, M - j)
  {
    constexpr int kV = kMaxTiles * kQT * kAnchor / 256;  // floats per thread
    static_assert(kV * 256 == kMaxTiles * kQT * kAnchor, "staging split");
    const long j0 = (long)tile0 * kQT * kAnchor;
    const int nval = (int)std::min<long>((long)tiles * kQT * kAnchor, std::max<long>(0, L - j0));
    float acc[kV];
#pragma unroll
    for (int i = 0; i < kV; ++i) acc[i] = 0.f;
    for (int grp = 0; grp < NG; ++grp) {
      const BufRes pe = buf_res(part + ((size_t)grp * H + h) * 2 * M, 4u * (unsigned)M);
      const BufRes po = buf_res(part + (((size_t)grp * H + h) * 2 + 1) * M, 4u * (unsigned)M);
      float x[2][kV];
#pragma unroll
      for (int i = 0; i < kV; ++i) {
        const int e = t + 256 * i;
        const int jj = (int)j0 + e;
        // past the split's range: an offset beyond the halves (reads zero)
        const int src = e >= nval ? M : (d == 0 || jj == 0 ? jj : M - jj);
        x[0][i] = buf_load(pe, 4 * src);
        x[1][i] = buf_load(po, 4 * src);
      }
#pragma unroll
      for (int i = 0; i < kV; ++i) {
        const int jj = (int)j0 + t + 256 * i;
        acc[i] += (d == 0 || jj == 0) ? x[0][i] + x[1][i] : x[0][i] - x[1][i];
      }
    }
#pragma unroll
    for (int i = 0; i < kV; ++i) {
      const int e = t + 256 * i;
      G[e / kAnchor][e % kAnchor] = acc[i];
    }
  }
  __syncthreads();

  for (int n0 = 0; n0 < N; n0 += kGM) {
    const int n = n0 + 16 * w + j;  // this lane's mode (column)
    double2 lam = make_double2(0.0, 0.0);
    if (n < N) {
      const size_t i = ((size_t)d * H + h) * N + n;
      const double re = (double)log_re[i];
      double sn, cs;
      sincos((double)log_im[i], &sn, &cs);
      const double m = exp(-re * re);
      lam = make_double2(m * cs, m * sn);
    }
    // right operands: Re and Im of lambda^(16 g + ks), ks < 16
    float bre[16], bim[16];
    {
      double2 x = zpow(lam, 16 * g);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        bre[ks] = (float)x.x;
        bim[ks] = (float)x.y;
        x = zmul(x, lam);
      }
    }
    const double2 mu = zpow(lam, kAnchor);
    const double2 mu16 = zpow(mu, kQT);
    // mu^q for this lane's first anchor row of the first tile: q = 16 tile0 + 4 g
    double2 mq = zpow(mu, (long)kQT * tile0 + 4 * g);
    double2 v0 = make_double2(0.0, 0.0), v1 = v0;
    for (int tt = 0; tt < tiles; ++tt) {
      f4 s0r = {0.f, 0.f, 0.f, 0.f}, s0i = s0r, s1r = s0r, s1i = s0r;
      const float* grow = &G[tt * kQT + j][16 * g];
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const float a = grow[ks];
        const float ar = a * (float)(16 * g + ks);
        s0r = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bre[ks], s0r, 0, 0, 0);
        s0i = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bim[ks], s0i, 0, 0, 0);
        s1r = __builtin_amdgcn_mfma_f32_16x16x4f32(ar, bre[ks], s1r, 0, 0, 0);
        s1i = __builtin_amdgcn_mfma_f32_16x16x4f32(ar, bim[ks], s1i, 0, 0, 0);
      }
      // rows 4 g + v of the tile: anchor q = 16 (tile0 + tt) + 4 g + v
      double2 m = mq;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const double q64 = 64.0 * (double)(kQT * (tile0 + tt) + 4 * g + v);
        const double2 a0 = make_double2((double)s0r[v], (double)s0i[v]);
        const double2 a1 = make_double2(q64 * a0.x + (double)s1r[v], q64 * a0.y + (double)s1i[v]);
        const double2 t0 = zmul(m, a0), t1 = zmul(m, a1);
        v0.x += t0.x;
        v0.y += t0.y;
        v1.x += t1.x;
        v1.y += t1.y;
        m = zmul(m, mu);
      }
      mq = zmul(mq, mu16);
    }
    // sum the four lane groups (anchor rows) of each mode
#pragma unroll
    for (int msk = 16; msk <= 32; msk <<= 1) {
      v0.x += shfl_xor_d(v0.x, msk);
      v0.y += shfl_xor_d(v0.y, msk);
      v1.x += shfl_xor_d(v1.x, msk);
      v1.y += shfl_xor_d(v1.y, msk);
    }
    if (g == 0 && n < N) {
      double2* o = parts + ((((size_t)d * H + h) * S + s) * N + n) * 2;
      o[0] = v0;
      o[1] = v1;
    }
  }
}

// dW, dlog_re, dlog_im per (direction, channel, mode) from the partial sums;
// dD per (direction, channel) from lag 0 of that direction's correlation.
__global__ __launch_bounds__(256) void grad_combine_kernel(
    const double2* __restrict__ parts, int S, int ndir, int H, int N,
    const float* __restrict__ log_re, const float2* __restrict__ W,
    const float* __restrict__ part, int M, int NG, float* __restrict__ dlog_re,
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
  if (n == 0) {  // lag 0, the same for both directions
    const int h = (int)(dh % H);
    float g = 0.f;
    for (int grp = 0; grp < NG; ++grp)
      g += part[((size_t)grp * H + h) * 2 * M] + part[(((size_t)grp * H + h) * 2 + 1) * M];
    dD[dh] = g;
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
  const int ntile = anchor_tiles(L);
  return std::max(1, (ntile + kMaxTiles - 1) / kMaxTiles);
}

hipError_t launch_grad_params(const float* part, int M, int NG, int H, int L, const float* log_re,
                              const float* log_im, const float* W, int N, int ndir, void* parts,
                              float* dlog_re, float* dlog_im, float* dW, float* dD,
                              hipStream_t st) {
  const int S = grad_splits(L);
  double2* pp = static_cast<double2*>(parts);
  for (int d = 0; d < ndir; ++d)
    launch_k(grad_vander_kernel, dim3((unsigned)(H * S)), dim3(256), st, KEvents{}, part, M, NG, H,
             L, log_re, log_im, N, d, S, pp);
  const long total = (long)ndir * H * N;
  launch_k(grad_combine_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), st, KEvents{},
           static_cast<const double2*>(pp), S, ndir, H, N, log_re,
           reinterpret_cast<const float2*>(W), part, M, NG, dlog_re, dlog_im,
           reinterpret_cast<float2*>(dW), dD);
  return hipGetLastError();
}

}  // namespace dssm
