// S5-style multi-input multi-output diagonal SSM forward
// ("Simplified State Space Layers for Sequence Modeling", section 3: one
// diagonal state of size P shared by all H inputs, B~ in C^{PxH},
// C~ in C^{HxP}, diagonal real D; section 2.2: the linear recurrence as a
// scan):
//
//   v_k = Bbar u_k,   x_k = lambda * x_{k-1} + v_k  (x_{-1} = 0),
//   y_k = Re(C x_k) + D * u_k.
//
// How (MI355X design): the two projections are dense contractions over H and
// over 2P real rows, done on the matrix cores in float32
// (v_mfma_f32_16x16x4f32); the recurrence is a segmented complex scan per
// (b, p) channel between them.  Intermediates v and x live in the workspace as
// [B][P][2][L] float32 (real row, imaginary row), which is exactly the
// [2P x L] right-hand operand of the output projection.
//   * pack kernel: Bbar and C rearranged into MFMA A-fragment order
//     (rows 2p / 2p+1 = Re / Im of Bbar[p,:]; columns 2p / 2p+1 = Re C[:,p] /
//     -Im C[:,p]), zero padded.
//   * gemm kernel: one workgroup = 4 waves x 64 rows x 64 time steps, the
//     whole reduction in registers; each lane loads one float4 of A and one
//     of B per 4-deep k step and issues 16 MFMAs.  The output projection adds
//     D u in its epilogue.
//   * scan kernel: one channel per workgroup, 16 steps per lane, carries by a
//     Hillis-Steele scan with multipliers lambda^(16 2^j) from float64, tiles
//     of 4096 steps chained by the carried state.
#include <algorithm>

#include "dssm_internal.h"

namespace dssm {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

// A-fragment layout for M x K (row block rb of 64 rows, k step ks of 4):
//   apk[((rb * KS + ks) * 64 + lane) * 4 + r] = A[rb*64 + r*16 + lane%16][ks*4 + lane/16]
// kind 0: A = [Re Bbar; Im Bbar] interleaved by p   (M = 2P, K = H)
// kind 1: A = [Re C, -Im C] interleaved by p        (M = H,  K = 2P)
__global__ __launch_bounds__(256) void s5_pack_kernel(const float2* __restrict__ Bbar,
                                                      const float2* __restrict__ C, int H, int P,
                                                      float* __restrict__ apk_in,
                                                      float* __restrict__ apk_out) {
  const int kind = blockIdx.y;
  const int M = kind == 0 ? 2 * P : H;
  const int K = kind == 0 ? H : 2 * P;
  const int MB = (M + 63) / 64, KS = (K + 3) / 4;
  const long total = (long)MB * KS * 64 * 4;
  float* out = kind == 0 ? apk_in : apk_out;
  for (long e = (long)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (long)gridDim.x * blockDim.x) {
    const int r = (int)(e & 3);
    const int lane = (int)((e >> 2) & 63);
    const long t = e >> 8;
    const int ks = (int)(t % KS);
    const int rb = (int)(t / KS);
    const int i = rb * 64 + r * 16 + (lane & 15);
    const int k = ks * 4 + (lane >> 4);
    float v = 0.f;
    if (i < M && k < K) {
      if (kind == 0) {
        const float2 b = Bbar[(size_t)(i >> 1) * H + k];
        v = (i & 1) ? b.y : b.x;
      } else {
        const float2 c = C[(size_t)i * P + (k >> 1)];
        v = (k & 1) ? -c.y : c.x;
      }
    }
    out[e] = v;
  }
}

// out[b][i][j] = sum_k A[i][k] Bm[b][k][j]  (+ D[i] u[b][i][j] when kAddDu)
// A given as fragments (see above); Bm [B][K][L] row-major; out [B][M][L].
template <bool kAddDu>
__global__ __launch_bounds__(256) void s5_gemm_kernel(const float* __restrict__ apk,
                                                      const float* __restrict__ Bm, int M, int K,
                                                      int L, const float* __restrict__ D,
                                                      const float* __restrict__ u,
                                                      float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int MB = (M + 63) / 64, KS = (K + 3) / 4;
  const int rb = blockIdx.y * 4 + w;
  if (rb >= MB) return;  // no barriers in this kernel
  const int b = blockIdx.z;
  const int j0 = blockIdx.x * 64;
  const int jl = j0 + 4 * (lane & 15);  // this lane's 4 columns
  const bool vec = ((L & 3) == 0) && (jl + 3 < L);
  const float* Bb = Bm + (size_t)b * K * L;
  const v4f* ap = reinterpret_cast<const v4f*>(apk) + (size_t)rb * KS * 64 + lane;

  v4f acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = v4f{0.f, 0.f, 0.f, 0.f};

  // operands of k step ks: one float4 of A fragments, one float4 of B
  auto load_b = [&](int ks) {
    const int k = ks * 4 + (lane >> 4);
    v4f bv = v4f{0.f, 0.f, 0.f, 0.f};
    if (ks < KS && k < K) {
      const float* row = Bb + (size_t)k * L;
      if (vec) {
        bv = *reinterpret_cast<const v4f*>(row + jl);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) bv[c] = (jl + c < L) ? row[jl + c] : 0.f;
      }
    }
    return bv;
  };
  // one step of prefetch: the loads of step ks+1 are in flight while the 16
  // MFMAs of step ks run
  v4f a = ap[0];
  v4f bv = load_b(0);
  for (int ks = 0; ks < KS; ++ks) {
    const v4f a_n = (ks + 1 < KS) ? ap[(size_t)(ks + 1) * 64] : a;
    const v4f b_n = load_b(ks + 1);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], bv[c], acc[r][c], 0, 0, 0);
    a = a_n;
    bv = b_n;
  }

  // acc[r][c][v] holds row rb*64 + r*16 + 4*(lane/16) + v, column jl + c.
  float* ob = out + (size_t)b * M * L;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = rb * 64 + r * 16 + 4 * (lane >> 4) + v;
      if (i >= M) continue;
      v4f o = v4f{acc[r][0][v], acc[r][1][v], acc[r][2][v], acc[r][3][v]};
      if (kAddDu) {
        const float d = D[i];
        const float* ur = u + ((size_t)b * M + i) * L;
        if (vec) {
          const v4f uu = *reinterpret_cast<const v4f*>(ur + jl);
          o += d * uu;
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (jl + c < L) o[c] += d * ur[jl + c];
        }
      }
      float* orow = ob + (size_t)i * L;
      if (vec) {
        *reinterpret_cast<v4f*>(orow + jl) = o;
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (jl + c < L) orow[jl + c] = o[c];
      }
    }
  }
}

constexpr int kSeg = 16;       // steps per lane
constexpr int kLanes = 256;    // lanes per channel (one workgroup)
constexpr int kTile = kSeg * kLanes;
constexpr int kLevels = 8;     // log2(kLanes)

__device__ __forceinline__ float2 cm(float2 a, float2 b) {
  return make_float2(fmaf(a.x, b.x, -a.y * b.y), fmaf(a.x, b.y, a.y * b.x));
}

// x[b,p,:] = scan of v[b,p,:] with multiplier lambda[p]; planar re/im rows.
// Each tile of 4096 steps is staged through LDS (coalesced float4 global
// accesses; lane l then owns steps 16 l .. 16 l + 15, padded one slot per 16
// so the per-lane reads are conflict-free).
constexpr int kPadT = kTile + kTile / 16;
__device__ __forceinline__ int tpad(int e) { return e + (e >> 4); }

__global__ __launch_bounds__(kLanes) void s5_scan_kernel(const float2* __restrict__ lam,
                                                         const float* __restrict__ v, int P, int L,
                                                         float* __restrict__ x) {
  __shared__ float sre[kPadT], sim[kPadT];
  __shared__ float2 mu[kLevels + 1];  // lambda^(kSeg 2^j) for j <= 8
  __shared__ float2 blk[4];           // per-wave inclusive totals
  __shared__ float2 carry;
  const int p = blockIdx.x % P;
  const int b = blockIdx.x / P;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const float2 lm = lam[p];
  if (t <= kLevels) {
    // lambda^k = exp(k log|lambda|) cis(k arg lambda), k = kSeg 2^t, in float64
    const double lr = (double)lm.x, li = (double)lm.y;
    const double k = (double)kSeg * (double)(1 << t);
    const double lmag = 0.5 * log(lr * lr + li * li);
    const double ang = atan2(li, lr);
    double sn, cs;
    sincos(k * ang, &sn, &cs);
    const double m = exp(k * lmag);
    mu[t] = make_float2((float)(m * cs), (float)(m * sn));
  }
  if (t == 0) carry = make_float2(0.f, 0.f);

  const float* vre = v + ((size_t)b * P + p) * 2 * L;
  const float* vim = vre + L;
  float* xre = x + ((size_t)b * P + p) * 2 * L;
  float* xim = xre + L;
  const bool vec = (L & 3) == 0;

  for (int base = 0; base < L; base += kTile) {
    const int n = min(kTile, L - base);
    // stage the tile (zero beyond L)
    if (vec) {
#pragma unroll
      for (int k = 0; k < kTile / (4 * kLanes); ++k) {
        const int e = 4 * (t + kLanes * k);
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f), c = a;
        if (e < n) {
          a = *reinterpret_cast<const float4*>(vre + base + e);
          c = *reinterpret_cast<const float4*>(vim + base + e);
        }
        const int q = tpad(e);  // e is a multiple of 4: the 4 slots stay contiguous
        sre[q] = a.x; sre[q + 1] = a.y; sre[q + 2] = a.z; sre[q + 3] = a.w;
        sim[q] = c.x; sim[q + 1] = c.y; sim[q + 2] = c.z; sim[q + 3] = c.w;
      }
    } else {
      for (int e = t; e < kTile; e += kLanes) {
        sre[tpad(e)] = e < n ? vre[base + e] : 0.f;
        sim[tpad(e)] = e < n ? vim[base + e] : 0.f;
      }
    }
    __syncthreads();
    float2 vv[kSeg];
#pragma unroll
    for (int i = 0; i < kSeg; ++i) {
      const int q = 17 * t + i;  // tpad(16 t + i)
      vv[i] = make_float2(sre[q], sim[q]);
    }
    // local end state
    float2 s = make_float2(0.f, 0.f);
#pragma unroll
    for (int i = 0; i < kSeg; ++i) {
      const float2 m = cm(lm, s);
      s = make_float2(m.x + vv[i].x, m.y + vv[i].y);
    }
    const float2 cin = carry;
    if (t == 0) {  // the tile's first segment starts from the carried state
      const float2 m = cm(mu[0], cin);
      s.x += m.x;
      s.y += m.y;
    }
    // inclusive scan inside the wave
#pragma unroll
    for (int j = 0; j < 6; ++j) {
      const int o = 1 << j;
      float2 q;
      q.x = __shfl(s.x, max(lane - o, 0));
      q.y = __shfl(s.y, max(lane - o, 0));
      if (lane >= o) {
        const float2 m = cm(mu[j], q);
        s.x += m.x;
        s.y += m.y;
      }
    }
    // chain the four waves: carry into wave w = sum_{k<w} nu^(w-1-k) total_k
    if (lane == 63) blk[w] = s;
    __syncthreads();
    float2 cw = make_float2(0.f, 0.f);
    for (int k = 0; k < w; ++k) {
      const float2 m = cm(mu[6], cw);
      cw = make_float2(m.x + blk[k].x, m.y + blk[k].y);
    }
    {  // s += lambda^(kSeg (lane+1)) cw
      float2 pw = make_float2(1.f, 0.f);
      const int e = lane + 1;
#pragma unroll
      for (int j = 0; j < 7; ++j)
        if ((e >> j) & 1) pw = cm(pw, mu[j]);
      const float2 m = cm(pw, cw);
      s.x += m.x;
      s.y += m.y;
    }
    float2 xin;
    {
      float2 q;
      q.x = __shfl(s.x, max(lane - 1, 0));
      q.y = __shfl(s.y, max(lane - 1, 0));
      xin = (t == 0) ? cin : (lane == 0 ? cw : q);
    }
    __syncthreads();  // everyone has read `carry`, `blk` and its inputs
    if (t == kLanes - 1) carry = s;
    // outputs, back into the staging buffers
    float2 st = xin;
#pragma unroll
    for (int i = 0; i < kSeg; ++i) {
      const float2 m = cm(lm, st);
      st = make_float2(m.x + vv[i].x, m.y + vv[i].y);
      const int q = 17 * t + i;
      sre[q] = st.x;
      sim[q] = st.y;
    }
    __syncthreads();
    if (vec) {
#pragma unroll
      for (int k = 0; k < kTile / (4 * kLanes); ++k) {
        const int e = 4 * (t + kLanes * k);
        if (e < n) {
          const int q = tpad(e);
          *reinterpret_cast<float4*>(xre + base + e) = make_float4(sre[q], sre[q + 1], sre[q + 2], sre[q + 3]);
          *reinterpret_cast<float4*>(xim + base + e) = make_float4(sim[q], sim[q + 1], sim[q + 2], sim[q + 3]);
        }
      }
    } else {
      for (int e = t; e < n; e += kLanes) {
        xre[base + e] = sre[tpad(e)];
        xim[base + e] = sim[tpad(e)];
      }
    }
    __syncthreads();  // staging buffers and carry are reused by the next tile
  }
}

}  // namespace

S5Layout s5_layout(int B, int H, int P, int L) {
  S5Layout l;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  const size_t in_frag = (size_t)((2 * P + 63) / 64) * 64 * ((H + 3) / 4) * 4;
  const size_t out_frag = (size_t)((H + 63) / 64) * 64 * ((2 * P + 3) / 4) * 4;
  l.apk_in = take(in_frag * sizeof(float));
  l.apk_out = take(out_frag * sizeof(float));
  l.v = take((size_t)B * P * 2 * L * sizeof(float));
  l.x = take((size_t)B * P * 2 * L * sizeof(float));
  l.total = off;
  return l;
}

hipError_t launch_s5_pack(const float* Bbar, const float* C, int H, int P, float* apk_in,
                          float* apk_out, hipStream_t st, KEvents ev) {
  launch_k(s5_pack_kernel, dim3(256, 2), dim3(256), st, ev, reinterpret_cast<const float2*>(Bbar),
           reinterpret_cast<const float2*>(C), H, P, apk_in, apk_out);
  return hipGetLastError();
}

hipError_t launch_s5_proj_in(const float* apk_in, const float* u, int B, int H, int P, int L,
                             float* v, hipStream_t st, KEvents ev) {
  const int M = 2 * P;
  const dim3 grid((unsigned)((L + 63) / 64), (unsigned)(((M + 63) / 64 + 3) / 4), (unsigned)B);
  launch_k(s5_gemm_kernel<false>, grid, dim3(256), st, ev, apk_in, u, M, H, L,
           static_cast<const float*>(nullptr), static_cast<const float*>(nullptr), v);
  return hipGetLastError();
}

hipError_t launch_s5_scan(const float* lambda, const float* v, int B, int P, int L, float* x,
                          hipStream_t st, KEvents ev) {
  launch_k(s5_scan_kernel, dim3((unsigned)(B * P)), dim3(kLanes), st, ev,
           reinterpret_cast<const float2*>(lambda), v, P, L, x);
  return hipGetLastError();
}

hipError_t launch_s5_proj_out(const float* apk_out, const float* x, const float* D,
                              const float* u, int B, int H, int P, int L, float* y,
                              hipStream_t st, KEvents ev) {
  const int M = H;
  const dim3 grid((unsigned)((L + 63) / 64), (unsigned)(((M + 63) / 64 + 3) / 4), (unsigned)B);
  launch_k(s5_gemm_kernel<true>, grid, dim3(256), st, ev, apk_out, x, M, 2 * P, L, D, u, y);
  return hipGetLastError();
}

}  // namespace dssm
