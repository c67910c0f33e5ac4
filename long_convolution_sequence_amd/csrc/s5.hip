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
// over 2P real rows, done on the matrix cores (v_mfma_f32_16x16x32_f16) on
// split float32 operands: fp16 hi + lo, three products, float32 accumulation,
// each operand row or column first scaled by an exact power of two.  The
// recurrence is a segmented complex scan per (b, p) channel between them.
// Intermediates v and x live in the workspace as [B][P][2][L] float32 (real
// row, imaginary row), which is exactly the [2P x L] right-hand operand of the
// output projection.
//   * pack kernel: Bbar and C as split MFMA fragments of A^T (rows 2p / 2p+1 =
//     Re / Im of Bbar[p,:]; columns 2p / 2p+1 = Re C[:,p] / -Im C[:,p]), zero
//     padded, with one scale exponent per row.
//   * gemm kernel: one workgroup = 4 waves x 64 rows by 64 time steps; the
//     right-hand tile is staged through LDS transposed and split (per-column
//     scale), the products are formed transposed so each lane stores four
//     consecutive time steps.  The output projection adds D u in its epilogue.
//   * scan kernel: one channel per workgroup, 16 steps per lane, carries by a
//     Hillis-Steele scan with multipliers lambda^(16 2^j) from float64, tiles
//     of 4096 steps chained by the carried state.
#include <algorithm>
#include <climits>

#include "dssm_internal.h"
#include "mfma_split.h"

namespace dssm {
namespace {

using namespace mx;

typedef float v4f __attribute__((ext_vector_type(4)));

// Tile sizes of the contractions out[b][i][j] = sum_k A[i][k] Bm[b][k][j]:
// a workgroup (4 waves) owns 256 rows i (64 per wave) and 64 columns j (time
// steps) and runs over k in chunks of 256.  Each workgroup reads the whole
// split A^T table (from L2), so wider column tiles read it less often; 64 keeps
// the LDS tile at 68 KB (two workgroups per CU) and makes each wave's tile load
// instruction read one row (a wave-uniform row address).
constexpr int kRowsWG = 256;
constexpr int kColsWG = 64;
constexpr int kKC = 256;
constexpr int kNJ = kColsWG / 16;        // column tiles of 16
constexpr int kQL = kKC / 32;            // 8-deep k groups per thread
constexpr int kBTS = kKC + 8;  // LDS row stride (fp16) of the transposed B tile

// Element A[i][k] of a contraction (zero outside M x K):
// kind 0: A = [Re Bbar; Im Bbar] interleaved by p (M = 2P rows, K = H)
// kind 1: A = [Re C, -Im C] interleaved by p      (M = H rows,  K = 2P)
// kind 2: Bbar in the fused form's row order (M = 32 ceil(P / 16) rows,
//         K = H): row i is Re (bit 4 of i clear) or Im of Bbar[16 (i / 32) + i % 16, :]
// Branch-free: the load always reads an in-range element (clamped indices)
// and the result is selected afterwards, so a thread's loads of several
// elements are all in flight together instead of one round trip each.
__device__ __forceinline__ float a_elem(int kind, const float2* __restrict__ Bbar,
                                        const float2* __restrict__ C, int H, int P, int i, int k) {
  const bool k0 = kind != 1;
  const int pb = kind == 2 ? 16 * (i >> 5) + (i & 15) : i >> 1;  // state of a Bbar row
  const bool imb = kind == 2 ? ((i >> 4) & 1) : (i & 1);         // its imaginary part
  const bool in = k0 ? (pb < P && k < H) : (i < H && k < 2 * P);
  const size_t idx = k0 ? (size_t)min(pb, P - 1) * H + min(k, H - 1)
                        : (size_t)min(i, H - 1) * P + min(k >> 1, P - 1);
  const float2 v = (k0 ? Bbar : C)[idx];
  const float e = k0 ? (imb ? v.y : v.x) : ((k & 1) ? -v.y : v.x);
  return in ? e : 0.f;
}

// A^T as the B operand of v_mfma_f32_16x16x32_f16, split: for row tile it
// (rows 16 it .. + 15) and k step ks (32 k), lane l holds
// A[16 it + l % 16][32 ks + 8 (l / 16) + e] * 2^rexp[i], e < 8, as fp16 hi and
// lo: apk[((it * KS + ks) * 2 + hl) * 64 + l].  rexp[i] brings row i's largest
// magnitude into [2^14, 2^15).  One workgroup per (row tile, kind); a row
// tile past a kind's rows returns at once (the whole workgroup).
__global__ __launch_bounds__(256) void s5_pack_kernel(const float2* __restrict__ Bbar,
                                                      const float2* __restrict__ C, int H, int P,
                                                      half8* __restrict__ apk_in,
                                                      int* __restrict__ rexp_in,
                                                      half8* __restrict__ apk_out,
                                                      int* __restrict__ rexp_out, int fused, int kpad) {
  __shared__ float red[16][17];
  __shared__ int rexp_s[16];
  const int kind = blockIdx.y == 1 ? 1 : (fused ? 2 : 0);
  const int M = kind == 0 ? 2 * P : kind == 2 ? 64 * ((32 * ((P + 15) / 16) + 63) / 64) : H;
  const int K = kind == 1 ? 2 * P : H;
  const int it = blockIdx.x;
  if (16 * it >= M) return;
  const int KS = kpad > 0 ? kpad : (K + 31) / 32;  // k steps (zero past K)
  const int t = threadIdx.x, r = t & 15, part = t >> 4;
  // row maxima: thread (r, part) scans k = part, part + 16, ... (16 independent
  // loads in flight per step: one step covers K = 256)
  float m = 0.f;
  for (int k0 = part; k0 < K; k0 += 16 * 16) {
    float e16[16];
#pragma unroll
    for (int e = 0; e < 16; ++e)
      e16[e] = fabsf(a_elem(kind, Bbar, C, H, P, 16 * it + r, k0 + 16 * e));
#pragma unroll
    for (int e = 0; e < 16; ++e) m = fmaxf(m, e16[e]);
  }
  red[r][part] = m;
  __syncthreads();
  if (t < 16) {
    float mm = 0.f;
    for (int q = 0; q < 16; ++q) mm = fmaxf(mm, red[t][q]);
    rexp_s[t] = scale_exp(mm);
    (kind != 1 ? rexp_in : rexp_out)[16 * it + t] = rexp_s[t];
  }
  __syncthreads();
  half8* out = (kind != 1 ? apk_in : apk_out) + (size_t)it * KS * 2 * 64;
  // fragments: two (k step, lane) entries per thread and step, all 16 loads
  // issued before the first is used
  for (int idx0 = t; idx0 < KS * 64; idx0 += 512) {
    float v[2][8];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int idx = idx0 + 256 * h2;
      const int ks = idx >> 6, l = idx & 63;
      const int i = 16 * it + (l & 15), k0 = 32 * ks + 8 * (l >> 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[h2][e] = idx < KS * 64 ? a_elem(kind, Bbar, C, H, P, i, k0 + e) : 0.f;
    }
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int idx = idx0 + 256 * h2;
      if (idx >= KS * 64) break;
      const int ks = idx >> 6, l = idx & 63;
      half8 hi, lo;
      split8(v[h2], hi, lo, rexp_s[l & 15]);
      out[(size_t)(ks * 2) * 64 + l] = hi;
      out[(size_t)(ks * 2 + 1) * 64 + l] = lo;
    }
  }
}

// The same fragments and exponents for K <= kPackLdsK, with one read of the
// matrices: workgroup (row tile it, kind, k group g) stages the tile's 16
// rows (all K) in LDS, takes each row's maximum there, and writes the
// fragments of k steps kPackKS g .. + kPackKS - 1 (the row maxima are formed
// redundantly by the k groups of a tile; the k group 0 writes the exponents).
constexpr int kPackLdsK = 1024;
constexpr int kPackKS = 2;  // k steps (of 32) per workgroup
__global__ __launch_bounds__(256) void s5_pack_lds_kernel(const float2* __restrict__ Bbar,
                                                          const float2* __restrict__ C, int H,
                                                          int P, half8* __restrict__ apk_in,
                                                          int* __restrict__ rexp_in,
                                                          half8* __restrict__ apk_out,
                                                          int* __restrict__ rexp_out, int fused, int kpad) {
  __shared__ float A[16][kPackLdsK + 4];
  __shared__ float red[16][17];
  __shared__ int rexp_s[16];
  const int kind = blockIdx.y == 1 ? 1 : (fused ? 2 : 0);
  const int M = kind == 0 ? 2 * P : kind == 2 ? 64 * ((32 * ((P + 15) / 16) + 63) / 64) : H;
  const int K = kind == 1 ? 2 * P : H;
  const int it = blockIdx.x, g = blockIdx.z;
  const int KS = kpad > 0 ? kpad : (K + 31) / 32;  // k steps (zero past K)
  if (16 * it >= M || kPackKS * g >= KS) return;  // the whole workgroup
  const int KP = 32 * KS;  // staged row length (zero past K)
  const int t = threadIdx.x;
  // stage: thread (row t / 16, c = t % 16) takes columns c + 16 q, sixteen
  // loads in flight per round
  {
    const int r = t >> 4, c = t & 15;
    for (int q0 = 0; 16 * q0 < KP; q0 += 16) {
      float v[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) v[q] = a_elem(kind, Bbar, C, H, P, 16 * it + r, c + 16 * (q0 + q));
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (16 * (q0 + q) < KP) A[r][c + 16 * (q0 + q)] = v[q];
    }
  }
  __syncthreads();
  {
    const int r = t & 15, part = t >> 4;
    float m = 0.f;
    for (int k = part; k < KP; k += 16) m = fmaxf(m, fabsf(A[r][k]));
    red[r][part] = m;
  }
  __syncthreads();
  if (t < 16) {
    float mm = 0.f;
    for (int q = 0; q < 16; ++q) mm = fmaxf(mm, red[t][q]);
    rexp_s[t] = scale_exp(mm);
    if (g == 0) (kind != 1 ? rexp_in : rexp_out)[16 * it + t] = rexp_s[t];
  }
  __syncthreads();
  const int ks = kPackKS * g + (t >> 6);
  if (t < 64 * kPackKS && ks < KS) {
    const int l = t & 63, i = l & 15, k0 = 32 * ks + 8 * (l >> 4);
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = A[i][k0 + e];
    half8 hi, lo;
    split8(v, hi, lo, rexp_s[i]);
    half8* out = (kind != 1 ? apk_in : apk_out) + (size_t)it * KS * 2 * 64;
    out[(size_t)(ks * 2) * 64 + l] = hi;
    out[(size_t)(ks * 2 + 1) * 64 + l] = lo;
  }
}

// out[b][i][j] = sum_k A[i][k] Bm[b][k][j]  (+ D[i] u[b][i][j] when kAddDu);
// Bm [B][K][L] row-major, out [B][M][L].  Computed transposed, outT = Bm^T A^T,
// so each lane's four results are consecutive time steps (16-byte stores).
// Per k chunk the workgroup stages Bm[chunk][j0 .. j0 + kColsWG) in LDS as
// BT[j][k] (fp16 hi and lo), each column j scaled by 2^cexp[j] from its
// largest magnitude in the chunk; the A^T fragments come prepacked (scaled per
// row).  With several k chunks (kMulti) each chunk's products are unscaled into
// a running total.
template <bool kAddDu, bool kMulti>
__global__ __launch_bounds__(256, 2) void s5_gemm_kernel(const half8* __restrict__ apk,
                                                         const int* __restrict__ rexp,
                                                         const float* __restrict__ Bm, int M,
                                                         int K, int L, const float* __restrict__ D,
                                                         const float* __restrict__ u,
                                                         float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) _Float16 Bh[kColsWG][kBTS];
  __shared__ __attribute__((aligned(16))) _Float16 Bl[kColsWG][kBTS];
  __shared__ float cmax[4][kColsWG];
  __shared__ __attribute__((aligned(16))) int cexp[kColsWG];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, g = lane >> 4;
  const int b = blockIdx.z;
  const int j0 = blockIdx.x * kColsWG;
  const int i0 = blockIdx.y * kRowsWG + 64 * w;  // this wave's first row
  const bool rows_here = i0 < M;                  // waves past M load but do not multiply
  const int KS = (K + 31) / 32;
  const float* Bb = Bm + (size_t)b * K * L;

  v4f acc[kNJ][4], tot[kNJ][4];
#pragma unroll
  for (int jt = 0; jt < kNJ; ++jt)
#pragma unroll
    for (int it = 0; it < 4; ++it) tot[jt][it] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int kc = 0; kc < K; kc += kKC) {
    if (kc) __syncthreads();  // the previous chunk's tile is read
    // 1. tile: thread (column j = lane, wave w) loads k = kc + 8 (w + 4 q) + e,
    //    q < 8, e < 8: each load instruction reads 64 consecutive columns of one
    //    row, through a raw buffer over that row (a wave-uniform descriptor):
    //    columns past L read zero, and a row past K has an empty range.  No
    //    load sits under a branch (each would be waited on).
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const unsigned jb = 4u * (unsigned)(j0 + lane);
    float v[kQL][8];
#pragma unroll
    for (int q = 0; q < kQL; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = kc + 8 * (wu + 4 * q) + e;
        const BufRes row =
            buf_res_uniform(Bb + (size_t)min(k, K - 1) * L, k < K ? 4u * (unsigned)L : 0u);
        v[q][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(row, jb, 0, 0));
      }
    __builtin_amdgcn_sched_barrier(0);  // every load of the tile in flight before the first wait
    float m = 0.f;
#pragma unroll
    for (int q = 0; q < kQL; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[q][e]));
    cmax[w][lane] = m;
    __syncthreads();
    const int sc = scale_exp(fmaxf(fmaxf(cmax[0][lane], cmax[1][lane]),
                                   fmaxf(cmax[2][lane], cmax[3][lane])));
    if (w == 0) cexp[lane] = sc;
#pragma unroll
    for (int q = 0; q < kQL; ++q) {
      half8 hi, lo;
      split8(v[q], hi, lo, sc);
      *reinterpret_cast<half8*>(&Bh[lane][8 * (w + 4 * q)]) = hi;
      *reinterpret_cast<half8*>(&Bl[lane][8 * (w + 4 * q)]) = lo;
    }
    __syncthreads();

    // 2. outT[j][i] for the kColsWG columns (tiles jt) by this wave's 64 rows (4 tiles it)
#pragma unroll
    for (int jt = 0; jt < kNJ; ++jt)
#pragma unroll
      for (int it = 0; it < 4; ++it) acc[jt][it] = v4f{0.f, 0.f, 0.f, 0.f};
    if (rows_here) {
      const int ks0 = kc / 32, ks1 = min(KS, (kc + kKC) / 32);
      const half8* ap = apk + (size_t)(i0 / 16) * KS * 2 * 64 + lane;
      // A^T fragments of k step ks into buffer slot (the next step's loads are
      // in flight while the current step multiplies)
      half8 ah[2][4], al[2][4];
      auto load_a = [&](int ks, int slot) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const half8* f = ap + ((size_t)it * KS + ks) * 2 * 64;
          ah[slot][it] = f[0];
          al[slot][it] = f[64];
        }
      };
      auto multiply = [&](int ks, int slot) {
        const int kk = 32 * (ks - ks0) + 8 * g;
#pragma unroll
        for (int jt = 0; jt < kNJ; ++jt) {
          const half8 bh = *reinterpret_cast<const half8*>(&Bh[16 * jt + (lane & 15)][kk]);
          const half8 bl = *reinterpret_cast<const half8*>(&Bl[16 * jt + (lane & 15)][kk]);
#pragma unroll
          for (int it = 0; it < 4; ++it) {
            acc[jt][it] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bh, ah[slot][it], acc[jt][it], 0, 0, 0);
            acc[jt][it] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bh, al[slot][it], acc[jt][it], 0, 0, 0);
            acc[jt][it] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bl, ah[slot][it], acc[jt][it], 0, 0, 0);
          }
        }
      };
      // Loads are unconditional (a step index past the chunk is clamped, the
      // fragments then simply unused): a load under a branch would make the
      // wait at the join cover the prefetch too.
      load_a(ks0, 0);
      for (int ks = ks0; ks < ks1; ks += 2) {
        load_a(min(ks + 1, ks1 - 1), 1);
        multiply(ks, 0);
        load_a(min(ks + 2, ks1 - 1), 0);
        if (ks + 1 < ks1) multiply(ks + 1, 1);
      }
    }
    // acc[jt][it][v]: column j0 + 16 jt + 4 g + v, row i0 + 16 it + lane % 16
    if (kMulti) {
#pragma unroll
      for (int jt = 0; jt < kNJ; ++jt) {
        const int4 ce = *reinterpret_cast<const int4*>(&cexp[16 * jt + 4 * g]);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          tot[jt][it][0] += __builtin_amdgcn_ldexpf(acc[jt][it][0], -ce.x);
          tot[jt][it][1] += __builtin_amdgcn_ldexpf(acc[jt][it][1], -ce.y);
          tot[jt][it][2] += __builtin_amdgcn_ldexpf(acc[jt][it][2], -ce.z);
          tot[jt][it][3] += __builtin_amdgcn_ldexpf(acc[jt][it][3], -ce.w);
        }
      }
    }
  }
  if (!rows_here) return;  // no barriers follow

  // 3. epilogue: unscale (row exponent, and the column exponents of a single
  //    chunk), add D u, store four consecutive time steps per lane.  The u
  //    loads are all issued before the first store (a load issued after a
  //    store would wait for it).
  const bool vec = (L & 3) == 0;
  float* ob = out + (size_t)b * M * L;
  v4f du[kNJ][4];
  if (kAddDu) {
    const float* ub = u + (size_t)b * M * L;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int i = i0 + 16 * it + (lane & 15);
      const float d = i < M ? D[i] : 0.f;
#pragma unroll
      for (int jt = 0; jt < kNJ; ++jt) {
        const int jj = j0 + 16 * jt + 4 * g;
        if (vec) {
          const bool ok = i < M && jj + 3 < L;
          const v4f x = *reinterpret_cast<const v4f*>(ok ? ub + (size_t)i * L + jj : ub);
          du[jt][it] = ok ? d * x : v4f{0.f, 0.f, 0.f, 0.f};
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const bool ok = i < M && jj + c < L;
            const float x = *(ok ? ub + (size_t)i * L + jj + c : ub);
            du[jt][it][c] = ok ? d * x : 0.f;
          }
        }
      }
    }
  }
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int i = i0 + 16 * it + (lane & 15);
    if (i >= M) continue;
    const int re = rexp[i];
    float* orow = ob + (size_t)i * L;
#pragma unroll
    for (int jt = 0; jt < kNJ; ++jt) {
      const int jj = j0 + 16 * jt + 4 * g;
      v4f o;
      if (kMulti) {
#pragma unroll
        for (int c = 0; c < 4; ++c) o[c] = __builtin_amdgcn_ldexpf(tot[jt][it][c], -re);
      } else {
        const int4 ce = *reinterpret_cast<const int4*>(&cexp[16 * jt + 4 * g]);
        o[0] = __builtin_amdgcn_ldexpf(acc[jt][it][0], -(re + ce.x));
        o[1] = __builtin_amdgcn_ldexpf(acc[jt][it][1], -(re + ce.y));
        o[2] = __builtin_amdgcn_ldexpf(acc[jt][it][2], -(re + ce.z));
        o[3] = __builtin_amdgcn_ldexpf(acc[jt][it][3], -(re + ce.w));
      }
      if (kAddDu) o += du[jt][it];
      if (vec && jj + 3 < L) {
        *reinterpret_cast<v4f*>(orow + jj) = o;
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (jj + c < L) orow[jj + c] = o[c];
      }
    }
  }
}

#ifdef DSSM_PHASE_STAMPS
constexpr size_t kProjInRows = 8192;  // stamp rows of the output projection before the input's
#endif

// Persistent form for K <= 256 (one k chunk).  A workgroup of 8 waves owns
// 256 rows (32 per wave: its split A^T fragments stay in registers for the
// whole kernel, read from L2 once) and walks the column tiles t = blockIdx.x,
// blockIdx.x + gridDim.x, ... over all batch rows.  The right-hand tile of the
// next column tile is loaded straight into LDS (buffer-to-LDS loads, no
// registers) while the current one is multiplied from the split tile; the
// u of the current tile's D u terms (output projection) is requested before
// it, so that wait -- memory loads retiring in issue order -- never holds for
// the next tile.
constexpr int kPW = 8;  // waves per workgroup of the persistent form

// VEC: L % 4 == 0 (16-byte accesses along the sequence)
template <bool kAddDu, bool VEC>
__global__ __launch_bounds__(512, 1) void s5_gemm_pipe_kernel(
    const half8* __restrict__ apk, const int* __restrict__ rexp, const float* __restrict__ Bm,
    int M, int K, int L, int B, const float* __restrict__ D, const float* __restrict__ u,
    float* __restrict__ out) {
  PhaseClock pc;  // phase stamps (instrumented builds only): slots below
  __shared__ __attribute__((aligned(16))) _Float16 Bh[kColsWG][kBTS];
  __shared__ __attribute__((aligned(16))) _Float16 Bl[kColsWG][kBTS];
  __shared__ __attribute__((aligned(16))) float Braw[kKC][kColsWG];  // the next tile, fp32
  __shared__ float cmax[kPW][kColsWG];
  __shared__ __attribute__((aligned(16))) int cexp[kColsWG];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, g = lane >> 4;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int i0 = blockIdx.y * kRowsWG + 32 * w;  // this wave's first row
  const bool rows_here = i0 < M;
  const int KS = (K + 31) / 32;  // <= 8
  const int njb = (L + kColsWG - 1) / kColsWG;
  const int ntiles = B * njb;

  // this wave's A^T fragments: row tiles i0 / 16 + it (it < 2), k steps < KS
  half8 ah[2][8], al[2][8];
  int rx[2] = {0, 0};
  if (rows_here) {
    const half8* ap = apk + (size_t)(i0 / 16) * KS * 2 * 64 + lane;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const half8* f = ap + ((size_t)it * KS + min(ks, KS - 1)) * 2 * 64;
        ah[it][ks] = f[0];
        al[it][ks] = f[64];
      }
      const int i = i0 + 16 * it + (lane & 15);
      rx[it] = rexp[min(i, M - 1)];
    }
  }

  // right-hand tile tt = (b, jb) into Braw[k][column]: wave w requests rows
  // k = 8 (w + 8 q) + e (q < 4, e < 8), the rows its own threads read back in
  // stage().  VEC: four rows per load, 16 bytes (four columns) per lane,
  // through one raw buffer over the batch row's K x L floats (rows past K read
  // zero; columns past L read the next row's, or zero, and only feed outputs
  // past L, which are not stored); else one row per load, a dword per lane,
  // through a buffer over that row (columns past L read zero).
  auto load_tile = [&](int tt) {
    const int b = tt / njb, jb = tt - b * njb;
    const float* Bb = Bm + (size_t)b * K * L;
    if (VEC) {
      const BufRes all = buf_res_uniform(Bb, 4u * (unsigned)K * (unsigned)L);
      const int rl = lane >> 4, cl = 4 * (lane & 15);  // row within the four, first column
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e4 = 0; e4 < 2; ++e4) {
          const int k = 8 * (wu + kPW * q) + 4 * e4;  // first of four rows
          const unsigned off = 4u * ((unsigned)(k + rl) * (unsigned)L + (unsigned)(jb * kColsWG + cl));
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              all, (__attribute__((address_space(3))) void*)&Braw[k][0], 16, off, 0, 0, 0);
        }
    } else {
      const unsigned jbyte = 4u * (unsigned)(jb * kColsWG + lane);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int k = 8 * (wu + kPW * q) + e;
          const BufRes row =
              buf_res_uniform(Bb + (size_t)min(k, K - 1) * L, k < K ? 4u * (unsigned)L : 0u);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              row, (__attribute__((address_space(3))) void*)&Braw[k][0], 4, jbyte, 0, 0, 0);
        }
    }
  };
  // the requested tile, scaled per column by 2^cexp and split into Bh / Bl
  // (after every wave's product has read the previous tile: the first barrier)
  auto stage = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's rows are in Braw
    float v[4][8];
    float m = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[q][e] = Braw[8 * (w + kPW * q) + e][lane];
        m = fmaxf(m, fabsf(v[q][e]));
      }
    cmax[w][lane] = m;
    __syncthreads();
    float cm = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < kPW; ++w2) cm = fmaxf(cm, cmax[w2][lane]);
    const int sc = scale_exp(cm);
    if (w == 0) cexp[lane] = sc;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      half8 hi, lo;
      split8(v[q], hi, lo, sc);
      *reinterpret_cast<half8*>(&Bh[lane][8 * (w + kPW * q)]) = hi;
      *reinterpret_cast<half8*>(&Bl[lane][8 * (w + kPW * q)]) = lo;
    }
    __syncthreads();
  };

  int tt = blockIdx.x;
  if (tt < ntiles) {
    load_tile(tt);
    stage();
  }
  pc.mark(0);  // prologue: fragments, first tile loaded and staged
  for (; tt < ntiles; tt += gridDim.x) {
    const int tn = tt + gridDim.x;
    const bool has_next = tn < ntiles;  // the same in the whole workgroup
    const int b = tt / njb, jb = tt - b * njb;
    // u of this lane's outputs (for D u), requested before the next tile: every
    // load unconditional, at a clamped address (positions past L masked in the
    // epilogue), and nothing computed from them before the product
    v4f du[2][4];
    float dv[2];
    if (kAddDu) {
      const float* ub = u + (size_t)b * M * L;
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int i = min(i0 + 16 * it + (lane & 15), M - 1);
        dv[it] = D[i];
        const float* urow = ub + (size_t)i * L;
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          const int jj = jb * kColsWG + 16 * jt + 4 * g;
          if (VEC) {
            du[it][jt] = *reinterpret_cast<const v4f*>(urow + min(jj, L - 4));
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) du[it][jt][c] = urow[min(jj + c, L - 1)];
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // (the u loads stay ahead of the tile's)
    load_tile(has_next ? tn : tt);  // unconditional: no load under a branch
    pc.mark(1);  // D u and the next tile requested

    v4f acc[4][2];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) acc[jt][0] = acc[jt][1] = v4f{0.f, 0.f, 0.f, 0.f};
    if (rows_here) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        if (ks >= KS) break;
        const int kk = 32 * ks + 8 * g;
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          const half8 bh = *reinterpret_cast<const half8*>(&Bh[16 * jt + (lane & 15)][kk]);
          const half8 bl = *reinterpret_cast<const half8*>(&Bl[16 * jt + (lane & 15)][kk]);
#pragma unroll
          for (int it = 0; it < 2; ++it) {
            acc[jt][it] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bh, ah[it][ks], acc[jt][it], 0, 0, 0);
            acc[jt][it] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bh, al[it][ks], acc[jt][it], 0, 0, 0);
            acc[jt][it] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bl, ah[it][ks], acc[jt][it], 0, 0, 0);
          }
        }
      }
      pc.mark(2);  // product (matrix cores)
    }
    if (kAddDu) {  // the D u terms arrive here, after the product (in every wave: no
                   // branch the compiler could sink their loads into)
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        asm volatile("" : "+v"(dv[it]));
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) asm volatile("" : "+v"(du[it][jt]));
      }
    }
    if (rows_here) {
      // acc[jt][it][c]: column 64 jb + 16 jt + 4 g + c, row i0 + 16 it + lane % 16
      float* ob = out + (size_t)b * M * L;
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int i = i0 + 16 * it + (lane & 15);
        if (i >= M) continue;
        float* orow = ob + (size_t)i * L;
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          const int jj = jb * kColsWG + 16 * jt + 4 * g;
          const int4 ce = *reinterpret_cast<const int4*>(&cexp[16 * jt + 4 * g]);
          v4f o;
          o[0] = __builtin_amdgcn_ldexpf(acc[jt][it][0], -(rx[it] + ce.x));
          o[1] = __builtin_amdgcn_ldexpf(acc[jt][it][1], -(rx[it] + ce.y));
          o[2] = __builtin_amdgcn_ldexpf(acc[jt][it][2], -(rx[it] + ce.z));
          o[3] = __builtin_amdgcn_ldexpf(acc[jt][it][3], -(rx[it] + ce.w));
          if (kAddDu) {
#pragma unroll
            for (int c = 0; c < 4; ++c) o[c] += jj + c < L ? dv[it] * du[it][jt][c] : 0.f;
          }
          if (VEC && jj + 3 < L) {
            *reinterpret_cast<v4f*>(orow + jj) = o;
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (jj + c < L) orow[jj + c] = o[c];
          }
        }
      }
    }
    pc.mark(3);  // outputs scaled (D u added), stores issued
    if (has_next) stage();
    pc.mark(4);  // next tile received, scaled, split, staged (two barriers)
  }
#ifdef DSSM_PHASE_STAMPS
  // (the input projection writes its stamps past the output projection's:
  // rows from kProjInRows on, so one forward leaves both)
  if (!kAddDu && g_phase_buf && (threadIdx.x & 63) == 0) {
    const size_t wgl = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
    const size_t base = (kProjInRows + wgl * (blockDim.x >> 6) + (threadIdx.x >> 6)) * kPhaseSlots;
    for (int k = 0; k < kPhaseSlots; ++k) g_phase_buf[base + k] = pc.acc[k];
  } else {
    pc.write();
  }
#else
  pc.write();
#endif
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
// so the per-lane reads are conflict-free).  With L a multiple of 4 the next
// tile is loaded into registers once the current one is in LDS and its
// segments' end states are formed, so the loads overlap the carries, the
// outputs and the stores of the current tile.
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

  // float4 groups e = 4 (t + kLanes k) of the next tile (zero beyond L; with
  // L a multiple of 4 a group lies wholly inside or outside)
  constexpr int kG = kTile / (4 * kLanes);
  float4 nre[kG], nim[kG];
  auto fetch = [&](int at) {
    const int m = min(kTile, L - at);
#pragma unroll
    for (int k = 0; k < kG; ++k) {
      const int e = 4 * (t + kLanes * k);
      nre[k] = nim[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e < m) {
        nre[k] = *reinterpret_cast<const float4*>(vre + at + e);
        nim[k] = *reinterpret_cast<const float4*>(vim + at + e);
      }
    }
  };
  if (vec) fetch(0);

  for (int base = 0; base < L; base += kTile) {
    const int n = min(kTile, L - base);
    // stage the tile (zero beyond L)
    if (vec) {
#pragma unroll
      for (int k = 0; k < kG; ++k) {
        const int q = tpad(4 * (t + kLanes * k));  // the 4 slots stay contiguous
        const float4 a = nre[k], c = nim[k];
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
    if (vec && base + kTile < L) fetch(base + kTile);
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

// The same recurrence for a continuous-time system with a step size that
// changes from step to step ("Simplified State Space Layers for Sequence
// Modeling", section 3: zero-order hold of a diagonal system with a timescale
// per state; a different timescale supplied at each step for irregular
// sampling): with z = lam_c[p] step[b,k] delta[p],
//   x_k = exp(z) x_{k-1} + (exp(z) - 1) / lam_c[p] v_k     (v = B~ u)
// ((exp(z) - 1) / lam_c -> step delta as lam_c -> 0).  The per-step
// multipliers differ, so the carries use the general associative pair
// (A, X) o (A', X') = (A' A, A' X + X'): each lane folds its 16 steps into
// (A, X), a wave combines its lanes by shuffles, the four waves through LDS,
// and the tile's total carries into the next tile; the next tile's inputs are
// loaded while the current one's carries and outputs are formed.  z is formed in float64 and its
// phase reduced there to a quadrant and a remainder in [-pi/4, pi/4]; the
// exponential, the sine and cosine and exp(z) - 1 (as expm1(a) cos b -
// (1 - cos b) + i e^a sin b, 1 - cos b without cancellation) then run in
// float32.

// sin and cos of x = q pi/2 + r, |r| <= pi/4, from the Taylor series of sin r
// (to r^9) and cos r (to r^10): truncation below 3e-9 relative on that range;
// the quadrant q (mod 4) swaps the pair and flips signs, without branches.
__device__ __forceinline__ void sincos_quadrant(float r, int q, float& sn, float& cs) {
  const float r2 = r * r;
  float ps = fmaf(r2, 1.f / 362880.f, -1.f / 5040.f);
  ps = fmaf(ps, r2, 1.f / 120.f);
  ps = fmaf(ps, r2, -1.f / 6.f);
  const float s = fmaf(ps * r2, r, r);
  float pc = fmaf(r2, -1.f / 3628800.f, 1.f / 40320.f);
  pc = fmaf(pc, r2, -1.f / 720.f);
  pc = fmaf(pc, r2, 1.f / 24.f);
  pc = fmaf(pc, r2, -0.5f);
  const float c = fmaf(pc, r2, 1.f);
  const bool odd = (q & 1) != 0;
  // q = 0: (s, c); 1: (c, -s); 2: (-s, -c); 3: (-c, s)
  sn = __int_as_float(__float_as_int(odd ? c : s) ^ ((q & 2) << 30));
  cs = __int_as_float(__float_as_int(odd ? s : c) ^ (((q + 1) & 2) << 30));
}

// (ir, ii) = 1 / lam_c; lam_zero: lam_c = 0 (then the gain is the step length).
__device__ __forceinline__ void zoh_step(float lr, float li, float ir, float ii, bool lam_zero,
                                         double ld, float s, float2& a, float2& beta) {
  const double dt = ld * (double)s;
  const double zr = (double)lr * dt, zi = (double)li * dt;
  // phase: quadrant q and remainder |r| <= pi/4 in float64
  const double kHalfPi = 1.5707963267948966192313216916398;
  const double kInvHalfPi = 0.63661977236758134307553505349006;
  const double q = rint(zi * kInvHalfPi);
  const double q4 = fma(-4.0, floor(q * 0.25), q);  // q mod 4, exact
  float sn, cs;
  sincos_quadrant((float)fma(-q, kHalfPi, zi), (int)q4, sn, cs);
  const float em1r = expm1f((float)zr);
  const float e = 1.f + em1r;
  a = make_float2(e * cs, e * sn);
  // 1 - cos b without cancellation: sin^2 b / (1 + cos b) for cos b > 0, both
  // forms evaluated and one selected
  const float omc_pos = sn * sn * __builtin_amdgcn_rcpf(1.f + fmaxf(cs, 0.f));
  const float omc = cs > 0.f ? omc_pos : 1.f - cs;
  const float2 em1 = make_float2(em1r * cs - omc, e * sn);
  beta = lam_zero ? make_float2((float)dt, 0.f)
                  : make_float2(em1.x * ir - em1.y * ii, em1.x * ii + em1.y * ir);
}

__global__ __launch_bounds__(kLanes) __attribute__((amdgpu_waves_per_eu(2))) void s5_scan_tv_kernel(const float2* __restrict__ lam_c,
                                                            const float* __restrict__ delta,
                                                            const float* __restrict__ step,
                                                            const float* __restrict__ v, int P,
                                                            int L, float* __restrict__ x) {
  __shared__ float sre[kPadT], sim[kPadT], sst[kPadT];
  __shared__ float2 bA[4], bX[4];  // per-wave inclusive totals
  __shared__ float2 carry;
  const int p = blockIdx.x % P;
  const int b = blockIdx.x / P;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const float2 lm = lam_c[p];
  const double ld = (double)delta[p];
  const float den = lm.x * lm.x + lm.y * lm.y;
  const bool lam_zero = !(den > 0.f);
  const float ir = lam_zero ? 0.f : lm.x / den, ii = lam_zero ? 0.f : -lm.y / den;
  if (t == 0) carry = make_float2(0.f, 0.f);

  const float* vre = v + ((size_t)b * P + p) * 2 * L;
  const float* vim = vre + L;
  const float* srow = step + (size_t)b * L;
  float* xre = x + ((size_t)b * P + p) * 2 * L;
  float* xim = xre + L;

  // the next tile's elements t + kLanes i (zero beyond L)
  float nre[kSeg], nim[kSeg], nst[kSeg];
  auto fetch = [&](int at) {
    const int m = min(kTile, L - at);
#pragma unroll
    for (int i = 0; i < kSeg; ++i) {
      const int e = t + kLanes * i;
      const bool in = e < m;
      nre[i] = in ? vre[at + e] : 0.f;
      nim[i] = in ? vim[at + e] : 0.f;
      nst[i] = in ? srow[at + e] : 0.f;
    }
  };
  fetch(0);
  for (int base = 0; base < L; base += kTile) {
    const int n = min(kTile, L - base);
#pragma unroll
    for (int i = 0; i < kSeg; ++i) {  // stage the tile
      const int q = tpad(t + kLanes * i);
      sre[q] = nre[i];
      sim[q] = nim[i];
      sst[q] = nst[i];
    }
    __syncthreads();
    float2 va[kSeg], vb[kSeg];  // multipliers, input gains times inputs
    float2 A = make_float2(1.f, 0.f), X = make_float2(0.f, 0.f);
#pragma unroll
    for (int i = 0; i < kSeg; ++i) {
      const int q = 17 * t + i;  // tpad(16 t + i)
      float2 a, beta;
      zoh_step(lm.x, lm.y, ir, ii, lam_zero, ld, sst[q], a, beta);
      va[i] = a;
      vb[i] = cm(beta, make_float2(sre[q], sim[q]));
      const float2 m = cm(a, X);
      X = make_float2(m.x + vb[i].x, m.y + vb[i].y);
      A = cm(a, A);
    }
    // the next tile's loads overlap the carries, the outputs and the stores
    // (issued after the steps' arithmetic, whose temporaries need the registers)
    if (base + kTile < L) fetch(base + kTile);
    // inclusive scan inside the wave: earlier (A', X') then this lane's (A, X)
#pragma unroll
    for (int j = 0; j < 6; ++j) {
      const int o = 1 << j;
      const int src = max(lane - o, 0);
      const float2 pA = make_float2(__shfl(A.x, src), __shfl(A.y, src));
      const float2 pX = make_float2(__shfl(X.x, src), __shfl(X.y, src));
      if (lane >= o) {
        const float2 m = cm(A, pX);
        X = make_float2(m.x + X.x, m.y + X.y);
        A = cm(A, pA);
      }
    }
    if (lane == 63) {
      bA[w] = A;
      bX[w] = X;
    }
    __syncthreads();
    const float2 cin = carry;
    // prefix of the earlier waves, then the carried state
    float2 wA = make_float2(1.f, 0.f), wX = make_float2(0.f, 0.f);
    for (int k = 0; k < w; ++k) {
      const float2 m = cm(bA[k], wX);
      wX = make_float2(m.x + bX[k].x, m.y + bX[k].y);
      wA = cm(bA[k], wA);
    }
    {
      const float2 m = cm(wA, cin);
      wX = make_float2(wX.x + m.x, wX.y + m.y);  // state entering wave w
    }
    {
      const float2 m = cm(A, wX);
      X = make_float2(X.x + m.x, X.y + m.y);  // state after this lane's steps
    }
    float2 xin;  // state before this lane's steps
    {
      const float2 q = make_float2(__shfl(X.x, max(lane - 1, 0)), __shfl(X.y, max(lane - 1, 0)));
      xin = lane == 0 ? wX : q;
    }
    __syncthreads();  // everyone has read `carry`, the totals and its inputs
    if (t == kLanes - 1) carry = X;
    float2 st = xin;
#pragma unroll
    for (int i = 0; i < kSeg; ++i) {
      const float2 m = cm(va[i], st);
      st = make_float2(m.x + vb[i].x, m.y + vb[i].y);
      const int q = 17 * t + i;
      sre[q] = st.x;
      sim[q] = st.y;
    }
    __syncthreads();
    for (int e = t; e < n; e += kLanes) {
      xre[base + e] = sre[tpad(e)];
      xim[base + e] = sim[tpad(e)];
    }
    __syncthreads();  // the tile's buffers are read before the next tile's staging
  }
}

// ---------------------------------------------------------------------------
// Fused S5 form (P <= 128, H <= 256): per 64-step tile of one batch row,
// v = Bbar u on the matrix cores, the recurrence on the tile in registers, and
// y = Re(C x) + D u on the matrix cores, so v and x never leave the CU.  The
// sequence of a batch row is cut into segments of whole tiles (one workgroup
// each).  A state-only pass (the input projection and the recurrence from
// zero) leaves the state at the end of every segment but the last; the output
// pass forms the state entering its segment from those (float64 Horner steps
// with lambda^S, S the steps of a segment) and runs the whole tile pipeline.
//
// One workgroup of 4 waves per CU, one wave per SIMD (so a wave may hold up to
// 512 registers: accumulators and operands of 16 independent products, and in
// the state-only pass the input projection's fragments).  LDS: the fp32 u tile
// [H][64] (filled by buffer-to-LDS loads one tile ahead, so u needs no
// registers in flight), the staged right-hand operand [64 steps][256 k] as
// fp16 hi and lo (u, then x), per-step maxima and exponents.  Wave w owns 64
// rows of each product: for the input projection the real and the imaginary
// rows of states 32 w .. 32 w + 31, 16 states per 32 rows (the packed Bbar
// takes that row order), so after the product lane (q, g) holds v of states
// 32 w + q and 32 w + 16 + q at the 16 consecutive steps 16 g .. 16 g + 15 of
// the tile (the staged operand's rows are read in that time order).  The
// recurrence: a float32 chain of 16 steps from zero per lane and state, the
// four quarters joined with lambda^16, lambda^32, lambda^48 (float64, rounded
// once), each step completed by lambda^(j+1) times its quarter's entering
// state, the tile's last state by lambda^64.  The output projection's operand
// x is scaled per step (the largest magnitude over all 2P rows, across the
// waves through LDS) and split into fp16 hi and lo like u.
// ---------------------------------------------------------------------------
constexpr int kFT = kColsWG;  // steps per tile

struct S5FusedArgs {
  const half8* apk_in;  // Bbar as A in the fused row order (s5_fused_rows), K = H
  const int* rexp_in;
  const half8* apk_out;  // C as A: M = H rows, K = 2P
  const int* rexp_out;
  const float* u;
  const float2* lam;
  const float* D;
  float* y;
  float2* sout;  // [B][nseg][P]: the state leaving each segment but the last
  const float4* lp;     // [P][2]: lambda^16, lambda^32 | lambda^48, lambda^64
  const double2* apow;  // [P][nseg]: lambda^(S n), S the steps of a segment
  int B, H, P, L, nseg, seg_tiles;
};

__device__ __forceinline__ float2 cmad(float2 m, float2 x, float2 c) {  // m x + c
  return make_float2(fmaf(m.x, x.x, fmaf(-m.y, x.y, c.x)), fmaf(m.x, x.y, fmaf(m.y, x.x, c.y)));
}

// lambda^k from the float64 logarithm of lambda (lambda != 0).
__device__ __forceinline__ double2 lam_pow_d(float2 lm, double k) {
  const double lr = (double)lm.x, li = (double)lm.y;
  const double lmag = 0.5 * log1p((lr * lr - 1.0) + li * li);
  double sn, cs;
  sincos(fmod(k * atan2(li, lr), 2.0 * M_PI), &sn, &cs);
  const double m = exp(k * lmag);
  return make_double2(m * cs, m * sn);
}
__device__ __forceinline__ float2 lam_pow64(float2 lm, double k) {
  const double2 z = lam_pow_d(lm, k);
  return make_float2((float)z.x, (float)z.y);
}

// Per-call constants of the fused form (float64 from the logarithm of lambda,
// rounded once): lp[p] = lambda^16, lambda^32, lambda^48, lambda^64 (the
// recurrence on a tile); apow[p][n] = lambda^(S n) for n < nseg (joining the
// segment states; lambda^0 = 1).
__global__ __launch_bounds__(256) void s5_fused_consts_kernel(const float2* __restrict__ lam,
                                                              int P, int nseg, double S,
                                                              float4* __restrict__ lp,
                                                              double2* __restrict__ apow) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long na = (long)P * nseg;
  if (i < na) {
    const int p = (int)(i / nseg), n = (int)(i % nseg);
    const float2 lm = lam[p];
    const bool nz = lm.x != 0.f || lm.y != 0.f;
    apow[i] = n == 0 ? make_double2(1.0, 0.0)
                     : (nz ? lam_pow_d(lm, S * (double)n) : make_double2(0.0, 0.0));
  } else if (i < na + P) {
    const int p = (int)(i - na);
    const float2 lm = lam[p];
    float2 l16 = make_float2(0.f, 0.f), l32 = l16, l48 = l16, l64 = l16;
    if (lm.x != 0.f || lm.y != 0.f) {
      l16 = lam_pow64(lm, 16.0);
      l32 = lam_pow64(lm, 32.0);
      l48 = lam_pow64(lm, 48.0);
      l64 = lam_pow64(lm, 64.0);
    }
    lp[2 * p] = make_float4(l16.x, l16.y, l32.x, l32.y);
    lp[2 * p + 1] = make_float4(l48.x, l48.y, l64.x, l64.y);
  }
}

// One dword per lane from a raw buffer into LDS at lds + 4 lane (zero where
// the lane's offset is past the buffer).  Issued from inline assembly so the
// compiler tracks no LDS write by it: every reader of that LDS is ordered by
// an explicit vmcnt(0) wait and a barrier.
__device__ __forceinline__ void dma_dword(BufRes rs, unsigned lds, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rs)
               : "memory");
}

// 16-byte chunk c (8 halves of k) of the staged operand's row `step`, swizzled
// so that a k step's matrix-core reads and the staging writes meet every LDS
// bank equally often.
__device__ __forceinline__ int sw_chunk(int step, int c) { return c ^ ((step >> 4) << 2); }
// Float index of u[k][j] within row k of the u tile (16-byte slots swizzled by k).
__device__ __forceinline__ int u_slot(int k, int j) { return (((j >> 2) ^ (k & 15)) << 2) | (j & 3); }

__device__ __forceinline__ int opaque_s(int x) {  // a scalar the optimiser recomputes at its use
  asm volatile("" : "+s"(x));
  return x;
}

#ifdef DSSM_PHASE_STAMPS
constexpr size_t kStateRows = 4096;  // stamp rows of the fused output pass before the state pass's
#endif

// KS: k steps (of 32) of both products, the fragments zero-padded to 32 KS;
// FI: 16-row tiles per wave of each product (2: 8 waves, 4: 4 waves)
template <bool STATE_ONLY, int KS, int FI>
__global__ __launch_bounds__(1024 / FI, 1) void s5_fused_kernel(const S5FusedArgs a) {
  constexpr int kFW = 16 / FI;  // waves (256 rows of each product)
  constexpr int kFI = FI;
  constexpr int kFR = 16 * FI;  // rows per wave
  constexpr int NS = FI / 2;    // states per lane
  PhaseClock pc;  // phase stamps (instrumented builds only): slots below
  __shared__ __attribute__((aligned(16))) _Float16 Sh[kFT][kBTS];  // staged operand, hi
  __shared__ __attribute__((aligned(16))) _Float16 Sl[kFT][kBTS];  // staged operand, lo
  __shared__ __attribute__((aligned(16))) float U[kRowsWG][kFT];   // u tile, fp32
  __shared__ float cmax[kFW][kFT];
  __shared__ __attribute__((aligned(16))) int cexp[kFT];
  __shared__ float2 cin_s[128];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int q = lane & 15, g = lane >> 4;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int H = a.H, P = a.P, L = a.L;
  const int M1 = 32 * ((P + 15) / 16), K1 = H, M2 = H;
  const int nt = (L + kFT - 1) / kFT;
  const int wg = blockIdx.x;
  const int b = wg / a.nseg, seg = wg % a.nseg;
  const int tile0 = seg * a.seg_tiles, tile1 = min(nt, tile0 + a.seg_tiles);
  if (STATE_ONLY && tile1 == nt) return;  // (whole workgroup) no later segment needs its state
  const int i0 = kFR * wu;                // this wave's first row (both products)
  const float* ub = a.u + (size_t)b * H * L;

  // this lane's states (rows of the input projection: it = 2 s Re, 2 s + 1 Im)
  int ps[NS];
  bool pin[NS];
  float2 lm[NS], l16[NS], l32[NS], l48[NS], l64[NS];
#pragma unroll
  for (int s2 = 0; s2 < NS; ++s2) {
    ps[s2] = 16 * (NS * wu + s2) + q;
    pin[s2] = ps[s2] < P;
    lm[s2] = l16[s2] = l32[s2] = l48[s2] = l64[s2] = make_float2(0.f, 0.f);
    if (pin[s2]) {
      lm[s2] = a.lam[ps[s2]];
      const float4 c0 = a.lp[2 * ps[s2]], c1 = a.lp[2 * ps[s2] + 1];
      l16[s2] = make_float2(c0.x, c0.y);
      l32[s2] = make_float2(c0.z, c0.w);
      l48[s2] = make_float2(c1.x, c1.y);
      l64[s2] = make_float2(c1.z, c1.w);
    }
  }
  // per-row scale exponents of this wave's rows of each product, D of its output rows
  int rx1[kFI], rx2[kFI];
  float dd[kFI];
#pragma unroll
  for (int it = 0; it < kFI; ++it) {
    const int i = i0 + 16 * it + q;
    rx1[it] = i0 < M1 ? a.rexp_in[min(i, M1 - 1)] : 0;
    rx2[it] = !STATE_ONLY && i0 < M2 ? a.rexp_out[min(i, M2 - 1)] : 0;
    dd[it] = !STATE_ONLY && i0 < M2 ? a.D[min(i, M2 - 1)] : 0.f;
  }

  // the state entering this segment (output pass):
  //   x_in(seg) = sum_{m < seg} lambda^(S (seg - 1 - m)) sout[m],
  // thread (state t / NP, part t % NP) sums a part of the terms in float64; its
  // first 16 terms are loaded before the first u tile (memory returns in order)
  constexpr int NP = kFW / 2;  // threads per state (128 states)
  const int cst = t / NP, cpart = t % NP;
  int cm0 = 0, cm1 = 0;
  float2 co[16];
  double2 cc[16];
  const float2* cso = a.sout + (size_t)b * a.nseg * P + cst;
  const double2* cap = a.apow + (size_t)cst * a.nseg + (seg - 1);
  auto carry_load = [&](int m) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int mm = min(m + e, cm1 - 1);  // in range; terms past cm1 zeroed below
      co[e] = cso[(size_t)mm * P];
      cc[e] = cap[-mm];
    }
  };
  double2 h = make_double2(0.0, 0.0);
  auto carry_add = [&](int m) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const double2 c = m + e < cm1 ? cc[e] : make_double2(0.0, 0.0);
      h = make_double2(fma(c.x, (double)co[e].x, fma(-c.y, (double)co[e].y, h.x)),
                       fma(c.x, (double)co[e].y, fma(c.y, (double)co[e].x, h.y)));
    }
  };
  const bool cany = !STATE_ONLY && cst < P && seg > 0;
  if (cany) {
    const int cs = (seg + NP - 1) / NP;
    cm0 = min(seg, cpart * cs);
    cm1 = min(seg, cm0 + cs);
    if (cm0 < cm1) carry_load(cm0);
  }

  // u tile jb into U: wave w fills rows k = w + W i, lane l dword l of the row
  // (the column whose slot is l / 4); columns past L take an offset beyond the
  // buffer (zero).  The batch row's u is one buffer (H L floats < 2^31 bytes).
  // Rows k = w + W i have k % 16 = w + W (i % FI): FI lane patterns.
  const BufRes ubuf = buf_res_uniform(ub, 4u * (unsigned)(H * L));
  int upat[FI];
#pragma unroll
  for (int r = 0; r < FI; ++r) upat[r] = (((lane >> 2) ^ (wu + kFW * r)) << 2) | (lane & 3);
  auto issue_u = [&](int jb) {
    int o[FI];
#pragma unroll
    for (int r = 0; r < FI; ++r) {
      const int j = jb * kFT + upat[r];
      o[r] = j < L ? 4 * j : INT_MIN;
    }
    int rowoff = opaque_s(4 * wu * L);  // 4 k L, a running scalar
    for (int k0 = wu; k0 < H; k0 += 16) {
#pragma unroll
      for (int r = 0; r < FI; ++r) {
        const int k = k0 + kFW * r;
        if (k < H) {
          // past L: a negative lane offset, beyond the buffer as unsigned (zero)
          dma_dword(ubuf, (unsigned)(size_t)&U[k][0], o[r] < 0 ? -1 : rowoff + o[r]);
        }
        rowoff += 4 * kFW * L;
      }
    }
  };
  issue_u(tile0);

  if (cany) {
    for (int m = cm0; m < cm1; m += 16) {
      if (m > cm0) carry_load(m);
      carry_add(m);
    }
  }
  if (!STATE_ONLY) {
#pragma unroll
    for (int o = 1; o < NP; o *= 2) {  // the parts (adjacent lanes)
      h.x += __shfl_xor(h.x, o, 64);
      h.y += __shfl_xor(h.y, o, 64);
    }
    if (cpart == 0) cin_s[cst] = make_float2((float)h.x, (float)h.y);
  }
  pc.mark(0);  // prologue: parameters, the entering state joined, first u tile requested

  // lane-derived indices, re-derived every tile from an opaque copy of the
  // lane id so that the compiler forms LDS addresses where they are used
  // instead of keeping dozens of them live across the tile loop
  int ln = lane, lq = q, lg = g, a4 = (lane & 15) >> 2;
  int brow = 16 * a4 + (lane & 3);  // staged row (step) of MFMA tile jt = 0 for this lane

  // out^T[step][i] = sum_k A[i][k] S[k][step] for this wave's 64 rows and the
  // tile's 64 steps: the fragments of A from L2 (one buffer, the wave's part in
  // the scalar offset); lane (q, g) gets rows 16 it + q at steps 16 g + 4 jt + r
  auto fragments = [&](const half8* __restrict__ apk, int M) {
    const unsigned frag_bytes = (unsigned)(((M + 63) / 64) * 4 * KS * 2 * 64 * 16);
    const BufRes fb = buf_res_uniform(apk, frag_bytes);
    const int tb = opaque_s(__builtin_amdgcn_readfirstlane((i0 / 16) * KS * 2 * 64 * 16));
    return [=](int it, int ks, int hl) {
      const int so = tb + (it * KS + ks) * 2048 + hl * 1024;
      const u32x4 r = __builtin_amdgcn_raw_buffer_load_b128(fb, 16 * lane, so, 0);
      return __builtin_bit_cast(half8, r);
    };
  };
  // the products of k step ks with the fragments (fh, fl) of the wave's row
  // tiles.  The staged operand is read one group of JG column tiles ahead of
  // the products that use it (LDS latency hidden behind the matrix cores); the
  // three split products of an accumulator are 2 JG kFI instructions apart (a
  // matrix-core result feeding the next product at once would stall).  Two
  // column tiles per group in both passes (the state-only pass with one: 8%
  // slower, the register need the same).
  constexpr int JG = 2;  // column tiles per group
  constexpr int NG = 4 / JG;                         // groups per k step
  typedef half8 BOp[2][JG];                          // [hi, lo][column tile]
  auto bread = [&](int gi, BOp& bo) {  // group gi = NG ks + j: its staged operands
    const int ks = gi / NG, j0 = JG * (gi % NG);
    // chunk 4 ks + g of the lane's staged row, swizzled: 4 (ks ^ a4) + g
    const int kc = 8 * (4 * (ks ^ a4) + lg);
#pragma unroll
    for (int j = 0; j < JG; ++j) {
      bo[0][j] = *reinterpret_cast<const half8*>(&Sh[brow + 4 * (j0 + j)][kc]);
      bo[1][j] = *reinterpret_cast<const half8*>(&Sl[brow + 4 * (j0 + j)][kc]);
    }
  };
  auto mgroup = [&](int gi, const BOp& bo, const half8 (&fh)[kFI], const half8 (&fl)[kFI],
                    v4f (&acc)[4][kFI]) {
    const int j0 = JG * (gi % NG);
#pragma unroll
    for (int j = 0; j < JG; ++j)
#pragma unroll
      for (int it = 0; it < kFI; ++it)
        acc[j0 + j][it] =
            __builtin_amdgcn_mfma_f32_16x16x32_f16(bo[0][j], fh[it], acc[j0 + j][it], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < JG; ++j)
#pragma unroll
      for (int it = 0; it < kFI; ++it)
        acc[j0 + j][it] =
            __builtin_amdgcn_mfma_f32_16x16x32_f16(bo[0][j], fl[it], acc[j0 + j][it], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < JG; ++j)
#pragma unroll
      for (int it = 0; it < kFI; ++it)
        acc[j0 + j][it] =
            __builtin_amdgcn_mfma_f32_16x16x32_f16(bo[1][j], fh[it], acc[j0 + j][it], 0, 0, 0);
  };
  // out^T over all k steps: fragment(ks) yields the fragments of k step ks
  // (loaded one k step ahead by the caller, or held in registers)
  auto gemm = [&](v4f (&acc)[4][kFI], auto&& kstep_begin, auto&& frags_of) {
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int it = 0; it < kFI; ++it) acc[jt][it] = v4f{0.f, 0.f, 0.f, 0.f};
    BOp bo[2];
    bread(0, bo[0]);
#pragma unroll
    for (int gi = 0; gi < KS * NG; ++gi) {
      if (gi % NG == 0) {
        __builtin_amdgcn_sched_barrier(0);  // one k step's operands (and the next's loads) live at a time
        kstep_begin(gi / NG);
      }
      if (gi + 1 < KS * NG) bread(gi + 1, bo[(gi + 1) & 1]);
      const auto& fr = frags_of(gi / NG);
      mgroup(gi, bo[gi & 1], fr.h, fr.l, acc);
    }
  };
  struct Frags {
    half8 h[kFI], l[kFI];
  };
  // Memory loads retire in order: a wait for a fragment also waits for every
  // memory access issued before it, so the next u tile is issued once the
  // product's last fragment loads are (after_loads).
  auto product = [&](const half8* __restrict__ apk, int M, v4f (&acc)[4][kFI],
                     auto&& after_loads) {
    const auto frag = fragments(apk, M);
    Frags fb[2];  // one k step ahead of its products
#pragma unroll
    for (int it = 0; it < kFI; ++it) {
      fb[0].h[it] = frag(it, 0, 0);
      fb[0].l[it] = frag(it, 0, 1);
    }
    gemm(acc,
         [&](int ks) {
           if (ks + 1 < KS) {
#pragma unroll
             for (int it = 0; it < kFI; ++it) {
               fb[(ks + 1) & 1].h[it] = frag(it, ks + 1, 0);
               fb[(ks + 1) & 1].l[it] = frag(it, ks + 1, 1);
             }
             if (ks + 2 == KS) after_loads();
           }
         },
         [&](int ks) -> const Frags& { return fb[ks & 1]; });
  };
  // the state-only pass keeps the input projection's fragments in registers
  // (loaded once): its products wait for no memory
  Frags rf[STATE_ONLY ? KS : 1];
  if (STATE_ONLY && i0 < M1) {
    const auto frag = fragments(a.apk_in, M1);
#pragma unroll
    for (int ks = 0; ks < (STATE_ONLY ? KS : 1); ++ks)
#pragma unroll
      for (int it = 0; it < kFI; ++it) {
        rf[ks].h[it] = frag(it, ks, 0);
        rf[ks].l[it] = frag(it, ks, 1);
      }
  }

  float2 carry[NS];  // the states entering the tile
#pragma unroll
  for (int s2 = 0; s2 < NS; ++s2) carry[s2] = make_float2(0.f, 0.f);
  for (int jb = tile0; jb < tile1; ++jb) {
    ln = opaque(lane);
    lq = ln & 15;
    lg = ln >> 4;
    a4 = lq >> 2;
    brow = 16 * a4 + (lq & 3);
    if (STATE_ONLY || jb == tile0) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's part of the u tile is in LDS
      __syncthreads();
      if (!STATE_ONLY && jb == tile0) {
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2)
          if (pin[s2]) carry[s2] = cin_s[ps[s2]];
      }
    }
    pc.mark(1);  // u tile in LDS (first tile; every tile of the state-only pass), barrier
    // 1. u into the staged operand: thread (step = lane, wave w) takes rows
    //    k = 8 (w + W qq) + e, scaled per step
    {
      float uv[2 * FI][8];
      float mx = 0.f;
#pragma unroll
      for (int qq = 0; qq < 2 * FI; ++qq)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int k = 8 * (wu + kFW * qq) + e;
          uv[qq][e] = k < K1 ? U[k][u_slot(k, ln)] : 0.f;
          mx = fmaxf(mx, fabsf(uv[qq][e]));
        }
      cmax[wu][ln] = mx;
      __syncthreads();
      float cm = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kFW; ++w2) cm = fmaxf(cm, cmax[w2][ln]);
      const int sc = scale_exp(cm);
      if (wu == 0) cexp[ln] = sc;
#pragma unroll
      for (int qq = 0; qq < 2 * FI; ++qq) {
        half8 hi, lo;
        split8(uv[qq], hi, lo, sc);
        const int c = sw_chunk(ln, wu + kFW * qq);
        *reinterpret_cast<half8*>(&Sh[ln][8 * c]) = hi;
        *reinterpret_cast<half8*>(&Sl[ln][8 * c]) = lo;
      }
    }
    // D u of this lane's output positions (rows 16 it + q, steps 16 g + 4 jt ..)
    v4f du[kFI][4];
    if (!STATE_ONLY) {
#pragma unroll
      for (int it = 0; it < kFI; ++it)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          const int i = i0 + 16 * it + lq;  // i % 16 == q
          du[it][jt] = i < M2 ? dd[it] * *reinterpret_cast<const v4f*>(&U[i][4 * ((4 * lg + jt) ^ lq)])
                              : v4f{0.f, 0.f, 0.f, 0.f};
        }
    }
    __syncthreads();  // the staged u and its exponents are complete; U may be refilled
    pc.mark(2);  // u scaled, split and staged, D u (two barriers)
    const bool more = jb + 1 < tile1;
    if (STATE_ONLY && more) issue_u(jb + 1);

    // 2. v = Bbar u, then the recurrence on the tile (two states per lane)
    float2 xs[NS][16];
    if (i0 < M1) {
      v4f acc[4][kFI];
      if (STATE_ONLY) {
        gemm(acc, [](int) {}, [&](int ks) -> const Frags& { return rf[STATE_ONLY ? ks : 0]; });
      } else {
        product(a.apk_in, M1, acc, [&] {
          if (more) issue_u(jb + 1);
        });
      }
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const int4 ce = *reinterpret_cast<const int4*>(&cexp[16 * lg + 4 * jt]);
        const int cr[4] = {ce.x, ce.y, ce.z, ce.w};
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            xs[s2][4 * jt + r] =
                make_float2(__builtin_amdgcn_ldexpf(acc[jt][2 * s2][r], -(rx1[2 * s2] + cr[r])),
                            __builtin_amdgcn_ldexpf(acc[jt][2 * s2 + 1][r], -(rx1[2 * s2 + 1] + cr[r])));
      }
    } else {
      if (!STATE_ONLY && more) issue_u(jb + 1);
    }
    pc.mark(3);  // input projection v = Bbar u (matrix cores), next u tile requested
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2)  // states past P (and waves past the rows) carry zero
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (!pin[s2] || i0 >= M1) xs[s2][j] = make_float2(0.f, 0.f);
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) {
      float2 x = make_float2(0.f, 0.f);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        x = cmad(lm[s2], x, xs[s2][j]);
        xs[s2][j] = x;
      }
      // the quarters' states from zero: lanes q + 16 k hold quarter k of this state
      float2 e4[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        e4[k] = make_float2(__shfl(x.x, lq + 16 * k, 64), __shfl(x.y, lq + 16 * k, 64));
      const float2 c0 = carry[s2];
      float2 ent = c0;  // state entering this lane's quarter
      if (lg == 1) ent = cmad(l16[s2], c0, e4[0]);
      if (lg == 2) ent = cmad(l32[s2], c0, cmad(l16[s2], e4[0], e4[1]));
      if (lg == 3) ent = cmad(l48[s2], c0, cmad(l32[s2], e4[0], cmad(l16[s2], e4[1], e4[2])));
      carry[s2] = cmad(l64[s2], c0,
                       cmad(l48[s2], e4[0], cmad(l32[s2], e4[1], cmad(l16[s2], e4[2], e4[3]))));
      if (!STATE_ONLY) {
        float2 pw = lm[s2];  // lambda^(j + 1)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          xs[s2][j] = cmad(pw, ent, xs[s2][j]);
          pw = cmad(pw, lm[s2], make_float2(0.f, 0.f));
        }
      }
    }
    pc.mark(4);  // recurrence on the tile
    if (STATE_ONLY) continue;  // the next tile's first barrier orders the reads of the staged u

    // 3. x as the output product's operand: rows k = 2p (Re), 2p + 1 (Im), one
    //    scale per step from the largest magnitude over all rows
    {
      float m16[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float m = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2) m = fmaxf(m, fmaxf(fabsf(xs[s2][j].x), fabsf(xs[s2][j].y)));
        m16[j] = row_max16(m);
      }
      float mine = m16[0];
#pragma unroll
      for (int j = 1; j < 16; ++j) mine = lq == j ? m16[j] : mine;
      cmax[wu][16 * lg + lq] = mine;  // this wave's maximum at step 16 g + q
    }
    __syncthreads();  // the maxima are complete; every wave is past its reads of the staged u
    int sc16[16];
    {
      float cm = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kFW; ++w2) cm = fmaxf(cm, cmax[w2][16 * lg + lq]);
      const int scm = scale_exp(cm);
#pragma unroll
      for (int j = 0; j < 16; ++j) sc16[j] = __shfl(scm, 16 * lg + j, 64);
    }
    if (i0 < M1) {
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) {
        const int c = 4 * (NS * wu + s2) + (lq >> 2);  // chunk of k = 2p
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int step = 16 * lg + j;
          _Float16 hr, lr, hi_, li;
          split16(__builtin_amdgcn_ldexpf(xs[s2][j].x, sc16[j]), hr, lr);
          split16(__builtin_amdgcn_ldexpf(xs[s2][j].y, sc16[j]), hi_, li);
          const int o = 8 * sw_chunk(step, c) + 2 * (lq & 3);
          half2v vh, vl;
          vh[0] = hr;
          vh[1] = hi_;
          vl[0] = lr;
          vl[1] = li;
          *reinterpret_cast<half2v*>(&Sh[step][o]) = vh;
          *reinterpret_cast<half2v*>(&Sl[step][o]) = vl;
        }
      }
    }
    pc.mark(5);  // x: per-step maximum (barrier), scaled, split and staged
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next u tile is in LDS
    __syncthreads();                     // the staged x is complete (and the next u tile)
    pc.mark(6);  // next u tile in LDS, barrier

    // 4. y = Re(C x) + D u
    if (i0 < M2) {
      v4f acc[4][kFI];
      product(a.apk_out, M2, acc, [] {});
      const bool vec = (L & 3) == 0;
#pragma unroll
      for (int it = 0; it < kFI; ++it) {
        const int i = i0 + 16 * it + lq;
        if (i >= M2) continue;
        float* orow = a.y + ((size_t)b * H + i) * L;
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          const int jj = jb * kFT + 16 * lg + 4 * jt;
          v4f o;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            o[r] = __builtin_amdgcn_ldexpf(acc[jt][it][r], -(rx2[it] + sc16[4 * jt + r])) +
                   du[it][jt][r];
          if (vec && jj + 3 < L) {
            *reinterpret_cast<v4f*>(orow + jj) = o;
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (jj + r < L) orow[jj + r] = o[r];
          }
        }
      }
    }
    pc.mark(7);  // output projection y = Re(C x) + D u (matrix cores), stores issued
  }
  // the state leaving a segment that is not the last (all its tiles are full)
  if (STATE_ONLY && g == 0) {
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2)
      if (pin[s2]) a.sout[((size_t)b * a.nseg + seg) * P + ps[s2]] = carry[s2];
  }
#ifdef DSSM_PHASE_STAMPS
  // (the state-only pass writes its stamps past the output pass's: rows from
  // kStateRows on, so one forward leaves both)
  if (STATE_ONLY && g_phase_buf && (threadIdx.x & 63) == 0) {
    const size_t base = (kStateRows + (size_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) *
                        kPhaseSlots;
    for (int k = 0; k < kPhaseSlots; ++k) g_phase_buf[base + k] = pc.acc[k];
  } else {
    pc.write();
  }
#else
  pc.write();
#endif
}

}  // namespace

S5Layout s5_layout(int B, int H, int P, int L, S5Form form) {
  S5Layout l;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  // split fragments: 16-row tiles x 32-deep k steps x (hi, lo) x 64 lanes x 16 B;
  // whole 64-row groups, as a wave of the contraction reads four tiles (tiles
  // past the rows are read, never written, and their products never stored)
  auto frag_bytes = [](int M, int K) {
    return (size_t)((M + 63) / 64) * 4 * ((K + 31) / 32) * 2 * 64 * sizeof(half8);
  };
  // the fused form pads both products to the same k steps and may have up to
  // 32 ceil(P / 16) rows of Bbar (whole 64-row groups)
  const bool fused = form == kS5Fused;
  const int kf = fused ? 32 * s5_fused_ks(H, P) : 0;
  l.apk_in = take(frag_bytes(2 * P, fused ? kf : H));
  l.rexp_in = take((size_t)((2 * P + 63) / 64) * 64 * sizeof(int));
  l.apk_out = take(frag_bytes(H, fused ? kf : 2 * P));
  l.rexp_out = take((size_t)((H + 15) / 16) * 16 * sizeof(int));
  if (fused) {
    // the fused form keeps v and x on chip: only the segment states
    const S5FusedPlan f = s5_fused_plan(B, L);
    l.sout = take((size_t)B * f.nseg * P * sizeof(float2));
    l.fconst = take((size_t)P * (2 * sizeof(float4) + f.nseg * sizeof(double2)));
  } else {
    l.v = take((size_t)B * P * 2 * L * sizeof(float));
    l.x = take((size_t)B * P * 2 * L * sizeof(float));
    if (form == kS5Conv) l.spec = take((size_t)P * 2 * ((size_t)1 << fft_log2m(L)) * sizeof(float2));
  }
  l.total = off;
  return l;
}

hipError_t launch_s5_pack(const float* Bbar, const float* C, int H, int P, void* apk_in,
                          int* rexp_in, void* apk_out, int* rexp_out, hipStream_t st, KEvents ev,
                          bool fused) {
  // (fused: whole 64-row groups, as a wave of the fused form reads four row tiles)
  const int m_in = fused ? 64 * ((32 * ((P + 15) / 16) + 63) / 64) : 2 * P;
  const int tiles = (std::max(m_in, H) + 15) / 16;
  const int kpad = fused ? s5_fused_ks(H, P) : 0;  // both kinds padded to the same k steps
  const int kmax = std::max(std::max(2 * P, H), 32 * kpad);
  if (kmax <= kPackLdsK) {
    const int groups = ((kmax + 31) / 32 + kPackKS - 1) / kPackKS;
    launch_k(s5_pack_lds_kernel, dim3((unsigned)tiles, 2, (unsigned)groups), dim3(256), st, ev,
             reinterpret_cast<const float2*>(Bbar), reinterpret_cast<const float2*>(C), H, P,
             static_cast<half8*>(apk_in), rexp_in, static_cast<half8*>(apk_out), rexp_out,
             fused ? 1 : 0, kpad);
    return hipGetLastError();
  }
  launch_k(s5_pack_kernel, dim3((unsigned)tiles, 2), dim3(256), st, ev,
           reinterpret_cast<const float2*>(Bbar), reinterpret_cast<const float2*>(C), H, P,
           static_cast<half8*>(apk_in), rexp_in, static_cast<half8*>(apk_out), rexp_out,
           fused ? 1 : 0, kpad);
  return hipGetLastError();
}

namespace {
int cu_count() {
  static int n = 0;
  if (!n) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}

template <bool kAddDu>
void launch_gemm(const void* apk, const int* rexp, const float* Bm, int M, int K, int L, int B,
                 const float* D, const float* u, float* out, hipStream_t st, KEvents ev) {
  const half8* a = static_cast<const half8*>(apk);
  const int nrb = (M + kRowsWG - 1) / kRowsWG;
  if (K <= kKC) {
    // one persistent workgroup per CU (per row block), walking the column tiles
    const long ntiles = (long)B * ((L + kColsWG - 1) / kColsWG);
    const long per = std::max(1, cu_count() / nrb);
    const dim3 grid((unsigned)std::min(ntiles, per), (unsigned)nrb);
    // (16-byte tile loads need L % 4 == 0 and a batch row's K x L floats under 2 GB)
    if ((L & 3) == 0 && (size_t)4 * K * L < ((size_t)1 << 31))
      launch_k(s5_gemm_pipe_kernel<kAddDu, true>, grid, dim3(64 * kPW), st, ev, a, rexp, Bm, M, K,
               L, B, D, u, out);
    else
      launch_k(s5_gemm_pipe_kernel<kAddDu, false>, grid, dim3(64 * kPW), st, ev, a, rexp, Bm, M, K,
               L, B, D, u, out);
    return;
  }
  const dim3 grid((unsigned)((L + kColsWG - 1) / kColsWG), (unsigned)nrb, (unsigned)B);
  launch_k(s5_gemm_kernel<kAddDu, true>, grid, dim3(256), st, ev, a, rexp, Bm, M, K, L, D, u, out);
}
}  // namespace

hipError_t launch_s5_proj_in(const void* apk_in, const int* rexp_in, const float* u, int B, int H,
                             int P, int L, float* v, hipStream_t st, KEvents ev) {
  launch_gemm<false>(apk_in, rexp_in, u, 2 * P, H, L, B, nullptr, nullptr, v, st, ev);
  return hipGetLastError();
}

hipError_t launch_s5_scan(const float* lambda, const float* v, int B, int P, int L, float* x,
                          hipStream_t st, KEvents ev) {
  launch_k(s5_scan_kernel, dim3((unsigned)(B * P)), dim3(kLanes), st, ev,
           reinterpret_cast<const float2*>(lambda), v, P, L, x);
  return hipGetLastError();
}

hipError_t launch_s5_scan_tv(const float* lam_c, const float* delta, const float* step,
                            const float* v, int B, int P, int L, float* x, hipStream_t st,
                            KEvents ev) {
  launch_k(s5_scan_tv_kernel, dim3((unsigned)(B * P)), dim3(kLanes), st, ev,
           reinterpret_cast<const float2*>(lam_c), delta, step, v, P, L, x);
  return hipGetLastError();
}

bool s5_fused_supported(int H, int P, int L) {
  // a batch row's u within one buffer of 32-bit byte offsets
  return P <= 128 && H <= kRowsWG && (long)H * L <= (1L << 29);
}

int s5_fused_ks(int H, int P) {
  const int ks = (std::max(H, 2 * P) + 31) / 32;
  return ks <= 2 ? 2 : ks <= 4 ? 4 : 8;
}

S5FusedPlan s5_fused_plan(int B, int L) {
  S5FusedPlan f;
  const int nt = (L + kFT - 1) / kFT;
  // one workgroup per CU: about 256 segments over the batch rows
  const int want = std::max(1, (256 + B - 1) / B);
  f.seg_tiles = std::max(1, (nt + want - 1) / want);
  f.nseg = (nt + f.seg_tiles - 1) / f.seg_tiles;
  return f;
}

hipError_t launch_s5_fused(const void* apk_in, const int* rexp_in, const void* apk_out,
                           const int* rexp_out, const float* lambda, const float* D,
                           const float* u, int B, int H, int P, int L, float* y, float2* sout,
                           void* consts, hipStream_t st, KEvents ev_consts, KEvents ev_state,
                           KEvents ev_out) {
  const S5FusedPlan f = s5_fused_plan(B, L);
  float4* lp = static_cast<float4*>(consts);
  double2* apow = reinterpret_cast<double2*>(lp + 2 * (size_t)P);
  {
    const long n = (long)P * f.nseg + P;
    launch_k(s5_fused_consts_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), st, ev_consts,
             reinterpret_cast<const float2*>(lambda), P, f.nseg, (double)f.seg_tiles * kFT, lp,
             apow);
  }
  S5FusedArgs a{};
  a.lp = lp;
  a.apow = apow;
  a.apk_in = static_cast<const half8*>(apk_in);
  a.rexp_in = rexp_in;
  a.apk_out = static_cast<const half8*>(apk_out);
  a.rexp_out = rexp_out;
  a.u = u;
  a.lam = reinterpret_cast<const float2*>(lambda);
  a.D = D;
  a.y = y;
  a.sout = sout;
  a.B = B;
  a.H = H;
  a.P = P;
  a.L = L;
  a.nseg = f.nseg;
  a.seg_tiles = f.seg_tiles;
  // 8 waves of 32 rows (the state-only pass with its input fragments in registers)
  const dim3 grid((unsigned)(B * f.nseg));
  const int ks = s5_fused_ks(H, P);
  auto kern = [&](bool state_only) {
    if (ks == 2) return state_only ? s5_fused_kernel<true, 2, 2> : s5_fused_kernel<false, 2, 2>;
    if (ks == 4) return state_only ? s5_fused_kernel<true, 4, 2> : s5_fused_kernel<false, 4, 2>;
    return state_only ? s5_fused_kernel<true, 8, 2> : s5_fused_kernel<false, 8, 2>;
  };
  if (f.nseg > 1) {
    launch_k(kern(true), grid, dim3(512), st, ev_state, a);
  } else {
    // one segment: no state to carry (the pass's events are stamped back to back)
    if (ev_state.start) (void)hipEventRecord(ev_state.start, st);
    if (ev_state.stop) (void)hipEventRecord(ev_state.stop, st);
  }
  launch_k(kern(false), grid, dim3(512), st, ev_out, a);
  return hipGetLastError();
}

hipError_t launch_s5_proj_out(const void* apk_out, const int* rexp_out, const float* x,
                              const float* D, const float* u, int B, int H, int P, int L, float* y,
                              hipStream_t st, KEvents ev) {
  launch_gemm<true>(apk_out, rexp_out, x, H, 2 * P, L, B, D, u, y, st, ev);
  return hipGetLastError();
}

}  // namespace dssm

#ifdef DSSM_PHASE_STAMPS
// Buffer for the fused S5 kernel's phase stamps (instrumented builds only).
extern "C" int dssm_phase_stamps_s5(void* buf) {
  return (int)hipMemcpyToSymbol(HIP_SYMBOL(dssm::g_phase_buf), &buf, sizeof(buf));
}
#endif
