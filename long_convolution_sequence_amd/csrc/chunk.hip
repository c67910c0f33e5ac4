// Chunked state-space form of the DLR bank on the matrix cores.
//
// What is computed: the same map as the recurrence ("The Annotated S4",
// Part 1, "Discrete-time SSM: the recurrent representation", with the DLR of
// "Simplifying and Understanding State Space Models with Diagonal Linear
// RNNs", section 2):
//   x_k = lambda x_{k-1} + u_k (x_{-1} = 0),  y_k = Re(sum_n W_n x_{k,n}) + D u_k,
// organised by chunks of T = 64 steps.  With S_c the state entering chunk c
// and t = cT + i:
//   s_c     = sum_{j<T} lambda^(T-1-j) u_{cT+j}                (chunk's own state)
//   S_{c+1} = lambda^T S_c + s_c                                (chunk recurrence)
//   y_t     = sum_{j<=i} K_{i-j} u_{cT+j} + D u_t + Re sum_n W_n lambda_n^(i+1) S_{c,n}
// with K_j = Re sum_n W_n lambda_n^j the DLR kernel (section 2: the convolution
// and recurrence views of the same map; within a chunk the convolution is a
// T x T Toeplitz product, across chunks the recurrence carries the state).
// The bidirectional form adds the same computation on the time-reversed input
// with the second parameter set, reversed back (section 2, bidirectional
// paragraph).
//
// How (MI355X design):
// * s = A1 U and y = A3 [U; S] are dense contractions per channel
//   (A1: 2N x T = 128 x 64, A3: T x (T + 2N) = 64 x 192, U: T x chunks) done on
//   the matrix cores with v_mfma_f32_16x16x32_f16 on split float32 operands
//   (fp16 hi + lo, three products, float32 accumulation; each operand group
//   scaled by an exact power of two first).
// * One workgroup (4 waves) runs one (channel, batch row).  Its prologue forms
//   the operands from the exactly promoted parameters (lambda, its powers and
//   the taps in float64, rounded once) and splits them into the MFMA fragments
//   each wave keeps in registers, while the first block's input is in flight.
//   Then blocks of 64 chunks: u to LDS (split), GEMM1 -> chunk states, the
//   chunk recurrence (a wave per quarter of the block, a lane per mode;
//   quarters combined with lambda^(16T)), GEMM3 -> y.  The next block's input
//   is requested before the current block is computed.
#include <algorithm>

#include "dssm_internal.h"
#include "mfma_split.h"

namespace dssm {
namespace {

using namespace mx;

constexpr int kT = 64;            // steps per chunk
constexpr int kCB = 64;           // chunks per block
constexpr int kModes = 64;        // modes handled (N <= 64; padded with zero modes)
constexpr int kR = 2 * kModes;    // state rows (re, im interleaved)

// Workgroup i runs on XCD i % 8; when the grid divides by 8, consecutive
// logical workgroups (the batch rows of one channel) share an XCD.
__device__ __forceinline__ int xcd_grouped(int i, int n) {
  return (n % 8 == 0) ? (i % 8) * (n / 8) + i / 8 : i;
}

__device__ __forceinline__ float2 cfma(float2 m, float2 p, float2 acc) {  // acc + m p
  return make_float2(fmaf(m.x, p.x, fmaf(-m.y, p.y, acc.x)), fmaf(m.x, p.y, fmaf(m.y, p.x, acc.y)));
}

// LDS row strides chosen so the 16-byte fragment reads of 16 consecutive
// columns fall in different banks.  The chunk states S1[c] (float32) and the
// carried states S[c] (fp16 hi at byte 0, lo at byte 272 of the same 528-byte
// row) share row c: one wave reads all its rows' S1 values into registers
// before it writes their S, and no other wave touches those rows in between.
constexpr int kUS = kT + 8;          // U[c][j] fp16
constexpr int kS1S = kR + 4;         // S1[c][r] fp32 (528-byte rows)
constexpr int kSRow = kS1S * 4;      // bytes per chunk row
constexpr int kSLo = 272;            // byte offset of the lo half within a row

// LDS: the operand tables of the prologue and the block arrays of the main
// loop are alive at different times and share one buffer.  Row strides and
// plane offsets are padded so each table's accesses below are free of bank
// conflicts.
constexpr int kQS = kModes + 2;            // Q row stride (float2)
constexpr int kKS = kT + 1;                // KR row stride (double)
constexpr int kPS = kT + 4;                // power-plane row stride (float)
constexpr int kPlane = kModes * kPS + 32;  // Im plane starts 32 banks after Re
struct TablesLds {
  float2 Q[kT][kQS];  // Q[i][n] = (Re, -Im) of W_n lambda_n^(i+1)
  union {
    double KR[kModes][kKS];  // Re(W_n lambda_n^p), p < T (the taps' terms)
    float PP[2 * kPlane];    // planes Re, Im of lambda_n^p: [plane * kPlane + n * kPS + p]
  };
  double2 lam[kModes], wv[kModes];
  float ktp[2 * kT];  // ktp[T + m] = K_m (+ D_f + D_b at m = 0 of d = 0); 0 for m < 0
  float4 mult[kModes];  // lambda^T, lambda^(16T)
  float red[8];         // per-wave largest |Q| (0..3) and |K_m| (4..7)
};
struct BlockLds {
  _Float16 Uh[kCB * kUS], Ul[kCB * kUS];
  float S1[kCB * kS1S];
  float2 E[4][kModes];
  int eU[kCB];  // scale exponent of each chunk's input (U rows)
  int eS[4];    // scale exponent of the carried states of each quarter
  float2 Xl[kModes];  // the state entering the sequence's last chunk (end-state capture)
};
constexpr int kLdsBytes = sizeof(TablesLds) > sizeof(BlockLds) ? sizeof(TablesLds) : sizeof(BlockLds);

// Operand fragments of wave w for direction d of channel h:
//   a1[(rt * 2 + ks) * 2 + hl]: A1 rows r = 32 w + 16 rt + lane % 16, columns
//     j = 32 ks + 8 (lane / 16) + e: A1[2n][j] = Re lambda_n^(T-1-j),
//     A1[2n+1][j] = Im lambda_n^(T-1-j)
//   a3[ks * 2 + hl]: A3 row i = 16 w + lane % 16, columns k = 32 ks + 8 (lane / 16) + e:
//     k < T: Toeplitz K_{i-k} (k <= i), with D_f + D_b on the diagonal (d = 0);
//     k = T + 2n: Re(W_n lambda_n^(i+1)), k = T + 2n + 1: -Im(W_n lambda_n^(i+1))
//     with the Toeplitz columns scaled by 2^eT and the others by 2^eW (each
//     part's largest magnitude brought to [2^14, 2^15))
// and the chunk multipliers lambda^T, lambda^(16T) of mode `lane`.  lambda, its
// powers (chains of 16 products from lambda^(16 q), q < 4), W lambda^p and the
// taps K_m = Re sum_n W_n lambda_n^m are float64, each rounded once to float32.
// Modes n >= N are zero.  Ends with a barrier (the LDS is reused after it).
// Parameters of mode `lane` of direction d, channel h (wave 0 only; zero for
// n >= N and the other waves) and the feed-through D_f + D_b (the first
// direction's tap 0), read by the caller before anything it leaves in flight:
// vector memory operations complete in issue order, so the prologue's first
// wait would otherwise also wait for them.
struct ModeParams {
  float re, im;
  float2 w;
  float d0, d1;  // D of each direction (workgroup-uniform: scalar loads)
};

__device__ __forceinline__ ModeParams load_mode_params(
    const float* __restrict__ log_re, const float* __restrict__ log_im,
    const float2* __restrict__ W, const float* __restrict__ D, int ndir, int H, int N, int d,
    int h) {
  const int t = threadIdx.x, lane = t & 63;
  ModeParams mp{0.f, 0.f, make_float2(0.f, 0.f), 0.f, 0.f};
  if (t < 64 && lane < N) {
    const size_t i = ((size_t)d * H + h) * N + lane;
    mp.re = log_re[i];
    mp.im = log_im[i];
    mp.w = W[i];
  }
  if (d == 0) {
    mp.d0 = D[h];
    if (ndir == 2) mp.d1 = D[(size_t)H + h];
  }
  return mp;
}

// Marks the mode parameters as arriving here: the caller places it after
// the loads it leaves in flight, so nothing derived from the parameters is
// computed (and waited for) before those loads are issued.
__device__ __forceinline__ void params_here(ModeParams& mp) {
  asm volatile("" : "+v"(mp.re), "+v"(mp.im), "+v"(mp.w.x), "+v"(mp.w.y));
}

__device__ __forceinline__ void build_operands(const ModeParams& mp, int N, int d, TablesLds& tl,
                                               half8* a1, half8* a3, float2& lamT,
                                               float2& lam16T, int& eT, int& eW, PhaseClock& pc) {
  const int t = opaque(threadIdx.x), lane = t & 63, w = t >> 6;
  pc.mark(11);
  if (w == 0) {  // lambda_n, W_n (float64, from the exactly promoted parameters)
    const int n = lane;
    double2 lam = make_double2(0.0, 0.0), wv = lam;
    if (n < N) {
      const double re = (double)mp.re;
      double sn, cs;
      sincos((double)mp.im, &sn, &cs);
      const double m = exp(-re * re);
      lam = make_double2(m * cs, m * sn);
      wv = make_double2((double)mp.w.x, (double)mp.w.y);
    }
    tl.lam[n] = lam;
    tl.wv[n] = wv;
  }
  __syncthreads();
  pc.mark(12);
  float2 pw[16];  // lambda^p of this thread's 16 powers, kept for the planes
  float qm = 0.f;  // largest |Q| entry written by this thread
  {  // mode n = lane, powers p = 16 w .. 16 w + 15
    const int n = lane;
    const double2 lam = tl.lam[n], wv = tl.wv[n];
    double2 x = make_double2(n < N ? 1.0 : 0.0, 0.0), b = lam;  // lambda^(16 w)
    for (int e = 16 * w; e; e >>= 1) {
      if (e & 1) x = zmul(x, b);
      b = zmul(b, b);
    }
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int p = 16 * w + s;
      pw[s] = make_float2((float)x.x, (float)x.y);
      tl.KR[n][p] = wv.x * x.x - wv.y * x.y;
      x = zmul(x, lam);
      const double2 q = zmul(wv, x);
      const float2 qf = make_float2((float)q.x, (float)-q.y);
      tl.Q[p][n] = qf;
      qm = fmaxf(qm, fmaxf(fabsf(qf.x), fabsf(qf.y)));
    }
    if (w == 3) {  // x = lambda^T
      double2 b16 = zmul(x, x);
      b16 = zmul(b16, b16);
      b16 = zmul(b16, b16);
      b16 = zmul(b16, b16);
      tl.mult[n] = make_float4((float)x.x, (float)x.y, (float)b16.x, (float)b16.y);
    }
  }
  qm = wave_max(qm);
  if (lane == 0) tl.red[w] = qm;
  __syncthreads();
  pc.mark(13);
  {  // taps: wave w sums taps 16 w .. +15, a quarter of the modes per 16 lanes
    const int m = 16 * w + (lane & 15), q = lane >> 4;
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < 16; ++k) s += tl.KR[16 * q + k][m];
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    if (t == 0 && d == 0) s += (double)mp.d0 + (double)mp.d1;  // (m = 0: lane 0 of wave 0)
    const float kv = (float)s;
    if (q == 0) tl.ktp[kT + m] = kv;
    if (q == 1) tl.ktp[m] = 0.f;
    const float km = row_max16(q == 0 ? fabsf(kv) : 0.f);  // lanes 0..15 hold the taps
    if (lane == 0) tl.red[4 + w] = km;
  }
  __syncthreads();  // KR read: its space takes the power planes
  pc.mark(14);
  eW = scale_exp(fmaxf(fmaxf(tl.red[0], tl.red[1]), fmaxf(tl.red[2], tl.red[3])));
  eT = scale_exp(fmaxf(fmaxf(tl.red[4], tl.red[5]), fmaxf(tl.red[6], tl.red[7])));
  {
    float* pr = tl.PP + lane * kPS + 16 * w;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      *reinterpret_cast<f4*>(pr + 4 * s4) =
          f4{pw[4 * s4].x, pw[4 * s4 + 1].x, pw[4 * s4 + 2].x, pw[4 * s4 + 3].x};
      *reinterpret_cast<f4*>(pr + kPlane + 4 * s4) =
          f4{pw[4 * s4].y, pw[4 * s4 + 1].y, pw[4 * s4 + 2].y, pw[4 * s4 + 3].y};
    }
  }
  __syncthreads();
  pc.mark(15);
  const int g = lane >> 4;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int r = 32 * w + 16 * rt + (lane & 15);
    const float* row = tl.PP + (r & 1) * kPlane + (r >> 1) * kPS;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      // columns j = 32 ks + 8 g + e hold powers T - 1 - j = p0 + 7 - e
      f4 lo4, hi4;
      lds_read8(row + (kT - 8 - 32 * ks - 8 * g), lo4, hi4);
      const float v[8] = {hi4[3], hi4[2], hi4[1], hi4[0], lo4[3], lo4[2], lo4[1], lo4[0]};
      split8(v, a1[(rt * 2 + ks) * 2], a1[(rt * 2 + ks) * 2 + 1]);
      __builtin_amdgcn_sched_barrier(0);  // one fragment's temporaries live at a time
    }
  }
  const int i = 16 * w + (lane & 15);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {  // Toeplitz: K_{i-k} at ktp[T + i - k]
    const float* kt = tl.ktp + kT + i - 32 * ks - 8 * g;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = kt[-e];
    split8(v, a3[ks * 2], a3[ks * 2 + 1], eT);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int ks = 2; ks < 6; ++ks) {  // modes 16 (ks - 2) + 4 g .. + 3 at power i + 1
    f4 lo4, hi4;
    lds_read8(reinterpret_cast<const float*>(&tl.Q[i][16 * (ks - 2) + 4 * g]), lo4, hi4);
    const float v[8] = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
    split8(v, a3[ks * 2], a3[ks * 2 + 1], eW);
    __builtin_amdgcn_sched_barrier(0);
  }
  const float4 m = tl.mult[lane];
  lamT = make_float2(m.x, m.y);
  lam16T = make_float2(m.z, m.w);
  __syncthreads();
}

// What one launch of the chunked kernel does (all pointers device memory):
//   directions d in [dir0, dir0 + ndir_wg), each in its own time order
//   (d = 1: reversed time t' = Lp - 1 - t, Lp = chunks x T); with dir_in_grid
//   one direction per workgroup, dir0 + the workgroup's place in the grid
//   divided by H x row groups x segments (state-only passes only: they write
//   no outputs two directions could race on);
//   workgroup = (channel h, group of rpw batch rows, segment s), segments of
//   seg_blocks blocks of processing time;
//   the state entering the segment: x0 [B,H,N] (one direction, segment 0),
//   or cin [ndir][B][H][nseg][N], or zero;
//   outputs: y stored (add = 0, first direction of the workgroup) or added
//   (add = 1, and every later direction); none when state_only;
//   sout [ndir][B][H][nseg][N]: the state leaving each segment (state_only);
//   xend [B,H,N]: the state after step L - 1 (one direction).
struct ChunkArgs {
  const float* u;
  const float* log_re;
  const float* log_im;
  const float2* W;
  const float* D;
  float* y;
  const float2* x0;
  float2* xend;
  const float2* cin;
  float2* sout;
  int B, H, N, L, ndir;
  int dir0, ndir_wg, rpw, nseg, seg_blocks;
  int add, state_only;
  int dir_in_grid;  // the workgroup's one direction is dir0 + its grid position / (H groups segments)
};

// float64 lambda of mode n of direction d, channel h (zero for n >= N).
__device__ __forceinline__ double2 lambda64(const ChunkArgs& a, int d, int h, int n) {
  if (n >= a.N) return make_double2(0.0, 0.0);
  const size_t i = ((size_t)d * a.H + h) * a.N + n;
  const double re = (double)a.log_re[i];
  double sn, cs;
  sincos((double)a.log_im[i], &sn, &cs);
  const double m = exp(-re * re);
  return make_double2(m * cs, m * sn);
}

template <bool VEC, bool STATE_ONLY, bool CAPTURE, int RP = 1>
__global__ __launch_bounds__(256, 2) void chunk_kernel(const ChunkArgs a) {
  static_assert(RP == 1 || RP == 2 || RP == 4, "rows per block");
  static_assert(RP == 1 || (!STATE_ONLY && !CAPTURE), "rows share a block only without state");
  PhaseClock pc;  // phase stamps (instrumented builds only): slots below
  __shared__ __attribute__((aligned(16))) unsigned char lds_raw[kLdsBytes];
  TablesLds& tl = *reinterpret_cast<TablesLds*>(lds_raw);
  BlockLds& bl = *reinterpret_cast<BlockLds*>(lds_raw);
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int B = a.B, H = a.H, L = a.L;
  const int ngrp = (B + a.rpw - 1) / a.rpw;
  const int wg_all = xcd_grouped(blockIdx.x, gridDim.x);
  const int per_dir = H * ngrp * a.nseg;
  const int wg = a.dir_in_grid ? wg_all % per_dir : wg_all;
  const int dir0 = a.dir0 + (a.dir_in_grid ? wg_all / per_dir : 0);
  const int seg = wg % a.nseg;
  const int h = (wg / a.nseg) / ngrp, grp = (wg / a.nseg) % ngrp;
  const int b0 = grp * a.rpw, b1 = min(B, b0 + a.rpw);
  const int nchunk = (L + kT - 1) / kT;
  const int nblk = (nchunk + kCB - 1) / kCB;
  const int blk0 = seg * a.seg_blocks, blk1 = min(nblk, blk0 + a.seg_blocks);
  const int Lp = nchunk * kT;  // padded length (reversed-time origin)
  const int cl = nchunk - 1;   // the last chunk (holds step L - 1)
  const bool last_seg = blk1 == nblk;
  if (STATE_ONLY && last_seg) return;  // (whole workgroup) no later segment needs its state
  unsigned char* srow = reinterpret_cast<unsigned char*>(bl.S1);
  // RP > 1: rows of one block each (at most 64 / RP chunks; the launch
  // guarantees it, and no state in or out) share a block, row slot k taking
  // chunks k CR .. k CR + CR - 1 (CR = 64 / RP: a quarter or a half of the
  // block, i.e. the chunks of one or two waves' recurrence), their chunk
  // chains kept apart.
  constexpr int R = RP;
  constexpr int lgR = RP == 4 ? 2 : RP == 2 ? 1 : 0;
  constexpr int lgER = 12 - lgR;  // log2 of the elements per row slot (kCB kT / R)
  constexpr int lgCR = 6 - lgR;   // log2 of the chunks per row slot

  for (int dd = 0; dd < a.ndir_wg; ++dd) {
    const int d = dir0 + dd;
    const bool rev = d == 1;
    const bool add = a.add || dd > 0;
    // element e of block blk in processing time -> sequence position within
    // its row (out of range, hence zero on load and dropped on store, beyond
    // the sequence); the row is slot e >> lgER of the block's row group
    auto pos = [&](int blk, int e) {
      const int q = blk * kCB * kT + (e & ((1 << lgER) - 1));
      return rev ? Lp - 1 - q : q;
    };
    // a row of the group starting at row bg, as a buffer (empty beyond the
    // group's nv valid rows: zeros on load, stores dropped)
    auto row_buf = [&](const float* base, int bg, int k, int nv) {
      const bool valid = k < nv;
      return buf_res(base + ((size_t)(valid ? bg + k : 0) * H + h) * L,
                     valid ? 4u * (unsigned)L : 0u);
    };
    // input of block blk of the row group at bg: thread t takes elements
    // 4 t + 1024 q + c4 (c4 < 4, q < 4), each group q in one row slot
    auto load_block = [&](int bg, int blk, float* v, int nv) {
      if (VEC) {  // reversed: the four elements sit at descending positions, kept
                  // in memory order here (one load path for both directions, and no
                  // register permutation that would wait for the load); the
                  // staging reads them reversed
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const BufRes ub = row_buf(a.u, bg, (1024 * q) >> lgER, nv);
          const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(
              ub, 4 * pos(blk, 4 * t + 1024 * q + (rev ? 3 : 0)), 0, 0);
          v[4 * q + 0] = __uint_as_float(x.x);
          v[4 * q + 1] = __uint_as_float(x.y);
          v[4 * q + 2] = __uint_as_float(x.z);
          v[4 * q + 3] = __uint_as_float(x.w);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const BufRes ub = row_buf(a.u, bg, (1024 * (q >> 2)) >> lgER, nv);
          const int e = 4 * t + 1024 * (q >> 2) + (q & 3);
          v[q] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ub, 4 * pos(blk, e), 0, 0));
        }
      }
    };
    // element c4 of group q is un[4 q + c4], or un[4 q + 3 - c4] for a reversed
    // 16-byte load
    const bool swap4 = VEC && rev;
    ModeParams mp = load_mode_params(a.log_re, a.log_im, a.W, a.D, a.ndir, H, a.N, d, h);
    float un[16];
    load_block(b0, blk0, un, min(R, b1 - b0));  // in flight while the operands are formed
    params_here(mp);
    half8 a1[8], a3[12];
    float2 lamT, lam16T;
    int eT, eW;
    build_operands(mp, a.N, d, tl, a1, a3, lamT, lam16T, eT, eW, pc);

    for (int b = b0; b < b1; b += R) {
      const size_t row = (size_t)b * H + h;
      const int nv = min(R, b1 - b);  // rows of this group
      // (four named buffers, selected below: no array indexed at run time)
      const BufRes yb0 = row_buf(a.y, b, 0, nv), yb1 = row_buf(a.y, b, 1, nv),
                   yb2 = row_buf(a.y, b, 2, nv), yb3 = row_buf(a.y, b, 3, nv);
      // the state entering the segment, mode = lane (every wave keeps it)
      float2 carry = make_float2(0.f, 0.f);
      if (lane < a.N) {
        if (a.cin)
          carry = a.cin[((((size_t)d * B + b) * H + h) * a.nseg + seg) * a.N + lane];
        else if (a.x0 && seg == 0)
          carry = a.x0[row * a.N + lane];
      }

      pc.mark(0);  // prologue's end: operand fragments, barrier, the entering state
      for (int blk = blk0; blk < blk1; ++blk) {
        __syncthreads();  // the previous block's readers of U and S are done
        pc.mark(1);
        // 1. input to LDS, split: element e = 4 t + 1024 q + c4 -> chunk e / 64, step e % 64;
        //    the 16 lanes of a DPP row hold one chunk, scaled by 2^eU[chunk]
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int e = 4 * t + 1024 * q;
          const int c = e >> 6, j = e & 63;
          const int sc = scale_exp(row_max16(amax4(un + 4 * q)));
          if ((lane & 15) == 0) bl.eU[c] = sc;
          half4 vh, vl;
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4) {
            _Float16 p, r;
            split16(__builtin_amdgcn_ldexpf(un[4 * q + (swap4 ? 3 - c4 : c4)], sc), p, r);
            vh[c4] = p;
            vl[c4] = r;
          }
          *reinterpret_cast<half4*>(bl.Uh + c * kUS + j) = vh;
          *reinterpret_cast<half4*>(bl.Ul + c * kUS + j) = vl;
        }
        __builtin_amdgcn_sched_barrier(0);
        // in flight during this block: the next block of this row, or the
        // first block of the next row (zeros beyond the sequence or the rows)
        {
          const bool same = blk + 1 < blk1;
          load_block(same ? b : b + R, same ? blk + 1 : blk0, un,
                     same ? nv : min(R, b1 - (b + R)));
        }
        __builtin_amdgcn_sched_barrier(0);
        pc.mark(2);  // input staged, next block requested
        __syncthreads();
        pc.mark(3);
        // 2. chunk states: S1[c][r] = sum_j A1[r][j] U[j][c]; this wave: rows 32 w .. +31,
        //    in two halves of 32 columns (fewer accumulators live).  The output
        //    product's U part (the Toeplitz taps, rows 16 w .. +15) takes the same U
        //    fragments here: U is read from LDS once for both products.  Not in the
        //    streaming form: its end-state capture leaves no room for the 16
        //    accumulators held across the recurrence (they would spill to scratch)
        constexpr bool kFuseU = !CAPTURE;
        f4 accU[2][2];  // [column half][column tile]
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
          f4 acc[2][2];
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) acc[rt][ct] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            __builtin_amdgcn_sched_barrier(0);  // one k step's operands live at a time
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
              const int c = 32 * ch + 16 * ct + (lane & 15);
              const int k = 32 * ks + 8 * (lane >> 4);
              const half8 bh = *reinterpret_cast<const half8*>(bl.Uh + c * kUS + k);
              const half8 blo = *reinterpret_cast<const half8*>(bl.Ul + c * kUS + k);
#pragma unroll
              for (int rt = 0; rt < 2; ++rt) {
                const half8 ah = a1[(rt * 2 + ks) * 2], al = a1[(rt * 2 + ks) * 2 + 1];
                acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh, acc[rt][ct], 0, 0, 0);
                acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, blo, acc[rt][ct], 0, 0, 0);
                acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bh, acc[rt][ct], 0, 0, 0);
              }
              if (!STATE_ONLY && kFuseU) {
                f4& au = accU[ch][ct];
                if (ks == 0) au = f4{0.f, 0.f, 0.f, 0.f};
                const half8 th = a3[ks * 2], tlo = a3[ks * 2 + 1];
                au = __builtin_amdgcn_mfma_f32_16x16x32_f16(th, bh, au, 0, 0, 0);
                au = __builtin_amdgcn_mfma_f32_16x16x32_f16(th, blo, au, 0, 0, 0);
                au = __builtin_amdgcn_mfma_f32_16x16x32_f16(tlo, bh, au, 0, 0, 0);
              }
            }
          }
          // acc[rt][ct][v]: row r = 32 w + 16 rt + 4 (lane / 16) + v, column c = 32 ch + 16 ct + lane % 16
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
              const int c = 32 * ch + 16 * ct + (lane & 15);
              const int r = 32 * w + 16 * rt + 4 * (lane >> 4);
              *reinterpret_cast<f4*>(bl.S1 + c * kS1S + r) = acc[rt][ct];
            }
        }
        pc.mark(4);  // chunk states (matrix cores)
        __syncthreads();
        pc.mark(5);
        // 3. chunk recurrence: wave w takes chunks 16 w .. 16 w + 15, lane = mode.  The
        //    wave reads its rows' S1 values before it writes S over them.
        {
          const int n = lane;
          float2 sv[16];
#pragma unroll
          for (int c = 0; c < 16; ++c) {  // chunk states, unscaled (S1 carries 2^eU)
            const float2 v = *reinterpret_cast<const float2*>(bl.S1 + (16 * w + c) * kS1S + 2 * n);
            const int ec = -bl.eU[16 * w + c];
            sv[c] = make_float2(__builtin_amdgcn_ldexpf(v.x, ec), __builtin_amdgcn_ldexpf(v.y, ec));
          }
          float2 e = make_float2(0.f, 0.f);
#pragma unroll
          for (int c = 0; c < 16; ++c) e = cfma(lamT, e, sv[c]);
          bl.E[w][n] = e;
          pc.mark(6);  // recurrence, first part
          __syncthreads();
          pc.mark(7);
          float2 cin = carry;  // state entering quarter w (from its row slot's first quarter)
          for (int q = w & ~((4 >> lgR) - 1); q < w; ++q) cin = cfma(lam16T, cin, bl.E[q][n]);
          float2 cnext = carry;  // state leaving the block (every wave keeps it)
#pragma unroll
          for (int q = 0; q < 4; ++q) cnext = cfma(lam16T, cnext, bl.E[q][n]);
          carry = cnext;
          float2 st = cin;
          float m = 0.f;
#pragma unroll
          for (int c = 0; c < 16; ++c) {  // sv[c] becomes the state entering chunk 16 w + c
            const float2 nx = cfma(lamT, st, sv[c]);
            sv[c] = st;
            m = fmaxf(m, fmaxf(fabsf(st.x), fabsf(st.y)));
            st = nx;
          }
          // for the end state: the state entering the sequence's last chunk or,
          // when L is a whole number of chunks, the state leaving it (the end
          // state itself: the entering state of the next chunk, or st after the
          // quarter's last)
          if (CAPTURE && last_seg) {
            const int cloc = cl - blk * kCB - 16 * w;
            if (cloc >= 0 && cloc < 16) {
              const bool whole = (L % kT) == 0;
              const int ce = whole ? cloc + 1 : cloc;
              float2 s0 = st;
#pragma unroll
              for (int c = 0; c < 16; ++c)
                if (c == ce) s0 = sv[c];
              bl.Xl[n] = s0;
            }
          }
          const int es = scale_exp(wave_max(m));  // one exponent for the quarter's states
          if (lane == 0) bl.eS[w] = es;
#pragma unroll
          for (int c = 0; c < 16; ++c) {
            half2v hi, lo;
            _Float16 p, r;
            split16(__builtin_amdgcn_ldexpf(sv[c].x, es), p, r);
            hi[0] = p;
            lo[0] = r;
            split16(__builtin_amdgcn_ldexpf(sv[c].y, es), p, r);
            hi[1] = p;
            lo[1] = r;
            unsigned char* rw = srow + (16 * w + c) * kSRow;
            *reinterpret_cast<half2v*>(rw + 4 * n) = hi;
            *reinterpret_cast<half2v*>(rw + kSLo + 4 * n) = lo;
          }
        }
        pc.mark(8);  // recurrence, second part (states scaled, split, stored)
        if (STATE_ONLY) continue;  // the segment's end state is all this pass needs
        __syncthreads();
        pc.mark(9);
        // 4. outputs: Y[i][c] = sum_k A3[i][k] [U; S][k][c]; this wave: rows 16 w .. +15,
        //    in two halves of 32 columns.  The U part (k < T) and the S part are
        //    accumulated apart: each carries its own scale.
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
          f4 accS[2], accUo[2];
          accS[0] = accS[1] = f4{0.f, 0.f, 0.f, 0.f};
          if constexpr (kFuseU) {
#pragma unroll
            for (int ks = 2; ks < 6; ++ks) {  // (the U part, k < T: formed with the chunk states)
              __builtin_amdgcn_sched_barrier(0);  // one k step's operands live at a time
              const half8 ah = a3[ks * 2], al = a3[ks * 2 + 1];
#pragma unroll
              for (int ct = 0; ct < 2; ++ct) {
                const int c = 32 * ch + 16 * ct + (lane & 15);
                const int k = 32 * (ks - 2) + 8 * (lane >> 4);
                const unsigned char* rw = srow + c * kSRow;
                const half8 bh = *reinterpret_cast<const half8*>(rw + 2 * k);
                const half8 blo = *reinterpret_cast<const half8*>(rw + kSLo + 2 * k);
                f4& acc = accS[ct];
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, blo, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bh, acc, 0, 0, 0);
              }
            }
          } else {
            accUo[0] = accUo[1] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 6; ++ks) {  // the U part (k < T), then the S part
              __builtin_amdgcn_sched_barrier(0);
              const half8 ah = a3[ks * 2], al = a3[ks * 2 + 1];
#pragma unroll
              for (int ct = 0; ct < 2; ++ct) {
                const int c = 32 * ch + 16 * ct + (lane & 15);
                half8 bh, blo;
                if (ks < 2) {
                  const int k = 32 * ks + 8 * (lane >> 4);
                  bh = *reinterpret_cast<const half8*>(bl.Uh + c * kUS + k);
                  blo = *reinterpret_cast<const half8*>(bl.Ul + c * kUS + k);
                } else {
                  const int k = 32 * (ks - 2) + 8 * (lane >> 4);
                  const unsigned char* rw = srow + c * kSRow;
                  bh = *reinterpret_cast<const half8*>(rw + 2 * k);
                  blo = *reinterpret_cast<const half8*>(rw + kSLo + 2 * k);
                }
                f4& acc = ks < 2 ? accUo[ct] : accS[ct];
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, blo, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bh, acc, 0, 0, 0);
              }
            }
          }
          // acc*[ct][v]: step i = 16 w + 4 (lane / 16) + v of chunk c = 32 ch + 16 ct + lane % 16
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            const int c = 32 * ch + 16 * ct + (lane & 15);
            // processing time within the chunk's row (slot (32 ch + 16 ct) >> lgCR)
            const int e0 = (blk * kCB + (c & ((1 << lgCR) - 1))) * kT + 16 * w + 4 * (lane >> 4);
            const int slot = (32 * ch + 16 * ct) >> lgCR;
            const BufRes ybuf = slot == 0 ? yb0 : slot == 1 ? yb1 : slot == 2 ? yb2 : yb3;
            const int xu = -(eT + bl.eU[c]), xs = -(eW + bl.eS[c >> 4]);
            f4 acc;
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4)
              acc[v4] = __builtin_amdgcn_ldexpf(kFuseU ? accU[ch][ct][v4] : accUo[ct][v4], xu) +
                        __builtin_amdgcn_ldexpf(accS[ct][v4], xs);
            if (VEC) {
              // four consecutive processing times: one 16-byte group (ascending
              // positions forward, descending reversed; 16-byte aligned as L % 4 == 0)
              const int p0 = rev ? Lp - 4 - e0 : e0;
              f4 o = rev ? f4{acc[3], acc[2], acc[1], acc[0]} : acc;
              if (add) {
                // added to the earlier direction's output (read past the L1, which
                // may hold lines from before this workgroup's own stores)
                const u32x4 old = __builtin_amdgcn_raw_buffer_load_b128(ybuf, 4 * p0, 0, 1);
                o += f4{__uint_as_float(old.x), __uint_as_float(old.y), __uint_as_float(old.z),
                        __uint_as_float(old.w)};
              }
              u32x4 ov;
              ov.x = __float_as_uint(o[0]);
              ov.y = __float_as_uint(o[1]);
              ov.z = __float_as_uint(o[2]);
              ov.w = __float_as_uint(o[3]);
              __builtin_amdgcn_raw_buffer_store_b128(ov, ybuf, 4 * p0, 0, 0);
            } else {
#pragma unroll
              for (int v4 = 0; v4 < 4; ++v4) {
                const int p = rev ? Lp - 1 - (e0 + v4) : e0 + v4;
                float o = acc[v4];
                if (add)
                  o += __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ybuf, 4 * p, 0, 1));
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o), ybuf, 4 * p, 0, 0);
              }
            }
          }
        }
        pc.mark(10);  // outputs (matrix cores), stored
      }
      // the state leaving a segment that is not the last (all its chunks are real)
      if (a.sout && !last_seg && w == 0 && lane < a.N)
        a.sout[((((size_t)d * B + b) * H + h) * a.nseg + seg) * a.N + lane] = carry;
      // the state after step L - 1: from the state entering the last chunk and
      // that chunk's first L - 64 cl inputs (still in LDS: the row's last block
      // holds the last chunk), advanced in float64 by one wave, lane = mode
      if (CAPTURE && last_seg) {
        __syncthreads();  // Xl written by the wave that held the last chunk
        if (w == 0 && (L % kT) == 0) {  // Xl is the state after step L - 1
          if (lane < a.N) a.xend[row * a.N + lane] = bl.Xl[lane];
        } else if (w == 0) {  // a partial last chunk: its real steps from Xl, in float64
          const int c = cl - (nblk - 1) * kCB;  // the last chunk's index in its block
          const double2 lam = lambda64(a, d, h, lane);
          const float2 s0 = bl.Xl[lane];
          double2 x = make_double2((double)s0.x, (double)s0.y);
          const float inv = __builtin_amdgcn_ldexpf(1.f, -bl.eU[c]);
          for (int j = 0; j < L - kT * cl; ++j) {
            const float uj = ((float)bl.Uh[c * kUS + j] + (float)bl.Ul[c * kUS + j]) * inv;
            x = make_double2(lam.x * x.x - lam.y * x.y + (double)uj, lam.x * x.y + lam.y * x.x);
          }
          if (lane < a.N) a.xend[row * a.N + lane] = make_float2((float)x.x, (float)x.y);
        }
      }
    }
    // this direction's stores are visible to the next one's sweep: both run in
    // this workgroup, whose vector memory operations stay in order on its CU
    // (the later direction reads y past the L1); a workgroup barrier orders
    // them, no agent-scope fence (an L2 write-back and invalidation) needed
    if (dd + 1 < a.ndir_wg) __syncthreads();
  }
  pc.write();
}

// The state entering each segment from the states the segments leave when
// started from zero (sout, a state-only pass's) and the caller's state x0
// (direction 0; zero without it):
//   cin[s] = A^s x0 + sum_{m < s} A^(s - 1 - m) sout[m],  A = lambda^S,
// S the steps of a segment, in float64, rounded once.  One workgroup per
// (direction, row, segment), lane = mode: wave w takes a quarter of the
// segments m < s by Horner's rule (the state leaving its last one from its
// terms alone), advanced by A^(s - its end) to the segment's start; the four
// partial states meet in LDS.  Every load is unconditional (buffers: lanes
// past N, and x0 when absent, read zero), so a wave's loads issue together.
// A is formed from the float64 logarithm, its powers A^k by squaring (at
// most 9 squarings for 512 segments: a relative error of a few hundred
// float64 ulp).
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ double2 zfma(double2 m, double2 x, double2 c) {  // m x + c
  return make_double2(fma(m.x, x.x, fma(-m.y, x.y, c.x)), fma(m.x, x.y, fma(m.y, x.x, c.y)));
}

__global__ __launch_bounds__(256) void chunk_join_kernel(const ChunkArgs a,
                                                         float2* __restrict__ cin) {
  __shared__ double2 part[256];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int seg = blockIdx.x % a.nseg;
  const int r = blockIdx.x / a.nseg;  // (d, b, h)
  const int h = r % a.H, b = (r / a.H) % a.B, d = r / (a.H * a.B);
  const bool live = lane < a.N;
  const size_t row = ((size_t)d * a.B + b) * a.H + h;
  const int lo = live ? 8 * lane : 1 << 30;  // (past every buffer: zero)
  auto load2 = [&](BufRes rs, int off) {
    const v2u v = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
    return make_float2(__uint_as_float(v.x), __uint_as_float(v.y));
  };
  const bool with_x0 = a.x0 && d == 0;
  const BufRes xr = buf_res_uniform(with_x0 ? a.x0 + ((size_t)b * a.H + h) * a.N : a.sout,
                                    with_x0 ? 8u * (unsigned)a.N : 0u);
  const float2 x0 = load2(xr, lo);
  float2* out = cin + (row * a.nseg + seg) * a.N;
  if (seg == 0) {  // (the whole workgroup)
    if (w == 0 && live) out[lane] = x0;
    return;
  }
  const BufRes sr = buf_res_uniform(a.sout + row * a.nseg * a.N, 8u * (unsigned)(a.nseg * a.N));
  const int q = (seg + 3) / 4;
  const int m0 = min(seg, w * q), m1 = min(seg, m0 + q);
  const size_t ip = ((size_t)d * a.H + h) * a.N + (live ? lane : 0);
  const float fre = a.log_re[ip], fim = a.log_im[ip];
  constexpr int kJ = 32;  // terms requested at once, in flight while A is formed
  float2 v[kJ];
#pragma unroll
  for (int e = 0; e < kJ; ++e) v[e] = load2(sr, lo + 8 * a.N * min(m0 + e, seg - 1));  // (past m1: unused)
  const double re = (double)fre, im = (double)fim;
  const double S = (double)a.seg_blocks * kCB * kT;
  double sn, cs;
  sincos(fmod(im * S, 2.0 * M_PI), &sn, &cs);  // (reduced exactly: the small-argument path)
  const double mag = exp(-re * re * S);
  const double2 A = make_double2(mag * cs, mag * sn);
  double2 F = make_double2(1.0, 0.0), p2 = A;
  for (int k = seg - m1; k; k >>= 1) {
    if (k & 1) F = zmul(F, p2);
    p2 = zmul(p2, p2);
  }
  double2 c = w == 0 ? make_double2((double)x0.x, (double)x0.y) : make_double2(0.0, 0.0);
  const int n0 = min(kJ, m1 - m0);  // (wave-uniform)
#pragma unroll
  for (int e = 0; e < kJ; ++e)
    if (e < n0) c = zfma(A, c, make_double2((double)v[e].x, (double)v[e].y));
  // (more than kJ segments per quarter, at most 512 segments: further groups)
  for (int m = m0 + kJ; m < m1; m += kJ) {
    float2 u[kJ];
#pragma unroll
    for (int e = 0; e < kJ; ++e) u[e] = load2(sr, lo + 8 * a.N * min(m + e, seg - 1));
    const int nm = min(kJ, m1 - m);
#pragma unroll
    for (int e = 0; e < kJ; ++e)
      if (e < nm) c = zfma(A, c, make_double2((double)u[e].x, (double)u[e].y));
  }
  part[t] = zmul(F, c);
  __syncthreads();
  if (w == 0) {
    double2 x = part[lane];
#pragma unroll
    for (int k = 1; k < 4; ++k)
      x = make_double2(x.x + part[64 * k + lane].x, x.y + part[64 * k + lane].y);
    if (live) out[lane] = make_float2((float)x.x, (float)x.y);
  }
}

void launch_chunk_args(const ChunkArgs& a, hipStream_t st, KEvents ev, int ndir_grid = 1) {
  const long nwg = (long)ndir_grid * a.H * ((a.B + a.rpw - 1) / a.rpw) * a.nseg;
  // 16-byte accesses need a length that a 16-byte access never straddles (rows
  // then also start 16-byte aligned)
  const dim3 g((unsigned)nwg), blk(256);
  const bool vec = (a.L % 4) == 0;
  if (a.state_only) {  // (no end state here)
    if (vec) launch_k(chunk_kernel<true, true, false>, g, blk, st, ev, a);
    else launch_k(chunk_kernel<false, true, false>, g, blk, st, ev, a);
  } else if (a.xend) {
    if (vec) launch_k(chunk_kernel<true, false, true>, g, blk, st, ev, a);
    else launch_k(chunk_kernel<false, false, true>, g, blk, st, ev, a);
  } else {
    // short stateless rows share blocks: 4 rows of at most 16 chunks, or 2 of
    // at most 32
    const int nchunk = (a.L + kT - 1) / kT;
    const int rp = (a.x0 || a.cin || a.nseg != 1) ? 1 : nchunk <= kCB / 4 ? 4 : nchunk <= kCB / 2 ? 2 : 1;
    if (rp == 4) {
      if (vec) launch_k(chunk_kernel<true, false, false, 4>, g, blk, st, ev, a);
      else launch_k(chunk_kernel<false, false, false, 4>, g, blk, st, ev, a);
    } else if (rp == 2) {
      if (vec) launch_k(chunk_kernel<true, false, false, 2>, g, blk, st, ev, a);
      else launch_k(chunk_kernel<false, false, false, 2>, g, blk, st, ev, a);
    } else {
      if (vec) launch_k(chunk_kernel<true, false, false>, g, blk, st, ev, a);
      else launch_k(chunk_kernel<false, false, false>, g, blk, st, ev, a);
    }
  }
}

}  // namespace

bool chunk_supported(int N) { return N >= 1 && N <= kModes; }

ChunkPlan chunk_plan(int B, int H, int L, int ndir) {
  ChunkPlan p;
  const int nchunk = (L + kT - 1) / kT;
  const int nblk = (nchunk + kCB - 1) / kCB;
  const long rows = (long)B * H;
  // enough workgroups for two per CU (the occupancy the kernel's registers
  // allow) on 256 CUs: several batch rows of a channel share one workgroup's
  // operands when rows are many; a long sequence is split into segments when
  // rows are few
  const long want = 512;
  p.rpw = (int)std::max(1L, std::min<long>(B, rows / want));
  p.nseg = 1;
  p.seg_blocks = nblk;
  // (each launch of a split runs one direction, or the directions side by side)
  if (rows < want && nblk > 1) {
    const long segs = std::min<long>(nblk, (want + rows - 1) / rows);
    p.seg_blocks = (int)((nblk + segs - 1) / segs);
    p.nseg = (nblk + p.seg_blocks - 1) / p.seg_blocks;
  }
  return p;
}

size_t chunk_workspace(int B, int H, int N, int L, int ndir) {
  const ChunkPlan p = chunk_plan(B, H, L, ndir);
  if (p.nseg == 1) return 0;
  // sout and cin
  return 2 * align_up((size_t)ndir * B * H * p.nseg * N * sizeof(float2), 256);
}

hipError_t launch_chunk(const float* u, const float* log_re, const float* log_im, const float* W,
                        const float* D, int B, int H, int N, int L, int ndir, float* y,
                        const float* x0, float* xend, void* ws, hipStream_t st, KEvents ev) {
  const ChunkPlan p = chunk_plan(B, H, L, ndir);
  ChunkArgs a{};
  a.u = u;
  a.log_re = log_re;
  a.log_im = log_im;
  a.W = reinterpret_cast<const float2*>(W);
  a.D = D;
  a.y = y;
  a.x0 = reinterpret_cast<const float2*>(x0);
  a.xend = reinterpret_cast<float2*>(xend);
  a.B = B;
  a.H = H;
  a.N = N;
  a.L = L;
  a.ndir = ndir;
  a.rpw = p.rpw;
  a.nseg = p.nseg;
  a.seg_blocks = p.seg_blocks;
  if (p.nseg == 1) {  // one pass over each row, every direction in one workgroup
    a.dir0 = 0;
    a.ndir_wg = ndir;
    launch_chunk_args(a, st, ev);
    return hipGetLastError();
  }
  // segments: (1) the state each segment leaves from zero, (2) the state each
  // one enters (a workgroup per segment joining the earlier ones' and x0),
  // (3) the outputs from those states, one direction per launch (the reversed
  // one adding into y)
  const size_t part = align_up((size_t)ndir * B * H * p.nseg * N * sizeof(float2), 256);
  float2* sout = static_cast<float2*>(ws);
  float2* cin = reinterpret_cast<float2*>(static_cast<char*>(ws) + part);
  const KEvents e_first{ev.start, nullptr}, e_last{nullptr, ev.stop};
  ChunkArgs s1 = a;
  s1.dir0 = 0;
  s1.ndir_wg = 1;
  s1.dir_in_grid = 1;  // the directions side by side (no outputs to share)
  s1.state_only = 1;
  s1.sout = sout;
  s1.x0 = nullptr;  // every segment from zero here; x0 enters through the join
  s1.xend = nullptr;
  launch_chunk_args(s1, st, e_first, ndir);
  ChunkArgs s2 = a;
  s2.sout = sout;
  launch_k(chunk_join_kernel, dim3((unsigned)((long)ndir * B * H * p.nseg)), dim3(256), st,
           KEvents{}, s2, cin);
  for (int d = 0; d < ndir; ++d) {
    ChunkArgs s3 = a;
    s3.dir0 = d;
    s3.ndir_wg = 1;
    s3.add = d > 0;
    s3.cin = cin;
    s3.x0 = nullptr;
    s3.xend = d == 0 ? a.xend : nullptr;
    launch_chunk_args(s3, st, d + 1 == ndir ? e_last : KEvents{});
  }
  return hipGetLastError();
}

}  // namespace dssm

#ifdef DSSM_PHASE_STAMPS
// Buffer for the chunked recurrence's phase stamps (instrumented builds only).
extern "C" int dssm_phase_stamps_chunk(void* buf) {
  return (int)hipMemcpyToSymbol(HIP_SYMBOL(dssm::g_phase_buf), &buf, sizeof(buf));
}
#endif
