// Causal long convolution of a DLR bank by FFT, staged in LDS.
//
// What is computed ("Simplifying and Understanding State Space Models with
// Diagonal Linear RNNs", section 2: the convolution y = K * u is a Toeplitz
// mat-vec, computed as a circulant mat-vec of size 2L on zero-padded
// operands; "The Annotated S4", Part 1, "Training SSMs: the convolutional
// representation": pad to twice the length, transform, multiply, invert,
// keep the first L samples):
//
//   y[b,h,:L] = ( IDFT_2M( DFT_2M(pad u[b,h]) * DFT_2M(pad Re K[h]) ) )[:L]
//               + D[h] u[b,h]
//
// with M = max(16, next power of two >= L), so 2M >= 2L and no wrap-around
// reaches the first L outputs.
//
// How (MI355X design):
// * Two batch rows of the same channel ride in one complex sequence
//   z = u[b1] + i u[b2].  The kernel spectrum is Hermitian and the product is
//   linear, so Re/Im of the inverse transform are the two real outputs; no
//   even/odd untangling step is needed.
// * The 2M-point transform of a sequence that is zero on its upper half splits
//   exactly into two M-point transforms: the even bins are DFT_M(z) and the
//   odd bins DFT_M(z * t) with t[n] = exp(-i pi n / M).  The inverse is the sum
//   of the two M-point inverses, the odd one multiplied by conj(t).  So a
//   workgroup only ever holds M complex points (<= 128 KiB + padding of LDS).
// * Each M-point transform is a sequence of in-place decimation-in-frequency
//   passes (radix 16, last pass radix 2/4/8/16) with 16 points per thread in
//   registers and one LDS exchange between passes.  The bins are left in the
//   passes' own (digit-reversed) order; the kernel spectrum is stored in the
//   same order, so the pointwise product happens in registers right after the
//   last forward pass and the inverse (decimation-in-time, the passes run
//   backwards with conjugate twiddles) starts from the same registers and ends
//   in natural order, ready for a coalesced store.
// * Twiddles: one table value exp(-2 pi i m / S) per thread and pass, powers by
//   a depth <= 5 product tree; the table (exact float32 roundings of float64
//   values) is built into the library.
#include <algorithm>
#include <type_traits>

#include "dssm_internal.h"
#include "twiddle_table.inc"

#define DSSM_FFT_CASES(X) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14)

namespace dssm {
namespace {

__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(fmaf(a.x, b.x, -a.y * b.y), fmaf(a.x, b.y, a.y * b.x));
}
__device__ __forceinline__ float2 cconj(float2 a) { return make_float2(a.x, -a.y); }
__device__ __forceinline__ float2 cscale(float2 a, float s) { return make_float2(a.x * s, a.y * s); }

// a * exp(-+ 2 pi i k / 16): forward (INV = false) multiplies by exp(-i theta),
// inverse by exp(+i theta), theta = 2 pi k / 16.  Exact for multiples of pi/2.
template <int K, bool INV>
__device__ __forceinline__ float2 rot16(float2 a) {
  constexpr int k = ((K % 16) + 16) % 16;
  constexpr float C1 = 0.92387953251128674f;  // cos(pi/8)
  constexpr float S1 = 0.38268343236508977f;  // sin(pi/8)
  constexpr float R = 0.70710678118654752f;   // sqrt(2)/2
  // (c, s) = (cos theta, sin theta)
  constexpr float cs[16][2] = {{1, 0},   {C1, S1},  {R, R},     {S1, C1},  {0, 1},   {-S1, C1},
                               {-R, R},  {-C1, S1}, {-1, 0},    {-C1, -S1}, {-R, -R}, {-S1, -C1},
                               {0, -1},  {S1, -C1}, {R, -R},    {C1, -S1}};
  constexpr float c = cs[k][0];
  constexpr float s = INV ? cs[k][1] : -cs[k][1];
  if constexpr (k == 0) {
    return a;
  } else if constexpr (k == 8) {
    return make_float2(-a.x, -a.y);
  } else if constexpr (k == 4 || k == 12) {
    // multiply by (0 + i s), s = +-1
    if constexpr (s > 0) return make_float2(-a.y, a.x);
    else return make_float2(a.y, -a.x);
  } else {
    return make_float2(fmaf(a.x, c, -a.y * s), fmaf(a.x, s, a.y * c));
  }
}

// cos and sin of pi k / 32 for 0 <= k <= 8 (the rest follow by symmetry).
__device__ constexpr float kCos32[9] = {1.0f, 0.99518472667219693f, 0.98078528040323043f,
                                        0.95694033573220882f, 0.92387953251128674f,
                                        0.88192126434835505f, 0.83146961230254524f,
                                        0.77301045336273699f, 0.70710678118654752f};
__device__ constexpr float kSin32[9] = {0.0f, 0.09801714032956060f, 0.19509032201612825f,
                                        0.29028467725446233f, 0.38268343236508978f,
                                        0.47139673682599764f, 0.55557023301960218f,
                                        0.63439328416364549f, 0.70710678118654752f};
constexpr float cos_pi32(int k) {  // cos(pi k / 32), 0 <= k < 32
  return k <= 8 ? kCos32[k] : k <= 16 ? kSin32[16 - k] : -cos_pi32(32 - k);
}
constexpr float sin_pi32(int k) {  // sin(pi k / 32), 0 <= k < 32
  return k <= 8 ? kSin32[k] : k <= 16 ? kCos32[16 - k] : sin_pi32(32 - k);
}

// a * exp(-+ i pi K / 32), K in [0, 32): the fixed part of the odd-bin
// pre-twiddle.  Exact for K = 0 and K = 16.
template <int K, bool INV>
__device__ __forceinline__ float2 rotpi32(float2 a) {
  static_assert(K >= 0 && K < 32, "rotpi32 index");
  if constexpr (K == 0) {
    return a;
  } else if constexpr (K == 16) {
    return INV ? make_float2(-a.y, a.x) : make_float2(a.y, -a.x);
  } else {
    constexpr float c = cos_pi32(K);
    constexpr float s = INV ? sin_pi32(K) : -sin_pi32(K);
    return make_float2(fmaf(a.x, c, -a.y * s), fmaf(a.x, s, a.y * c));
  }
}

// In-place DFT of 2, 4, 8 or 16 points held in registers (natural order in
// and out).  Forward kernel exp(-2 pi i n k / R); INV uses exp(+...).
template <bool INV>
__device__ __forceinline__ void dft2(float2& a, float2& b) {
  const float2 t = a;
  a = cadd(t, b);
  b = csub(t, b);
}

template <bool INV>
__device__ __forceinline__ void dft4(float2& a0, float2& a1, float2& a2, float2& a3) {
  const float2 t0 = cadd(a0, a2), t1 = csub(a0, a2), t2 = cadd(a1, a3), t3 = csub(a1, a3);
  a0 = cadd(t0, t2);
  a2 = csub(t0, t2);
  if (!INV) {  // t1 -+ i t3
    a1 = make_float2(t1.x + t3.y, t1.y - t3.x);
    a3 = make_float2(t1.x - t3.y, t1.y + t3.x);
  } else {
    a1 = make_float2(t1.x - t3.y, t1.y + t3.x);
    a3 = make_float2(t1.x + t3.y, t1.y - t3.x);
  }
}

// 8 points: n = 2 n1 + n2 (n1 < 4, n2 < 2), k = k1 + 4 k2.
template <bool INV>
__device__ __forceinline__ void dft8(float2* x) {
  float2 y0[4] = {x[0], x[2], x[4], x[6]};
  float2 y1[4] = {x[1], x[3], x[5], x[7]};
  dft4<INV>(y0[0], y0[1], y0[2], y0[3]);
  dft4<INV>(y1[0], y1[1], y1[2], y1[3]);
  y1[1] = rot16<2, INV>(y1[1]);
  y1[2] = rot16<4, INV>(y1[2]);
  y1[3] = rot16<6, INV>(y1[3]);
#pragma unroll
  for (int k1 = 0; k1 < 4; ++k1) {
    x[k1] = cadd(y0[k1], y1[k1]);
    x[k1 + 4] = csub(y0[k1], y1[k1]);
  }
}

// 16 points: n = 4 n1 + n2, k = k1 + 4 k2 (radix 4 x 4 with inner twiddles).
template <bool INV>
__device__ __forceinline__ void dft16(float2* x) {
  float2 y[4][4];  // y[n2][k1]
#pragma unroll
  for (int n2 = 0; n2 < 4; ++n2) {
    y[n2][0] = x[n2];
    y[n2][1] = x[4 + n2];
    y[n2][2] = x[8 + n2];
    y[n2][3] = x[12 + n2];
    dft4<INV>(y[n2][0], y[n2][1], y[n2][2], y[n2][3]);
  }
  y[1][1] = rot16<1, INV>(y[1][1]);
  y[1][2] = rot16<2, INV>(y[1][2]);
  y[1][3] = rot16<3, INV>(y[1][3]);
  y[2][1] = rot16<2, INV>(y[2][1]);
  y[2][2] = rot16<4, INV>(y[2][2]);
  y[2][3] = rot16<6, INV>(y[2][3]);
  y[3][1] = rot16<3, INV>(y[3][1]);
  y[3][2] = rot16<6, INV>(y[3][2]);
  y[3][3] = rot16<9, INV>(y[3][3]);
#pragma unroll
  for (int k1 = 0; k1 < 4; ++k1) {
    dft4<INV>(y[0][k1], y[1][k1], y[2][k1], y[3][k1]);
    x[k1] = y[0][k1];
    x[k1 + 4] = y[1][k1];
    x[k1 + 8] = y[2][k1];
    x[k1 + 12] = y[3][k1];
  }
}

template <int R, bool INV>
__device__ __forceinline__ void dftR(float2* x) {
  if constexpr (R == 16) {
    dft16<INV>(x);
  } else if constexpr (R == 8) {
    dft8<INV>(x);
  } else if constexpr (R == 4) {
    dft4<INV>(x[0], x[1], x[2], x[3]);
  } else {
    static_assert(R == 2, "radix");
    dft2<INV>(x[0], x[1]);
  }
}

// Powers p[q] = w^q, q = 1..15, by a product tree of depth <= 5.
__device__ __forceinline__ void powers16(float2 w, float2* p) {
  p[1] = w;
  p[2] = cmul(w, w);
  p[3] = cmul(p[2], w);
  p[4] = cmul(p[2], p[2]);
  p[8] = cmul(p[4], p[4]);
  p[12] = cmul(p[8], p[4]);
#pragma unroll
  for (int a = 4; a <= 12; a += 4)
#pragma unroll
    for (int b = 1; b < 4; ++b) p[a + b] = cmul(p[a], p[b]);
}

__device__ __forceinline__ float2 cmulc(float2 a, float2 b) {  // a * conj(b)
  return make_float2(fmaf(a.x, b.x, a.y * b.y), fmaf(a.y, b.x, -a.x * b.y));
}

// v[q] *= p[q] (or conj(p[q]) when CONJ), q = 1..15; with SHIFT also by the
// constant exp(-+ i pi q / 16) (the twiddle offset of a thread's second
// butterfly in the first pass).
template <bool CONJ, bool SHIFT, int Q = 1>
__device__ __forceinline__ void apply16(float2* v, const float2* p) {
  if constexpr (Q < 16) {
    float2 a = v[Q];
    if constexpr (SHIFT && CONJ) a = rotpi32<2 * Q, true>(a);
    a = CONJ ? cmulc(a, p[Q]) : cmul(a, p[Q]);
    if constexpr (SHIFT && !CONJ) a = rotpi32<2 * Q, false>(a);
    v[Q] = a;
    apply16<CONJ, SHIFT, Q + 1>(v, p);
  }
}

// Transform geometry.  M = 2^LOG2M points, PT points per thread (16 or 32),
// NB = PT / 16 radix-16 butterflies per thread, T = M / PT threads per
// transform.  Passes 0 .. NP-2 are radix 16 on sub-transforms of size
// S = M >> 4p (stride s = S / 16); the last pass has radix RLAST = M >> 4(NP-1).
template <int LOG2M, int PT_>
struct Cfg {
  static_assert(LOG2M >= 4 && LOG2M <= kMaxLog2M, "transform size");
  static_assert(PT_ == 16 || PT_ == 32, "points per thread");
  static constexpr int M = 1 << LOG2M;
  static constexpr int PT = PT_;
  static constexpr int NB = PT / 16;
  static constexpr int T = M / PT;
  static constexpr int NP = (LOG2M + 3) / 4;
  static constexpr int RLAST = 1 << (LOG2M - 4 * (NP - 1));
  static constexpr int G = T >= 64 ? 1 : 64 / T;  // transforms per workgroup
  static constexpr int WG = T * G;
  // LDS slot of position e: e + (e >> PADSH).  One pad slot per 16 (or 32)
  // points keeps every pass's access pattern at the minimum number of LDS
  // bank cycles for its lane stride.
  static constexpr int PADSH = (PT == 32) ? 5 : 4;
  static constexpr int LDSN = M + (M >> PADSH);   // padded complex slots
  static_assert(T >= 1 && (NB == 1 || NP >= 2), "shape");
  __device__ static __forceinline__ int pad(int e) { return e + (e >> PADSH); }
};

// Which positions thread lt's registers r = 16 i + j occupy in pass p (a pass
// reads and writes the same positions):
//   pass 0:        butterfly beta = lt + i T, element j at beta + j M/16
//   pass p >= 1:   butterfly (g, m) = (NB (lt / s) + i, lt % s), element j
//                  at g S + m + j s  -- a thread's NB butterflies share m,
//                  hence their twiddles
//   last pass:     positions PT lt + r.
// LDS slot = pad(position) = pad(base) + j s + (j s >> PADSH): s divides 2^PADSH
// or is a multiple of it, base is a multiple of S = 16 s plus m < s, so no
// carry crosses a pad boundary -- one base per butterfly, constant offsets.
// After pass 0 every sub-transform lies inside the positions owned by one wave
// (a wave owns the contiguous range [64 PT w, 64 PT (w + 1))), so only the
// exchange between passes 0 and 1 needs a workgroup barrier.
template <class C, int P>
struct PassGeom {
  static constexpr bool kLast = (P == C::NP - 1);
  static constexpr int S = kLast ? C::RLAST : (C::M >> (4 * P));
  static constexpr int s = kLast ? 1 : S / 16;
  __device__ static __forceinline__ int m_of(int lt) { return P == 0 ? lt : lt % s; }
  __device__ static __forceinline__ int base(int lt, int i) {
    if (P == 0) return lt + i * C::T;
    return (C::NB * (lt / s) + i) * S + (lt % s);
  }
  __device__ static constexpr int off(int j) { return j * s + ((j * s) >> C::PADSH); }
};

template <class C, int P>
__device__ __forceinline__ void lds_write(float2* lds, int lt, const float2* v) {
  using G = PassGeom<C, P>;
  if constexpr (G::kLast) {
    float2* b = lds + C::pad(C::PT * lt);
#pragma unroll
    for (int r = 0; r < C::PT; ++r) b[r + (r >> C::PADSH)] = v[r];
  } else {
#pragma unroll
    for (int i = 0; i < C::NB; ++i) {
      float2* b = lds + C::pad(G::base(lt, i));
#pragma unroll
      for (int j = 0; j < 16; ++j) b[G::off(j)] = v[16 * i + j];
    }
  }
}

template <class C, int P>
__device__ __forceinline__ void lds_read(const float2* lds, int lt, float2* v) {
  using G = PassGeom<C, P>;
  if constexpr (G::kLast) {
    const float2* b = lds + C::pad(C::PT * lt);
#pragma unroll
    for (int r = 0; r < C::PT; ++r) v[r] = b[r + (r >> C::PADSH)];
  } else {
#pragma unroll
    for (int i = 0; i < C::NB; ++i) {
      const float2* b = lds + C::pad(G::base(lt, i));
#pragma unroll
      for (int j = 0; j < 16; ++j) v[16 * i + j] = b[G::off(j)];
    }
  }
}

// The value of x, hidden from the optimiser (it cannot reuse values derived
// from x before this point).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Twiddle root of pass 0 for thread lt, w = exp(-2 pi i lt / M).  The index is
// opaque, so each use loads the root afresh instead of the compiler keeping it
// live across the kernel.
template <class C>
__device__ __forceinline__ float2 pass0_w(int lt) {
  using G = PassGeom<C, 0>;
  if constexpr (G::kLast) return make_float2(1.f, 0.f);
  else return g_twiddle[G::m_of(opaque(lt)) * (DSSM_TWN / G::S)];
}

// Powers of the pass-0 root (product tree); opaque, so they are recomputed
// per use and not kept live between uses.
template <class C>
__device__ __forceinline__ void pass0_powers(float2 w, float2* p) {
  if constexpr (!PassGeom<C, 0>::kLast) {
    asm volatile("" : "+v"(w.x), "+v"(w.y));
    powers16(w, p);
  }
}

// Twiddles of the wave-local radix-16 passes 1 .. NP-2, one LDS table per
// workgroup: entry off(P) + (q - 1) s + m = exp(-2 pi i m q / S) for q = 1..15,
// m < s (s = S / 16 <= 64), the exactly rounded table values.  A pass reads
// its 15 powers instead of forming them by a product tree.
template <class C>
struct TwTab {
  static constexpr int s_of(int P) { return C::M >> (4 * P + 4); }
  static constexpr int off(int P) {
    int o = 0;
    for (int q = 1; q < P; ++q) o += 15 * s_of(q);
    return o;
  }
  static constexpr int N = C::NP >= 3 ? off(C::NP - 1) : 0;  // entries
  static constexpr int kAlloc = N > 0 ? N : 1;
};

template <class C>
__device__ __forceinline__ void twtab_init(float2* tab) {
  using TT = TwTab<C>;
  for (int idx = threadIdx.x; idx < TT::N; idx += blockDim.x) {
    int P = 1;
    while (idx >= TT::off(P + 1)) ++P;
    const int sp = TT::s_of(P), rel = idx - TT::off(P);
    const int q = rel / sp + 1, m = rel % sp;
    tab[idx] = g_twiddle[m * q * (DSSM_TWN / (16 * sp))];  // m q < 16 sp = S
  }
}

// Powers of pass P >= 1 for thread lt, from the table.
template <class C, int P>
__device__ __forceinline__ void table_powers(const float2* tab, int lt, float2* p) {
  using G = PassGeom<C, P>;
  if constexpr (!G::kLast) {
    // opaque index: reloaded per use, not kept live between the halves
    const float2* t = tab + TwTab<C>::off(P) + G::m_of(opaque(lt)) - G::s;
#pragma unroll
    for (int q = 1; q < 16; ++q) p[q] = t[q * G::s];
  }
}

// Forward pass p on one register array: butterflies, then output twiddles.
template <class C, int P>
__device__ __forceinline__ void fwd_compute(float2* v, const float2* p) {
  using G = PassGeom<C, P>;
  if constexpr (G::kLast) {
#pragma unroll
    for (int i = 0; i < C::PT; i += C::RLAST) dftR<C::RLAST, false>(v + i);
  } else {
#pragma unroll
    for (int i = 0; i < C::NB; ++i) {
      dft16<false>(v + 16 * i);
      if (P == 0 && i == 1) apply16<false, true>(v + 16 * i, p);
      else apply16<false, false>(v + 16 * i, p);
    }
  }
}

// Inverse of pass p: conjugate input twiddles, then inverse butterflies.
template <class C, int P>
__device__ __forceinline__ void inv_compute(float2* v, const float2* p) {
  using G = PassGeom<C, P>;
  if constexpr (G::kLast) {
#pragma unroll
    for (int i = 0; i < C::PT; i += C::RLAST) dftR<C::RLAST, true>(v + i);
  } else {
#pragma unroll
    for (int i = 0; i < C::NB; ++i) {
      if (P == 0 && i == 1) apply16<true, true>(v + 16 * i, p);
      else apply16<true, false>(v + 16 * i, p);
      dft16<true>(v + 16 * i);
    }
  }
}

// Orders the LDS accesses of one wave (the exchanges after pass 0 stay inside
// the wave's own positions, so no workgroup barrier is needed): the LDS
// executes a wave's accesses in issue order; this keeps the compiler from
// moving them across.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Forward passes P .. NP-1 (P >= 1) of one array, wave-local.  Entry: v holds
// pass-P inputs; exit: the bins at positions PT lt + r.
template <class C, int P>
__device__ __forceinline__ void fwd_tail(float2* v, float2* lds, int lt, const float2* tab) {
  float2 p[16];
  table_powers<C, P>(tab, lt, p);
  fwd_compute<C, P>(v, p);
  if constexpr (P + 1 < C::NP) {
    lds_write<C, P>(lds, lt, v);
    wave_sync();
    lds_read<C, P + 1>(lds, lt, v);
    fwd_tail<C, P + 1>(v, lds, lt, tab);
  }
}

// Inverse passes P .. 1 of one array, wave-local.  Entry: v holds pass-P
// outputs (P = NP-1: the bins); exit: the pass-1 inputs at pass-1 positions.
template <class C, int P = C::NP - 1>
__device__ __forceinline__ void inv_head(float2* v, float2* lds, int lt, const float2* tab) {
  if constexpr (P >= 1) {
    float2 p[16];
    table_powers<C, P>(tab, lt, p);
    inv_compute<C, P>(v, p);
    if constexpr (P > 1) {
      lds_write<C, P>(lds, lt, v);
      wave_sync();
      lds_read<C, P - 1>(lds, lt, v);
      inv_head<C, P - 1>(v, lds, lt, tab);
    }
  }
}

// Forward transform of one array.  Entry: register r holds the point
// nat(lt, r); exit: the bin at position PT lt + r.  One workgroup barrier
// (which also publishes the twiddle table); all threads of the workgroup call
// it together.
template <class C>
__device__ __forceinline__ void forward1(float2* v, float2* lds, int lt, const float2* tab) {
  float2 p[16];
  pass0_powers<C>(pass0_w<C>(lt), p);
  fwd_compute<C, 0>(v, p);
  if constexpr (C::NP > 1) {
    lds_write<C, 0>(lds, lt, v);
    __syncthreads();
    lds_read<C, 1>(lds, lt, v);
    fwd_tail<C, 1>(v, lds, lt, tab);
  }
}

// Pass-0 inverse of an array whose passes NP-1 .. 1 were inverted by
// inv_head (one workgroup barrier); exit: the points nat(lt, r).
template <class C>
__device__ __forceinline__ void inverse_finish(float2* v, float2* lds, int lt) {
  lt = opaque(lt);  // LDS addresses recomputed rather than kept from pass 0
  const float2 w0 = pass0_w<C>(lt);
  if constexpr (C::NP > 1) {
    lds_write<C, 1>(lds, lt, v);
    __syncthreads();
    lds_read<C, 0>(lds, lt, v);
  }
  float2 p[16];
  pass0_powers<C>(w0, p);
  inv_compute<C, 0>(v, p);
}

// Natural-order index of register r (= 16 i + j) of thread lt.
template <class C>
__device__ __forceinline__ int nat(int lt, int r) {
  return lt + C::T * ((r >> 4) + (r & 15) * C::NB);
}

// v[r] *= exp(-+ i pi n(lt, r) / M) / t[lt] = exp(-+ i pi (i + j NB) / PT).
template <class C, bool INV, int R = 0>
__device__ __forceinline__ void odd_twiddle_fixed(float2* v) {
  if constexpr (R < C::PT) {
    constexpr int k = ((R >> 4) + (R & 15) * C::NB) * (32 / C::PT);
    v[R] = rotpi32<k, INV>(v[R]);
    odd_twiddle_fixed<C, INV, R + 1>(v);
  }
}

// Workgroup i runs on XCD i % 8; when the grid divides by 8, consecutive
// problems -- which read the same data: the two halves of a channel's
// spectrum, or the row pairs of a channel -- are placed on the same XCD so
// the second read is served by its L2.
__device__ __forceinline__ int xcd_grouped(int i, int n) {
  return (n % 8 == 0) ? (i % 8) * (n / 8) + i / 8 : i;
}

// Frequency index of transform position P, and its inverse, for the passes of
// Cfg C (in-place DIF: position digits, most significant first, are the
// frequency digits, least significant first; radix 16 except the last pass,
// radix RLAST).
template <class C>
__device__ __forceinline__ int freq_of_pos(int P) {
  int k = (P % C::RLAST) << (4 * (C::NP - 1));
  int q = P / C::RLAST;
#pragma unroll
  for (int i = C::NP - 2; i >= 0; --i) {
    k |= (q & 15) << (4 * i);
    q >>= 4;
  }
  return k;
}

template <class C>
__device__ __forceinline__ int pos_of_freq(int k) {
  int P = 0;
#pragma unroll
  for (int i = 0; i < C::NP - 1; ++i) P = P * 16 + ((k >> (4 * i)) & 15);
  return P * C::RLAST + (k >> (4 * (C::NP - 1)));
}

// Storage of a spectrum half (the kernel is real, so its 2M-point spectrum is
// Hermitian: X[-m] = conj X[m]).  With 16 points per thread the position
// 16 t + r of the convolution's transform holds frequency k, whose low digit
// (k mod 16, the first pass's index) is the position's top four bits.
// * Odd half, bins X[2k+1]: the partner of k is M - 1 - k, the complement of
//   every bit, hence of every position bit: thread T - 1 - t, register 15 - r.
// * Even half, bins X[2k]: the partner of k is -k mod M.  For k mod 16 = j != 0
//   that is 16 - j in the low digit and the complement of the rest, i.e.
//   thread (16 - j) Q + (Q - 1 - (t mod Q)), register 15 - r, Q = T / 16, where
//   j = t / Q.  The threads t < Q (k mod 16 = 0, the self-paired bins 0 and
//   M/2 among them) keep all 16 bins.
// Stored: registers r < 8 of every thread at slot r T + t, and for the even
// half registers r >= 8 of the threads t < Q at slot (23 - r) T + t: M/2 + M/32
// of the M slots of the even half, M/2 of the odd half.  Every other bin is the
// conjugate of a stored partner.  A reader's slot for register r >= 8 is then
// (15 - r) T + (a per-thread part): one lane offset, per-register scalar
// offsets.  Transforms below 256 points (T < 16) store every bin at r T + t.
template <int LOG2M>
struct SpecStore {
  using CM = Cfg<LOG2M, 16>;
  static constexpr bool kHerm = CM::T >= 16;
  static constexpr int Q = CM::T / 16;
  // whether bin (t, r) of `half` is stored, and its slot
  __device__ static __forceinline__ bool stored(int half, int t, int r) {
    return !kHerm || r < 8 || (half == 0 && t < Q);
  }
  __device__ static __forceinline__ int slot(int t, int r) {
    return (!kHerm || r < 8) ? r * CM::T + t : (23 - r) * CM::T + t;
  }
};

// Separated outputs of a PACK spectrum half for the convolution's column t
// (its 16 rows): lds holds the bins of the M/2-point transform of the packed
// z (or z exp(-2 pi i n / M) for half 1) at their transform positions.
// freq_of_pos is a permutation of bit fields, so the frequency of 16 t + r is
// kt | kr, with kr a compile-time constant.  Bins k and k + S share the pair
// Z[k mod S], Z[mirror]; k + S is the position bit RLAST/2 of the
// convolution's transform (top bit of its last digit), and its twiddle is -w.
template <int LOG2M>
__device__ __forceinline__ void pack_outputs(const float2* lds, int half, int t, float deff,
                                             float sg, float2* out) {
  using C = Cfg<LOG2M - 1, 16>;
  using CM = Cfg<LOG2M, 16>;
  using SS = SpecStore<LOG2M>;
  constexpr int M = CM::M, S = C::M;
  constexpr int RB = CM::RLAST / 2;
  const int kt = freq_of_pos<CM>(16 * t);
  const int kt1 = kt & (S - 1);
  const int pt = pos_of_freq<C>(kt1);
  // exp(-i pi (2 kt + half) / M): per-t table value
  const float2 wt = g_twiddle[(2 * kt + half) * (DSSM_TWN / (2 * M))];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (r & RB) continue;
    const bool st0 = SS::stored(half, t, r), st1 = SS::stored(half, t, r | RB);
    if (!st0 && !st1) continue;
    const int kr = freq_of_pos<CM>(r);
    const int k1 = kt1 | (kr & (S - 1));
    const int pa = pt + pos_of_freq<C>(kr & (S - 1));  // disjoint bit fields
    const int pb = half ? ((S - 1) ^ pa) : pos_of_freq<C>((S - k1) & (S - 1));
    const float2 A = lds[C::pad(pa)];
    const float2 B = lds[C::pad(pb)];
    // E = A + conj B, O = -i (A - conj B), X[k] = E + w O, X[k + S] = E - w O
    const float2 e = make_float2(A.x + B.x, A.y - B.y);
    const float2 o = make_float2(A.y + B.y, B.x - A.x);
    const float2 w = cmul(wt, g_twiddle[kr * (DSSM_TWN / M)]);
    const float2 wo = cmul(w, o);
    if (st0) out[SS::slot(t, r)] = make_float2(e.x + wo.x + deff, sg * (e.y + wo.y));
    if (st1) out[SS::slot(t, r | RB)] = make_float2(e.x - wo.x + deff, sg * (e.y - wo.y));
  }
}

// Raw buffer resource over `bytes` bytes at `base`.  The hardware range
// check of raw buffers returns zero for loads at or beyond `bytes` and drops
// such stores, so a row's tail and an inactive problem (bytes = 0) need no
// branches; one SGPR descriptor plus one lane offset addresses all of a
// thread's strided accesses.
typedef __amdgpu_buffer_rsrc_t BufRes;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ BufRes buf_res(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ float buf_load_f32(BufRes r, int voff, int soff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

__device__ __forceinline__ float2 buf_load_f32x2(BufRes r, int voff, int soff) {
  const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  return make_float2(__uint_as_float(w.x), __uint_as_float(w.y));
}

__device__ __forceinline__ void buf_store_f32(BufRes r, int voff, int soff, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, 0);
}

// Spectrum of the kernel, in the convolution's layout:
//   spec[h, half, e] = ( X[2 k + half] + D_f + D_b ) / (2M),
//   e = SpecStore slot of (t, r) for the stored bins (the others are the
//   conjugates of stored partners and are not written),
//   k = frequency of the convolution's transform position 16 t + r,
//   X = DFT_2M( pad(Re K_f) ) + conj( DFT_2M( pad(Re K_b) ) ).
// The feed-through D u is the convolution with D at tap 0, whose transform is
// the constant D: adding it to every bin makes the convolution produce y + D u.
// The backward DLR is a correlation with Re K_b, whose spectrum is the
// conjugate (no wrap-around reaches the first L outputs on a 2M circle).
// With conj != 0 the conjugate of the whole table is written (the transposed
// operator, for gradients); D may be NULL (no feed-through).
//
// Both real sequences of a channel ride in ONE complex transform, and the two
// real spectra are separated afterwards from the bins k and -k (the Hermitian
// symmetry of a real sequence's spectrum):
// * PACK (one direction): z[n] = K[2n] + i K[2n+1], n < S = M/2 (the even and
//   odd samples).  With Z = DFT_M(z): E = (Z[k] + conj Z[-k]) / 2 and
//   O = (Z[k] - conj Z[-k]) / 2i are the spectra of the even and odd samples,
//   and X[m] = E[m] + exp(-i pi m / M) O[m].  Even m need only Z at even
//   indices, DFT_S(z); odd m only Z at odd indices, DFT_S(z exp(-2 pi i n/M)):
//   workgroup `half` computes one S-point transform.
// * otherwise (two directions, or M = 16): z[n] = K_f[n] + i K_b[n], n < M,
//   and workgroup `half` computes the even or odd bins of its 2M-point
//   transform Z (an M-point transform of z, or of z t, t[n] = exp(-i pi n/M)),
//   then X[m] = (Z[m] + conj Z[-m]) / 2 + i (conj Z[m] - Z[-m]) / 2.
// After the transform the bins go to LDS in position order; each thread then
// reads the pairs its outputs need.
template <int LOG2M, bool PACK>
__global__ __launch_bounds__((Cfg<PACK ? LOG2M - 1 : LOG2M, 16>::WG)) void spectrum_kernel(
    const float* __restrict__ reK, const float* __restrict__ D, int ndir, int H, int L,
    float2* __restrict__ spec, int conj) {
  using C = Cfg<PACK ? LOG2M - 1 : LOG2M, 16>;  // the transform computed here
  using CM = Cfg<LOG2M, 16>;                     // the convolution's transform
  constexpr int M = CM::M, S = C::M;
  __shared__ float2 lds_all[C::G * C::LDSN];
  __shared__ float2 tab[TwTab<C>::kAlloc];
  twtab_init<C>(tab);
  const int lt = threadIdx.x % C::T;
  const int gi = threadIdx.x / C::T;
  float2* lds = lds_all + gi * C::LDSN;
  // the two halves of a channel, which read the same K row, share an XCD
  const int prob = xcd_grouped(blockIdx.x, gridDim.x) * C::G + gi;
  const bool active = prob < 2 * H;
  const int h = active ? (prob >> 1) : 0;
  const int half = prob & 1;

  // The factors 1/2 of the separation and 1/2M of the inverse transform are
  // applied to the input (the transform is linear).
  const float c = 0.25f / (float)M;
  float2 v[C::PT];
  {
    const float* kf = reK + (size_t)h * L;
    const float* kb = reK + ((size_t)(ndir - 1) * H + h) * L;
    // raw buffers over the rows: samples at or past L read zero
    const BufRes rf = buf_res(kf, active ? 4u * L : 0u);
    const BufRes rb = buf_res(kb, active && ndir == 2 ? 4u * L : 0u);
    const int lo = opaque(lt);
    if (PACK && (L & 1) == 0) {  // (K[2n], K[2n+1]) as one 8-byte load, wholly in or out of range
#pragma unroll
      for (int r = 0; r < C::PT; ++r) v[r] = buf_load_f32x2(rf, 8 * nat<C>(lo, r), 0);
    } else {
#pragma unroll
      for (int r = 0; r < C::PT; ++r) {
        const int n = nat<C>(lo, r);
        if (PACK)
          v[r] = make_float2(buf_load_f32(rf, 8 * n, 0), buf_load_f32(rf, 8 * n + 4, 0));
        else
          v[r] = make_float2(buf_load_f32(rf, 4 * n, 0), buf_load_f32(rb, 4 * n, 0));
      }
    }
  }
  if (half) {  // z t_S, t_S[n] = exp(-i pi n / S)
    const float2 tl = cscale(g_twiddle[lt * (DSSM_TWN / (2 * S))], c);
    odd_twiddle_fixed<C, false>(v);
#pragma unroll
    for (int r = 0; r < C::PT; ++r) v[r] = cmul(v[r], tl);
  } else {
#pragma unroll
    for (int r = 0; r < C::PT; ++r) v[r] = cscale(v[r], c);
  }
  forward1<C>(v, lds, lt, tab);
  // bins to LDS at their positions (this thread's own, wave-local positions)
  wave_sync();
  lds_write<C, C::NP - 1>(lds, lt, v);
  __syncthreads();
  if (!active) return;

  float deff = 0.f;
  if (D)
    for (int d = 0; d < ndir; ++d) deff += D[(size_t)d * H + h];
  const float sg = conj ? -1.f : 1.f;
  deff *= 1.0f / (2.0f * (float)M);
  float2* out = spec + ((size_t)h * 2 + half) * M;
  // Outputs of this thread: t = lt + T_S i (all the convolution's t), every r.
  // freq_of_pos is a permutation of bit fields, so the frequency of 16 t + r is
  // kt | kr, with kr a compile-time constant.
  static_assert(CM::T % C::T == 0, "output split");
#pragma unroll
  for (int i = 0; i < CM::T / C::T; ++i) {
    const int t = lt + C::T * i;
    const int kt = freq_of_pos<CM>(16 * t);
    if constexpr (PACK) {
      pack_outputs<LOG2M>(lds, half, t, deff, sg, out);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (!SpecStore<LOG2M>::stored(half, t, r)) continue;
        const int k = kt | freq_of_pos<CM>(r);  // output bin X[2k + half]
        const int k2 = half ? (M - 1 - k) : ((M - k) & (M - 1));
        const float2 A = lds[C::pad(pos_of_freq<C>(k))];
        const float2 B = lds[C::pad(pos_of_freq<C>(k2))];
        // (A + conj B) + i (conj A - B)
        out[SpecStore<LOG2M>::slot(t, r)] =
            make_float2(A.x + B.x + A.y + B.y + deff, sg * (A.y - B.y + A.x - B.x));
      }
    }
  }
}

// Points per thread of the convolution.  16 (1024 threads at M = 16384, four
// waves per SIMD) measured faster on MI355X than 32 (512 threads, two waves per
// SIMD): 56 us against 76 us for the long-sequence workload.
template <int LOG2M>
constexpr int conv_pt() { return 16; }

// Convolution of a pair of real rows (r1, r2: 4 L bytes each; r2 is absent
// when len2 = 0 and reads as zero) with one kernel spectrum, by one workgroup
// (C::G problems per workgroup when a transform is smaller than a wave).
// Both halves of the 2M spectrum are transformed: ve = z (even bins),
// vo = z t (odd bins), where z = r1 + i r2; outputs go to the rows o1, o2
// (o2 dropped when len2 = 0).  FULL selects the spectrum storage: every bin
// at slot r T + t (a complex kernel, whose spectrum has no symmetry), or the
// Hermitian half storage of SpecStore (a real kernel).  With a real kernel
// the real and imaginary parts of the result are the two rows' convolutions;
// with a complex one, z = Re + i Im of one complex row and the result is its
// convolution, real part to o1 and imaginary part to o2.
template <int LOG2M, bool FULL>
__device__ __forceinline__ void conv_rows(const float* __restrict__ r1,
                                          const float* __restrict__ r2, unsigned len1,
                                          unsigned len2, const float2* __restrict__ spec_h,
                                          int lt, float2* lds, const float2* tab,
                                          float* __restrict__ o1, float* __restrict__ o2,
                                          PhaseClock* pc = nullptr) {
  using C = Cfg<LOG2M, conv_pt<LOG2M>()>;
  // rows as buffers: element n of register r sits at byte 4 n, n = lt + T(...)
  const BufRes ur1 = buf_res(r1, len1);
  const BufRes ur2 = buf_res(r2, len2);

  // The whole element offset goes in the range-checked lane offset (the
  // scalar offset is added after the check).
  auto load_pair = [&](float2* v) {
    const int lo = opaque(lt);
#pragma unroll
    for (int r = 0; r < C::PT; ++r) {
      const int o = 4 * nat<C>(lo, r);
      v[r] = make_float2(buf_load_f32(ur1, o, 0), buf_load_f32(ur2, o, 0));
    }
  };
  // spectrum bin at position PT lt + r: stored at slot r T + lt, or (half
  // storage) the conjugate of a stored partner (SpecStore, shared with
  // spectrum_kernel, which uses the same PT); every access in range
  static_assert(C::PT == Cfg<LOG2M, 16>::PT, "spectrum layout is shared with spectrum_kernel");
  using SS = SpecStore<LOG2M>;
  constexpr bool kHerm = SS::kHerm && !FULL;
  const BufRes sr = buf_res(spec_h, 2u * C::M * 8u);
  auto load_spec = [&](auto half_c, float2* v) {
    constexpr int half = decltype(half_c)::value;
    const int lto = opaque(lt);
    const int o = 8 * lto;
#pragma unroll
    for (int r = 0; r < (kHerm ? 8 : C::PT); ++r)
      v[r] = buf_load_f32x2(sr, o, 8 * (half * C::M + r * C::T));
    if constexpr (kHerm) {
      // registers 8..15 at slot (15 - r) T + lane part: odd half, thread
      // T-1-lt conjugated; even half, the thread's own slots (lt < Q: lane
      // part 8T + lt) or the partner thread's, conjugated
      if constexpr (half == 1) {
        const int op = 8 * (C::T - 1 - lto);
#pragma unroll
        for (int r = 8; r < C::PT; ++r)
          v[r] = cconj(buf_load_f32x2(sr, op, 8 * (C::M + (15 - r) * C::T)));
      } else {
        constexpr int Q = SS::Q;
        // partner thread (16 - j) Q + (Q - 1 - (lt mod Q)) = 17 Q - 1 - lt
        const bool own = lto < Q;
        const int op = 8 * (own ? 8 * C::T + lto : 17 * Q - 1 - lto);
        const float sgn = own ? 1.f : -1.f;
#pragma unroll
        for (int r = 8; r < C::PT; ++r) {
          const float2 s = buf_load_f32x2(sr, op, 8 * (15 - r) * C::T);
          v[r] = make_float2(s.x, sgn * s.y);
        }
      }
    }
  };

  float2 ve[C::PT], vo[C::PT], sv[C::PT];
  load_pair(ve);
#pragma unroll
  for (int r = 0; r < C::PT; ++r) vo[r] = ve[r];
  {  // odd bins: pre-multiply by t[n] = t[lt] exp(-i pi (i + j NB) / PT)
    const float2 tl = g_twiddle[lt * (DSSM_TWN / (2 * C::M))];
    odd_twiddle_fixed<C, false>(vo);
#pragma unroll
    for (int r = 0; r < C::PT; ++r) vo[r] = cmul(vo[r], tl);
  }
  if (pc) pc->mark(0);  // entry: twiddle table, input requested
  // pass 0 of both halves (shared twiddles)
  {
    float2 p[16];
    pass0_powers<C>(pass0_w<C>(lt), p);
    fwd_compute<C, 0>(ve, p);
    fwd_compute<C, 0>(vo, p);
  }
  // even half: exchange, wave-local passes, product, inverse back to pass 0
  if constexpr (C::NP > 1) {
    lds_write<C, 0>(lds, lt, ve);
    __syncthreads();
    lds_read<C, 1>(lds, lt, ve);
    fwd_tail<C, 1>(ve, lds, lt, tab);
  }
  if (pc) pc->mark(1);  // even half forward
  load_spec(std::integral_constant<int, 0>{}, sv);
#pragma unroll
  for (int r = 0; r < C::PT; ++r) ve[r] = cmul(ve[r], sv[r]);
  if (pc) pc->mark(2);  // even half: spectrum read, product
  inv_head<C>(ve, lds, lt, tab);
  inverse_finish<C>(ve, lds, lt);
  if (pc) pc->mark(3);  // even half inverse
  // odd half: its pass-0 positions are disjoint from every other thread's,
  // so it may be written while others still read the even half's
  if constexpr (C::NP > 1) {
    lds_write<C, 0>(lds, lt, vo);
    __syncthreads();
    lds_read<C, 1>(lds, lt, vo);
    fwd_tail<C, 1>(vo, lds, lt, tab);
  }
  if (pc) pc->mark(4);  // odd half forward
  load_spec(std::integral_constant<int, 1>{}, sv);
#pragma unroll
  for (int r = 0; r < C::PT; ++r) vo[r] = cmul(vo[r], sv[r]);
  if (pc) pc->mark(5);  // odd half: spectrum read, product
  inv_head<C>(vo, lds, lt, tab);
  inverse_finish<C>(vo, lds, lt);
  if (pc) pc->mark(6);  // odd half inverse
  // The thread index is re-derived here (opaque to the compiler) so the store
  // addresses and t[lt] are recomputed instead of being kept live -- and
  // spilled -- across both transforms.
  const int lte = opaque(lt);
  {  // y = ye + conj(t) yo (D u is already in the spectrum)
    const float2 tlc = cconj(g_twiddle[lte * (DSSM_TWN / (2 * C::M))]);
    odd_twiddle_fixed<C, true>(vo);
#pragma unroll
    for (int r = 0; r < C::PT; ++r) ve[r] = cadd(ve[r], cmul(vo[r], tlc));
  }
  const BufRes yr1 = buf_res(o1, len1);
  const BufRes yr2 = buf_res(o2, len2);
#pragma unroll
  for (int r = 0; r < C::PT; ++r) {
    const int o = 4 * nat<C>(lte, r);
    buf_store_f32(yr1, o, 0, ve[r].x);
    buf_store_f32(yr2, o, 0, ve[r].y);
  }
  if (pc) pc->mark(7);  // combination, stores issued
}

// DLR convolution: workgroup problem = (channel h, row pair pr), the batch
// rows b1 = 2 pr and b2 = 2 pr + 1 of u [B, H, L] riding in one complex
// sequence, with the channel's real-kernel spectrum (Hermitian half storage).
template <int LOG2M>
__global__ __launch_bounds__((Cfg<LOG2M, conv_pt<LOG2M>()>::WG)) void conv_kernel(
    const float* __restrict__ u, const float2* __restrict__ spec, int B, int H, int L, int npairs,
    float* __restrict__ y) {
  using C = Cfg<LOG2M, conv_pt<LOG2M>()>;
  PhaseClock pc;
  __shared__ float2 lds_all[C::G * C::LDSN];
  __shared__ float2 tab[TwTab<C>::kAlloc];
  twtab_init<C>(tab);  // published by the first barrier, before its first use
  const int lt = threadIdx.x % C::T;
  const int gi = threadIdx.x / C::T;
  const int prob = xcd_grouped(blockIdx.x, gridDim.x) * C::G + gi;
  const bool active = prob < H * npairs;
  const int h = active ? prob / npairs : 0;
  const int pr = active ? prob % npairs : 0;
  const int b1 = 2 * pr, b2 = 2 * pr + 1;
  const bool has2 = active && b2 < B;
  const size_t o1 = ((size_t)b1 * H + h) * L;
  const size_t o2 = ((size_t)(has2 ? b2 : b1) * H + h) * L;
  conv_rows<LOG2M, false>(u + o1, u + o2, active ? 4u * L : 0u, has2 ? 4u * L : 0u,
                          spec + (size_t)h * 2 * C::M, lt, lds_all + gi * C::LDSN, tab, y + o1,
                          y + o2, &pc);
  pc.write();
}

// S5 convolution view: workgroup problem = one complex row (b, p) of
// v [B][P][2][L] (real row, imaginary row), convolved with the spectrum of
// lambda_p^j (full storage) into x [B][P][2][L].  Problems are numbered
// p-major, so the rows that read one spectrum share an XCD's L2.
template <int LOG2M>
__global__ __launch_bounds__((Cfg<LOG2M, conv_pt<LOG2M>()>::WG)) void s5_conv_kernel(
    const float* __restrict__ v, const float2* __restrict__ spec, int B, int P, int L,
    float* __restrict__ x) {
  using C = Cfg<LOG2M, conv_pt<LOG2M>()>;
  __shared__ float2 lds_all[C::G * C::LDSN];
  __shared__ float2 tab[TwTab<C>::kAlloc];
  twtab_init<C>(tab);
  const int lt = threadIdx.x % C::T;
  const int gi = threadIdx.x / C::T;
  const int prob = xcd_grouped(blockIdx.x, gridDim.x) * C::G + gi;
  const bool active = prob < B * P;
  const int p = active ? prob / B : 0;
  const int b = active ? prob % B : 0;
  const size_t o = ((size_t)b * P + p) * 2 * L;
  const unsigned len = active ? 4u * L : 0u;
  conv_rows<LOG2M, true>(v + o, v + o + L, len, len, spec + (size_t)p * 2 * C::M, lt,
                         lds_all + gi * C::LDSN, tab, x + o, x + o + L);
}

// Spectrum of the kernel kappa[j] = lambda_p^j (0 <= j < M, zero on the upper
// half of the 2M circle) in the convolution's full storage, scaled by 1/(2M):
//   spec[p, half, r T + t] = S[2 k + half],  k = frequency of position 16 t + r,
//   S[m] = (1/2M) sum_{j<M} (lambda w^m)^j = (1/2M) (1 - z^M) / (1 - z),
//   z = lambda w^m, w = exp(-i pi / M), z^M = (-1)^m lambda^M.
// Every output sample x_k = sum_{j<=k} lambda^j v_{k-j} (k < L <= M) is then
// the k-th sample of the 2M-circular convolution, as the taps j >= M never
// meet a nonzero input there ("Simplified State Space Layers for Sequence
// Modeling", section 2.3: the convolution kernel of a diagonal linear system
// is the powers of its eigenvalues).  float64 throughout, rounded once: near
// z = 1 (|lambda| close to 1 with a phase close to a bin's) the quotient is
// taken as expm1(M d) / expm1(d), d = log z, which has no cancellation.
__device__ __forceinline__ double2 zdiv(double2 a, double2 b) {
  const double den = b.x * b.x + b.y * b.y;
  return make_double2((a.x * b.x + a.y * b.y) / den, (a.y * b.x - a.x * b.y) / den);
}

// exp(d) - 1 for complex d = (x, y), without cancellation at small |d|:
// Re = expm1(x) cos y - 2 sin^2(y / 2), Im = exp(x) sin y.
__device__ __forceinline__ double2 zexpm1(double x, double y) {
  double sh, ch;
  sincos(0.5 * y, &sh, &ch);
  const double s = 2.0 * sh * ch, c = 1.0 - 2.0 * sh * sh;
  return make_double2(expm1(x) * c - 2.0 * sh * sh, exp(x) * s);
}

template <int LOG2M>
__global__ __launch_bounds__(256) void s5_spec_kernel(const float2* __restrict__ lam, int P,
                                                       float2* __restrict__ spec) {
  using CM = Cfg<LOG2M, 16>;
  constexpr int M = CM::M;
  const int p = blockIdx.y;
  const float2 lf = lam[p];
  const double lre = (double)lf.x, lim = (double)lf.y;
  // log lambda: log |lambda| = log1p(|lambda|^2 - 1) / 2 (the squares of the
  // float32 parts are exact in float64, so |lambda|^2 - 1 is formed exactly
  // up to one rounding), arg lambda
  const double a2m1 = (lre * lre - 1.0) + lim * lim;
  const double lmag = 0.5 * log1p(a2m1), larg = atan2(lim, lre);
  // lambda^M = exp(M log lambda); the phase M arg is reduced by sincos itself
  double sM, cM;
  sincos((double)M * larg, &sM, &cM);
  const double eM = exp((double)M * lmag);
  const double2 lamM = make_double2(eM * cM, eM * sM);
  const double scale = 1.0 / (2.0 * M);
  float2* out = spec + (size_t)p * 2 * M;
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < 2 * M; e += gridDim.x * blockDim.x) {
    const int half = e / M, slot = e % M;
    const int t = slot % CM::T, r = slot / CM::T;
    const int k = freq_of_pos<CM>(16 * t + r);
    const int m = 2 * k + half;
    double sw, cw;
    sincospi(-(double)m / (double)M, &sw, &cw);  // w^m = exp(-i pi m / M)
    const double2 z = make_double2(lre * cw - lim * sw, lre * sw + lim * cw);
    const double2 omz = make_double2(1.0 - z.x, -z.y);
    double2 q;
    if (omz.x * omz.x + omz.y * omz.y >= 1e-6) {
      const double sg = (m & 1) ? -1.0 : 1.0;  // z^M = (-1)^m lambda^M
      q = zdiv(make_double2(1.0 - sg * lamM.x, -sg * lamM.y), omz);
    } else {
      // d = log z = log lambda - i pi m / M, imaginary part reduced to [-pi, pi]
      double dy = larg - M_PI * ((double)m / (double)M);
      dy -= 2.0 * M_PI * rint(dy / (2.0 * M_PI));
      const double2 den = zexpm1(lmag, dy);
      if (den.x == 0.0 && den.y == 0.0) {
        q = make_double2((double)M, 0.0);  // z = 1: the sum of M ones
      } else {
        // M d: its phase M dy reduced by sincos inside zexpm1
        q = zdiv(zexpm1((double)M * lmag, (double)M * dy), den);
      }
    }
    out[e] = make_float2((float)(q.x * scale), (float)(q.y * scale));
  }
}

// Kernel cotangents of the gradients: the lagged correlations of the row
// pairs (u_b, dy_b) of channel h, summed over the batch in the frequency
// domain, on one half of the 2M circle ("Simplifying and Understanding State
// Space Models with Diagonal Linear RNNs", section 2: the convolution view;
// the correlation is the transposed Toeplitz product).  With
// C(m) = sum_b DY_b(m) conj U_b(m) and c = IDFT_2M(C):
//   G_f[j] = sum_b sum_i u_b[i] dy_b[i + j] = c[j],
//   G_b[j] = sum_b sum_i dy_b[i] u_b[i + j] = c[2M - j]   (0 <= j < L).
// One workgroup per (channel, half): for each b it transforms
// z = u_b + i dy_b (even bins: z; odd bins: z t, t[n] = exp(-i pi n / M)),
// meets each bin Z[m] with Z[-m] in LDS and adds
//   DY conj U = Im(Z[m] Z[-m]) / 2 - i (|Z[m]|^2 - |Z[-m]|^2) / 4
// (with the inverse's 1/2M) to its registers; after the batch it inverts its
// half and stores part[h][half][n] (n < M): the real part of the half's
// inverse, the odd half multiplied by conj t[n] first.  Then
//   c[n] = part[h][0][n] + part[h][1][n],  c[n + M] = part[h][0][n] - part[h][1][n].
// With G > 1 batch groups (few channels, many rows) workgroup (g, h, half)
// takes rows b = g, g + G, ... and stores part[g][h][half][n]; the groups'
// parts add up (the map from the rows to c is linear).
template <int LOG2M>
__global__ __launch_bounds__((Cfg<LOG2M, 16>::WG)) void corr_kernel(
    const float* __restrict__ u, const float* __restrict__ dy, int B, int H, int L, int G,
    float* __restrict__ part) {
  using C = Cfg<LOG2M, 16>;
  constexpr int M = C::M;
  __shared__ float2 lds_all[C::G * C::LDSN];
  __shared__ float2 tab[TwTab<C>::kAlloc];
  twtab_init<C>(tab);  // published by the first barrier
  const int lt = threadIdx.x % C::T;
  const int gi = threadIdx.x / C::T;
  float2* lds = lds_all + gi * C::LDSN;
  // the two halves of a channel, which read the same rows, share an XCD
  const int prob = xcd_grouped(blockIdx.x, gridDim.x) * C::G + gi;
  const bool active = prob < 2 * H * G;
  const int grp = active ? prob / (2 * H) : 0;
  const int h = active ? (prob % (2 * H)) >> 1 : 0;
  const int half = prob & 1;
  const int kt = freq_of_pos<C>(C::PT * lt);  // bins of this thread: kt | freq_of_pos(r)
  const float c1 = 0.25f / (float)M, c2 = 0.125f / (float)M;

  float2 acc[C::PT];
#pragma unroll
  for (int r = 0; r < C::PT; ++r) acc[r] = make_float2(0.f, 0.f);
  for (int b = grp; b < B; b += G) {
    float2 v[C::PT];
    {
      const BufRes ur = buf_res(u + ((size_t)b * H + h) * L, active ? 4u * L : 0u);
      const BufRes dr = buf_res(dy + ((size_t)b * H + h) * L, active ? 4u * L : 0u);
      const int lo = opaque(lt);
#pragma unroll
      for (int r = 0; r < C::PT; ++r) {
        const int o = 4 * nat<C>(lo, r);
        v[r] = make_float2(buf_load_f32(ur, o, 0), buf_load_f32(dr, o, 0));
      }
    }
    if (half) {  // z t
      const float2 tl = g_twiddle[lt * (DSSM_TWN / (2 * M))];
      odd_twiddle_fixed<C, false>(v);
#pragma unroll
      for (int r = 0; r < C::PT; ++r) v[r] = cmul(v[r], tl);
    }
    forward1<C>(v, lds, lt, tab);
    // bins to LDS at their positions, then each meets its mirror bin
    wave_sync();
    lds_write<C, C::NP - 1>(lds, lt, v);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < C::PT; ++r) {
      const int k = kt | freq_of_pos<C>(r);
      const int k2 = half ? (M - 1 - k) : ((M - k) & (M - 1));
      const float2 zm = lds[C::pad(pos_of_freq<C>(k2))];
      const float2 z = v[r];
      acc[r].x = fmaf(c1, fmaf(z.x, zm.y, z.y * zm.x), acc[r].x);
      acc[r].y = fmaf(-c2, (fmaf(z.x, z.x, z.y * z.y) - fmaf(zm.x, zm.x, zm.y * zm.y)), acc[r].y);
    }
    __syncthreads();  // mirror reads done before the next row's exchange
  }
  inv_head<C>(acc, lds, lt, tab);
  inverse_finish<C>(acc, lds, lt);
  const int lte = opaque(lt);
  if (half) {  // conj t[n]
    const float2 tlc = cconj(g_twiddle[lte * (DSSM_TWN / (2 * M))]);
    odd_twiddle_fixed<C, true>(acc);
#pragma unroll
    for (int r = 0; r < C::PT; ++r) acc[r] = cmul(acc[r], tlc);
  }
  const BufRes pr = buf_res(part + (((size_t)grp * H + h) * 2 + half) * M, active ? 4u * M : 0u);
#pragma unroll
  for (int r = 0; r < C::PT; ++r) buf_store_f32(pr, 4 * nat<C>(lte, r), 0, acc[r].x);
}

template <int LOG2M>
hipError_t corr_launch(const float* u, const float* dy, int B, int H, int L, int G, float* part,
                       hipStream_t st) {
  using C = Cfg<LOG2M, 16>;
  const long nprob = 2L * H * G;
  const long nblk = (nprob + C::G - 1) / C::G;
  launch_k(corr_kernel<LOG2M>, dim3((unsigned)nblk), dim3(C::WG), st, KEvents{}, u, dy, B, H, L, G,
           part);
  return hipGetLastError();
}

template <int LOG2M, bool PACK>
hipError_t spectrum_launch2(const float* reK, const float* D, int ndir, int H, int L,
                            float2* spec, hipStream_t st, KEvents ev, int conj) {
  using C = Cfg<PACK ? LOG2M - 1 : LOG2M, 16>;
  const int nprob = 2 * H;
  const int nblk = (nprob + C::G - 1) / C::G;
  launch_k(spectrum_kernel<LOG2M, PACK>, dim3(nblk), dim3(C::WG), st, ev, reK, D, ndir, H, L,
           spec, conj);
  return hipGetLastError();
}

// One direction packs even and odd samples (transforms of M/2 points) when M
// allows it; two directions pack forward and backward kernels.
template <int LOG2M>
hipError_t spectrum_launch(const float* reK, const float* D, int ndir, int H, int L, float2* spec,
                           hipStream_t st, KEvents ev, int conj) {
  if constexpr (LOG2M >= 5) {
    if (ndir == 1) return spectrum_launch2<LOG2M, true>(reK, D, ndir, H, L, spec, st, ev, conj);
  }
  return spectrum_launch2<LOG2M, false>(reK, D, ndir, H, L, spec, st, ev, conj);
}

template <int LOG2M>
hipError_t conv_launch(const float* u, const float2* spec, int B, int H, int L, float* y,
                       hipStream_t st, KEvents ev) {
  using C = Cfg<LOG2M, conv_pt<LOG2M>()>;
  const int npairs = (B + 1) / 2;
  const long nprob = (long)H * npairs;
  const long nblk = (nprob + C::G - 1) / C::G;
  launch_k(conv_kernel<LOG2M>, dim3((unsigned)nblk), dim3(C::WG), st, ev, u, spec, B, H, L, npairs,
           y);
  return hipGetLastError();
}

template <int LOG2M>
hipError_t s5_spec_launch(const float* lambda, int P, float2* spec, hipStream_t st, KEvents ev) {
  constexpr int M = 1 << LOG2M;
  const int per = std::max(1, 2 * M / 256);
  launch_k(s5_spec_kernel<LOG2M>, dim3((unsigned)std::min(per, 64), (unsigned)P), dim3(256), st,
           ev, reinterpret_cast<const float2*>(lambda), P, spec);
  return hipGetLastError();
}

template <int LOG2M>
hipError_t s5_conv_launch(const float* v, const float2* spec, int B, int P, int L, float* x,
                          hipStream_t st, KEvents ev) {
  using C = Cfg<LOG2M, conv_pt<LOG2M>()>;
  const long nprob = (long)B * P;
  const long nblk = (nprob + C::G - 1) / C::G;
  launch_k(s5_conv_kernel<LOG2M>, dim3((unsigned)nblk), dim3(C::WG), st, ev, v, spec, B, P, L, x);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_s5_spectrum(const float* lambda, int P, int log2m, float2* spec,
                              hipStream_t st, KEvents ev) {
  switch (log2m) {
#define X(n) \
  case n:    \
    return s5_spec_launch<n>(lambda, P, spec, st, ev);
    DSSM_FFT_CASES(X)
#undef X
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_s5_conv(const float* v, const float2* spec, int B, int P, int L, int log2m,
                          float* x, hipStream_t st, KEvents ev) {
  switch (log2m) {
#define X(n) \
  case n:    \
    return s5_conv_launch<n>(v, spec, B, P, L, x, st, ev);
    DSSM_FFT_CASES(X)
#undef X
    default:
      return hipErrorInvalidValue;
  }
}

int fft_log2m(int L) {
  int l = 4;
  while ((1 << l) < L) ++l;
  return l;
}


hipError_t launch_spectrum(const float* reK, const float* D, int ndir, int H, int L, int log2m,
                           float2* spec, hipStream_t st, KEvents ev, int conj) {
  switch (log2m) {
#define X(n) \
  case n:    \
    return spectrum_launch<n>(reK, D, ndir, H, L, spec, st, ev, conj);
    DSSM_FFT_CASES(X)
#undef X
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_conv(const float* u, const float2* spec, int B, int H, int L, int log2m, float* y,
                       hipStream_t st, KEvents ev) {
  switch (log2m) {
#define X(n) \
  case n:    \
    return conv_launch<n>(u, spec, B, H, L, y, st, ev);
    DSSM_FFT_CASES(X)
#undef X
    default:
      return hipErrorInvalidValue;
  }
}

int corr_groups(int B, int H) {
  // enough (channel, half, group) workgroups for the 256 CUs, at most one
  // group per row; a fixed count, so workspace sizes do not depend on the device
  const long want = (256 + 2L * H - 1) / (2L * H);
  return (int)std::max(1L, std::min<long>(B, want));
}

hipError_t launch_corr(const float* u, const float* dy, int B, int H, int L, int log2m,
                       float* part, hipStream_t st) {
  const int G = corr_groups(B, H);
  switch (log2m) {
#define X(n) \
  case n:    \
    return corr_launch<n>(u, dy, B, H, L, G, part, st);
    DSSM_FFT_CASES(X)
#undef X
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace dssm

#ifdef DSSM_PHASE_STAMPS
// Buffer for the convolution's phase stamps (instrumented builds only).
extern "C" int dssm_phase_stamps_fft(void* buf) {
  return (int)hipMemcpyToSymbol(HIP_SYMBOL(dssm::g_phase_buf), &buf, sizeof(buf));
}
#endif
