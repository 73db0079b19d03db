// Launch-invariant binary32 log1p for gfx950 (MI355X).
//
// The ROCm/TransformerEngine issue "CP LSE merge switches compiled variants on
// ROCm, breaking forward reproducibility" ("Root cause", "Minimal reproducer")
// shows an elementwise binary32 log1p whose results change with the launch
// shape: at some block shapes the compiler vectorises the body, the
// multiply-add contraction inside the library routine changes with it, and
// results move by about one ULP.  This kernel gives every input one result,
// whatever the launch: ln(1 + x) rounded once to the nearest binary32, ties to
// even.  A correctly rounded result is a function of x alone.  On top of that
// the build passes -ffp-contract=off and every fused multiply-add below is
// written out, so no code-generation choice can change an operation.
//
// Fast path, in binary64 (x is binary32, so X = x is exact):
//   u  = fl(1 + X); c = X - (u - 1), the rounding error of u, kept when u <= 2.
//        u is exact for 2^-29 <= |X| < 2^52, so c != 0 only when |u - 1| <= 2^-29.
//   u  = 2^k m with m in [sqrt(1/2), sqrt(2)); f = m - 1 (exact: Sterbenz).
//   s  = f / (2 + f), |s| <= 3 - 2 sqrt(2) < 0.1716, and
//        ln m = 2 atanh(s) = 2s + 2s^3/3 + 2s^5/5 + ..., summed to s^19
//        (the first term left out is below 2^-55 of the sum).
//   ln(1 + X) = k ln2_hi + (k ln2_lo + (ln m + c (2 - u))), where c (2 - u)
//        is c / u to within (u - 1)^2 relative, and k ln2_hi is exact.
// The rounding errors add up to less than 2^-50 of the result (division and
// 2 + f: 2 ulp; the series and the three sums: at most 3 more; the truncation
// 2^-55; relative to |result| >= 0.346 when k != 0).
//
// Rounding test: y is rounded to binary32 r.  If y lies farther than 2^-47 |y|
// from both midpoints between r and its binary32 neighbours, the exact value
// is on the same side of them and r is the correctly rounded result.  Other
// inputs (about one in four million) take the accurate path.
//
// Accurate path: the same steps in double-double arithmetic (unevaluated sums
// hi + lo with |lo| <= ulp(hi) / 2; Knuth's two-sum, the fma two-product,
// Dekker-style products and quotients), 1 + X held exactly, the atanh series
// to s^39 with double-double coefficients, ln 2 in three parts.  Its error is
// about 2^-100 relative; the double-double result is rounded to binary32 by
// comparing its distance from r with half the neighbouring binary32 spacing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace addrms {
namespace {

#define DEV __device__ __forceinline__

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ln 2 in parts.  LN2_HI has 44 significant bits, so k * LN2_HI is exact for
// |k| < 2^9; LN2_LO is the binary64 rounding of ln 2 - LN2_HI.  For the
// accurate path ln 2 = LN2_P1 + LN2_P2 + LN2_P3 to about 2^-150, with P1 and
// P2 of 44 bits each.  (Values from ln 2 to 80 digits.)
constexpr double LN2_HI = 0x1.62e42fefa3a00p-1;
constexpr double LN2_LO = -0x1.0ca86c3898d00p-49;
constexpr double LN2_P1 = 0x1.62e42fefa3a00p-1;
constexpr double LN2_P2 = -0x1.0ca86c3898c00p-49;
constexpr double LN2_P3 = -0x1.ff0342542fc33p-94;
constexpr double SQRT_HALF = 0.70710678118654752440;

DEV uint32_t fbits(float v) { return __builtin_bit_cast(uint32_t, v); }
DEV float ffrom(uint32_t b) { return __builtin_bit_cast(float, b); }

// u = 2^k m, m in [sqrt(1/2), sqrt(2)); u > 0 and finite.
DEV double reduce(double u, int* k) {
  double m = __builtin_amdgcn_frexp_mant(u);  // [0.5, 1)
  int e = __builtin_amdgcn_frexp_exp(u);
  if (m < SQRT_HALF) {
    m = m + m;
    e = e - 1;
  }
  *k = e;
  return m;
}

// ---------------------------------------------------------------- fast path

// ln(1 + X) in binary64 for X in (-1, FLT_MAX], relative error below 2^-50.
DEV double log1p_fast(double X) {
  const double u = X + 1.0;
  const double c = u <= 2.0 ? X - (u - 1.0) : 0.0;
  int k;
  const double m = reduce(u, &k);
  const double f = m - 1.0;
  const double s = f / (2.0 + f);
  const double z = s * s;
  // 2/3 + 2z/5 + ... + 2z^8/19
  double R = 2.0 / 19.0;
  R = __builtin_fma(R, z, 2.0 / 17.0);
  R = __builtin_fma(R, z, 2.0 / 15.0);
  R = __builtin_fma(R, z, 2.0 / 13.0);
  R = __builtin_fma(R, z, 2.0 / 11.0);
  R = __builtin_fma(R, z, 2.0 / 9.0);
  R = __builtin_fma(R, z, 2.0 / 7.0);
  R = __builtin_fma(R, z, 2.0 / 5.0);
  R = __builtin_fma(R, z, 2.0 / 3.0);
  const double ln_m = __builtin_fma(s * z, R, s + s);
  const double kd = (double)k;
  const double t1 = ln_m + c * (2.0 - u);
  const double t2 = __builtin_fma(kd, LN2_LO, t1);
  return __builtin_fma(kd, LN2_HI, t2);
}

// The binary32 rounding of y is certain when y, known to within 2^-47 |y|,
// is that far from both midpoints around it.  y != 0 and finite.
DEV bool rounding_is_certain(double y, float r) {
  const double a = __builtin_fabs(y);
  const float ra = __builtin_fabsf(r);
  const uint32_t rb = fbits(ra);  // >= 1: |y| > 2^-150 here
  const double up = (double)ffrom(rb + 1u);
  const double dn = (double)ffrom(rb - 1u);
  const double m_hi = ((double)ra + up) * 0.5;  // exact
  const double m_lo = ((double)ra + dn) * 0.5;
  const double tol = a * 0x1p-47;
  return (a - m_lo > tol) && (m_hi - a > tol);
}

// ---------------------------------------------------------------- accurate path

struct dd {
  double hi, lo;
};

DEV dd two_sum(double a, double b) {
  const double s = a + b;
  const double bb = s - a;
  const double e = (a - (s - bb)) + (b - bb);
  return {s, e};
}

DEV dd fast_two_sum(double a, double b) {  // |a| >= |b| or a == 0
  const double s = a + b;
  return {s, b - (s - a)};
}

DEV dd two_prod(double a, double b) {
  const double p = a * b;
  return {p, __builtin_fma(a, b, -p)};
}

DEV dd dd_add(dd x, dd y) {
  dd s = two_sum(x.hi, y.hi);
  const dd t = two_sum(x.lo, y.lo);
  s.lo = s.lo + t.hi;
  s = fast_two_sum(s.hi, s.lo);
  s.lo = s.lo + t.lo;
  return fast_two_sum(s.hi, s.lo);
}

DEV dd dd_mul(dd x, dd y) {
  dd p = two_prod(x.hi, y.hi);
  p.lo = __builtin_fma(x.hi, y.lo, p.lo);
  p.lo = __builtin_fma(x.lo, y.hi, p.lo);
  return fast_two_sum(p.hi, p.lo);
}

DEV dd dd_mul_d(dd x, double b) {
  dd p = two_prod(x.hi, b);
  p.lo = __builtin_fma(x.lo, b, p.lo);
  return fast_two_sum(p.hi, p.lo);
}

DEV dd dd_neg(dd x) { return {-x.hi, -x.lo}; }

// x / y by three quotient digits, each corrected against the remainder.
DEV dd dd_div(dd x, dd y) {
  const double q1 = x.hi / y.hi;
  dd r = dd_add(x, dd_neg(dd_mul_d(y, q1)));
  const double q2 = r.hi / y.hi;
  r = dd_add(r, dd_neg(dd_mul_d(y, q2)));
  const double q3 = r.hi / y.hi;
  const dd q = fast_two_sum(q1, q2);
  return dd_add(q, dd{q3, 0.0});
}

// 1 / n as a double-double: hi = fl(1/n), lo = fl((1 - hi n) / n), where the
// residual 1 - hi n is exact by fma.
DEV dd recip(double n) {
  const double hi = 1.0 / n;
  return {hi, __builtin_fma(-hi, n, 1.0) / n};
}

// ln(1 + X) as a double-double, relative error about 2^-100.
DEV dd log1p_accurate(double X) {
  const dd U = two_sum(1.0, X);  // exactly 1 + X
  int k;
  const double mh = reduce(U.hi, &k);
  const double ml = __builtin_amdgcn_ldexp(U.lo, -k);
  const dd F = two_sum(mh - 1.0, ml);  // m - 1, exact
  const dd D = dd_add(dd{2.0, 0.0}, F);
  const dd S = dd_div(F, D);
  const dd Z = dd_mul(S, S);
  // P = sum_{n=0}^{19} Z^n / (2n + 1), by Horner
  dd P = recip(39.0);
  for (int n = 18; n >= 0; --n) P = dd_add(dd_mul(P, Z), recip(2.0 * n + 1.0));
  dd L = dd_mul(S, P);
  L = {L.hi + L.hi, L.lo + L.lo};  // 2 S P: ln m
  const double kd = (double)k;
  const dd K = dd_add(two_sum(kd * LN2_P1, kd * LN2_P2), dd{kd * LN2_P3, 0.0});
  return dd_add(K, L);
}

// Nearest binary32 (ties to even) of the double-double Y, Y != 0.
DEV float round_dd_to_f32(dd Y) {
  const bool neg = Y.hi < 0.0;
  const double ah = neg ? -Y.hi : Y.hi;
  const double al = neg ? -Y.lo : Y.lo;
  float ra = (float)ah;
  const uint32_t rb = fbits(ra);
  const double diff = (ah - (double)ra) + al;  // ah - ra is exact
  if (diff > 0.0) {
    const double half = ((double)ffrom(rb + 1u) - (double)ra) * 0.5;
    if (diff > half || (diff == half && (rb & 1u))) ra = ffrom(rb + 1u);
  } else if (diff < 0.0) {
    const double half = ((double)ra - (double)ffrom(rb - 1u)) * 0.5;
    if (-diff > half || (-diff == half && (rb & 1u))) ra = ffrom(rb - 1u);
  }
  return neg ? -ra : ra;
}

// The accurate path, correctly rounded to binary32.  Rare, so it is kept out
// of line: one copy, called only by the lanes that need it.
__device__ __noinline__ float log1p_accurate_f32(double X) {
  return round_dd_to_f32(log1p_accurate(X));
}

// ---------------------------------------------------------------- one element

// IEEE special cases of log1p, then the fast path, then, when its rounding is
// not certain (or `accurate` asks for it), the accurate path.
DEV float log1p_f32_elem(float x, bool accurate) {
  const bool is_nan = x != x;
  const bool special = is_nan || x == 0.0f || x <= -1.0f || x == __builtin_inff();
  float special_val;
  if (is_nan)
    special_val = x + x;  // quiet NaN
  else if (x == 0.0f || x == __builtin_inff())
    special_val = x;  // +-0 keep their sign; +Inf
  else if (x == -1.0f)
    special_val = -__builtin_inff();
  else
    special_val = __builtin_nanf("");  // x < -1, -Inf
  const double X = special ? 0.5 : (double)x;
  const double y = log1p_fast(X);
  float r = (float)y;
  if (!special && (accurate || !rounding_is_certain(y, r))) r = log1p_accurate_f32(X);
  return special ? special_val : r;
}

// ---------------------------------------------------------------- kernel

struct Log1pParams {
  const float* x;
  float* out;
  int64_t n;
  int64_t tiles;  // ceil(n / (blockDim.x * E))
  int accurate;   // every element by the accurate path (test hook)
};

DEV __amdgpu_buffer_rsrc_t tile_rsrc(const float* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, bytes, 0x00020000);
}

// E consecutive elements per thread, blockDim.x * E per tile; workgroups loop
// over tiles.  Full tiles use E-wide nontemporal buffer loads and stores;
// the last, partial tile goes element by element with a bounds check.
template <int E>
__global__ __launch_bounds__(1024) void k_log1p(Log1pParams p) {
  const int B = blockDim.x;
  const int t = threadIdx.x;
  const bool acc = p.accurate != 0;
  for (int64_t tile = blockIdx.x; tile < p.tiles; tile += gridDim.x) {
    const int64_t base = tile * (int64_t)B * E;
    const int64_t left = p.n - base;
    if (left >= (int64_t)B * E) {
      const uint32_t bytes = (uint32_t)B * E * 4u;
      const __amdgpu_buffer_rsrc_t rx = tile_rsrc(p.x + base, bytes);
      const __amdgpu_buffer_rsrc_t ro = tile_rsrc(p.out + base, bytes);
      const int off = t * E * 4;
      if constexpr (E == 1) {
        const float v = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rx, off, 0, 2));
        __builtin_amdgcn_raw_buffer_store_b32(fbits(log1p_f32_elem(v, acc)), ro, off, 0, 2);
      } else if constexpr (E == 2) {
        f32x2 v = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rx, off, 0, 2));
        v.x = log1p_f32_elem(v.x, acc);
        v.y = log1p_f32_elem(v.y, acc);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), ro, off, 0, 2);
      } else {
        f32x4 v[E / 4];
#pragma unroll
        for (int h = 0; h < E / 4; ++h)
          v[h] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off + 16 * h,
                                                                                   0, 2));
#pragma unroll
        for (int h = 0; h < E / 4; ++h) {
          f32x4 w;
          w.x = log1p_f32_elem(v[h].x, acc);
          w.y = log1p_f32_elem(v[h].y, acc);
          w.z = log1p_f32_elem(v[h].z, acc);
          w.w = log1p_f32_elem(v[h].w, acc);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w), ro, off + 16 * h,
                                                 0, 2);
        }
      }
    } else {
      for (int e = 0; e < E; ++e) {
        const int64_t i = base + (int64_t)t * E + e;
        if (i < p.n) p.out[i] = log1p_f32_elem(p.x[i], acc);
      }
    }
  }
}

template <typename K>
int64_t resident_blocks(K kernel, int block_threads) {
  int dev = 0, per_cu = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block_threads, 0) !=
      hipSuccess)
    return 0;
  return (int64_t)per_cu * cus;
}

template <int E>
hipError_t go_log1p(const Log1pParams& p, int block_threads, int64_t grid_blocks,
                    hipStream_t s) {
  if (grid_blocks == -1) grid_blocks = resident_blocks(k_log1p<E>, block_threads);
  int64_t g = grid_blocks > 0 ? grid_blocks : p.tiles;
  const int64_t cap = (int64_t)1 << 30;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  hipLaunchKernelGGL(k_log1p<E>, dim3((unsigned)g), dim3(block_threads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_log1p(float* out, const float* x, int64_t n, int block_threads,
                        int elems_per_thread, int64_t grid_blocks, bool accurate_only,
                        hipStream_t s) {
  Log1pParams p;
  p.x = x;
  p.out = out;
  p.n = n;
  const int64_t per_tile = (int64_t)block_threads * elems_per_thread;
  p.tiles = (n + per_tile - 1) / per_tile;
  p.accurate = accurate_only ? 1 : 0;
  switch (elems_per_thread) {
    case 1: return go_log1p<1>(p, block_threads, grid_blocks, s);
    case 2: return go_log1p<2>(p, block_threads, grid_blocks, s);
    case 4: return go_log1p<4>(p, block_threads, grid_blocks, s);
    case 8: return go_log1p<8>(p, block_threads, grid_blocks, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace addrms
