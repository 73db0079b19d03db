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
// Regular inputs are x in (-1, +Inf) with |x| > 2^-25; the others are IEEE
// special cases or round to x itself (|x| <= 2^-25: ln(1 + x) = x - x^2/2 + ...
// lies within x^2/2 <= 2^-26 |x| of x, less than half the spacing around x).
//
// Fast path, in binary64 (X = x exactly):
//   u = 1 + X, exact here: X has 24 significant bits between 2^-48 and 2^51
//       (for X >= 2^52 the rounding of u moves ln u by under 2^-58 relative).
//   u = 2^k m with m in [sqrt(1/2), sqrt(2)).
//   i = round((m - 1) * 256) in [-75, 106]; from the table, inv_i = fl(1/c_i)
//       with c_i = 1 + i/256, and -ln(inv_i).  r = m * inv_i - 1 (one fma),
//       |r| <= 2^-8.5.
//   ln(1 + X) = k ln 2 + (-ln inv_i) + log1p(r), with log1p(r) = r - r^2/2 +
//       ... + r^7/7 (the next term is below 2^-62 of r).  k ln2_hi is exact.
// The result y is within 2^-49.5 of ln(1 + X) relative (a host sweep of all
// regular inputs against glibc's log1p finds at most 2^-51).
//
// Rounding test: the binary32 rounding of y drops the low 29 of y's 52
// fraction bits; y is within 128 binary64 ulps (at least 2^-46 |y|) of a
// binary32 midpoint exactly when those bits are within 128 of 2^28.  Outside
// that window the exact value rounds like y.  Inside it (about one input in
// two million) the accurate path decides.
//
// Accurate path: the same steps in double-double arithmetic (unevaluated sums
// hi + lo with |lo| <= ulp(hi) / 2; Knuth's two-sum and the fma two-product),
// with m * inv_i - 1 held exactly, -ln(inv_i) in two parts, log1p(r) to r^13
// and ln 2 in three parts: about 2^-100 relative.  The double-double result
// is rounded to binary32 by comparing its distance from the nearest binary32
// with half the spacing on that side.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"
#include "log1p_table.h"

namespace addrms {
namespace {

#define DEV __device__ __forceinline__

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

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
// fma(m, 256, ROUND_MAGIC) = 1.5 * 2^52 + round((m - 1) * 256): the low word
// of the result is that integer (two's complement).
constexpr double ROUND_MAGIC = 0x1.8p52 - 256.0;

DEV uint32_t fbits(float v) { return __builtin_bit_cast(uint32_t, v); }
DEV float ffrom(uint32_t b) { return __builtin_bit_cast(float, b); }
DEV uint32_t low_word(double v) { return (uint32_t)__builtin_bit_cast(uint64_t, v); }

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

// Table row of m: round((m - 1) * 256) - LOG1P_TABLE_MIN, in [0, 181].
DEV int table_row(double m) {
  return (int)low_word(__builtin_fma(m, 256.0, ROUND_MAGIC)) - LOG1P_TABLE_MIN;
}

// ---------------------------------------------------------------- fast path

// ln(1 + X) in binary64 for a regular X; inv_t = {inv_i, t_hi} of the row.
// `row` receives the table row for the accurate path.
template <typename Table>
DEV double log1p_fast(double X, const Table& tab, int* row) {
  const double u = X + 1.0;
  int k;
  const double m = reduce(u, &k);
  *row = table_row(m);
  const f64x2 it = tab(*row);
  const double r = __builtin_fma(m, it.x, -1.0);
  // log1p(r) = r + r^2 (-1/2 + r/3 - r^2/4 + r^3/5 - r^4/6 + r^5/7)
  double P = 1.0 / 7.0;
  P = __builtin_fma(P, r, -1.0 / 6.0);
  P = __builtin_fma(P, r, 1.0 / 5.0);
  P = __builtin_fma(P, r, -1.0 / 4.0);
  P = __builtin_fma(P, r, 1.0 / 3.0);
  P = __builtin_fma(P, r, -0.5);
  const double L = __builtin_fma(r * r, P, r);
  const double kd = (double)k;
  const double A = __builtin_fma(kd, LN2_LO, L);
  const double B = it.y + A;
  return __builtin_fma(kd, LN2_HI, B);
}

// True when y lies within 128 binary64 ulps of a binary32 rounding midpoint
// (y in the binary32 normal range).
DEV bool near_midpoint(double y) {
  const int32_t d = (int32_t)(low_word(y) & 0x1FFFFFFFu) - 0x10000000;
  return d <= 128 && d >= -128;
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

// (-1)^(n+1) / n as a double-double: hi = fl(1/n), lo = fl((1 - hi n) / n),
// the residual 1 - hi n exact by fma.
DEV dd series_coef(int n) {
  const double nd = (double)n;
  const double hi = 1.0 / nd;
  const dd c = {hi, __builtin_fma(-hi, nd, 1.0) / nd};
  return (n & 1) ? c : dd{-c.hi, -c.lo};
}

// ln(1 + X) as a double-double for a regular X, about 2^-100 relative.
DEV dd log1p_accurate(double X) {
  const dd U = two_sum(1.0, X);  // exactly 1 + X
  int k;
  const double mh = reduce(U.hi, &k);
  const double ml = __builtin_amdgcn_ldexp(U.lo, -k);
  const double* e = log1p_table[table_row(mh)];
  const double inv = e[0];
  // R = m * inv - 1: the product exactly, p - 1 exact (p within 2^-8 of 1)
  dd p = two_prod(mh, inv);
  p.lo = __builtin_fma(ml, inv, p.lo);
  const dd R = two_sum(p.hi - 1.0, p.lo);
  // log1p(R) = R * sum_{n=1}^{13} (-1)^(n+1) R^(n-1) / n, by Horner
  dd Q = series_coef(13);
  for (int n = 12; n >= 1; --n) Q = dd_add(dd_mul(Q, R), series_coef(n));
  const dd L = dd_mul(Q, R);
  const dd T = {e[1], e[2]};
  const double kd = (double)k;
  const dd K = dd_add(two_sum(kd * LN2_P1, kd * LN2_P2), dd{kd * LN2_P3, 0.0});
  return dd_add(K, dd_add(T, L));
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

// The accurate path, correctly rounded to binary32.
DEV float log1p_accurate_f32(double X) {
  return round_dd_to_f32(log1p_accurate(X));
}

// ---------------------------------------------------------------- one element

// The result of a non-regular x: NaN -> quiet NaN, |x| <= 2^-25 (with +-0)
// -> x, -1 -> -Inf, x < -1 -> NaN, +Inf -> +Inf.  Selects, no branches.
DEV float log1p_irregular(float x) {
  const float below = x == -1.0f ? -__builtin_inff() : __builtin_nanf("");
  const float v = x < -1.0f || x == -1.0f ? below : x;  // tiny, +Inf
  return x != x ? x + x : v;
}

DEV bool is_regular(float x) {
  return x > -1.0f && x < __builtin_inff() && __builtin_fabsf(x) > 0x1p-25f;  // NaN fails
}

// log1p of E elements in place.  The fast path of all E runs first, with no
// branch or call between them so that their instructions interleave; the
// rare elements whose rounding it cannot settle (or all, when `accurate`)
// are then recomputed by the accurate path.
template <int E, typename Table>
DEV void log1p_f32_vec(float (&v)[E], bool accurate, const Table& tab) {
  double y[E];
  bool reg[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    reg[e] = is_regular(v[e]);
    int row;
    y[e] = log1p_fast(reg[e] ? (double)v[e] : 0.5, tab, &row);
  }
  bool any = false;
#pragma unroll
  for (int e = 0; e < E; ++e) any = any || (reg[e] && (accurate || near_midpoint(y[e])));
  float r[E];
#pragma unroll
  for (int e = 0; e < E; ++e) r[e] = (float)y[e];
  if (any) {
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (reg[e] && (accurate || near_midpoint(y[e]))) r[e] = log1p_accurate_f32((double)v[e]);
  }
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] = reg[e] ? r[e] : log1p_irregular(v[e]);
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

// {inv_i, t_hi} rows of the table, staged in LDS once per workgroup.
struct LdsTable {
  const f64x2* rows;
  DEV f64x2 operator()(int row) const { return rows[row]; }
};

// E consecutive elements per thread, blockDim.x * E per tile; workgroups loop
// over tiles.  Full tiles use E-wide nontemporal buffer loads and stores;
// the last, partial tile goes element by element with a bounds check.
template <int E>
__global__ __launch_bounds__(1024) void k_log1p(Log1pParams p) {
  __shared__ f64x2 rows[LOG1P_TABLE_SIZE];
  const int B = blockDim.x;
  const int t = threadIdx.x;
  for (int i = t; i < LOG1P_TABLE_SIZE; i += B)
    rows[i] = f64x2{log1p_table[i][0], log1p_table[i][1]};
  __syncthreads();
  const LdsTable tab{rows};
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
        float v[1] = {__builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rx, off, 0, 2))};
        log1p_f32_vec(v, acc, tab);
        __builtin_amdgcn_raw_buffer_store_b32(fbits(v[0]), ro, off, 0, 2);
      } else if constexpr (E == 2) {
        const f32x2 q = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rx, off, 0, 2));
        float v[2] = {q.x, q.y};
        log1p_f32_vec(v, acc, tab);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, f32x2{v[0], v[1]}), ro, off,
                                              0, 2);
      } else {
        float v[E];
#pragma unroll
        for (int h = 0; h < E / 4; ++h) {
          const f32x4 q = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off + 16 * h, 0, 2));
          v[4 * h] = q.x;
          v[4 * h + 1] = q.y;
          v[4 * h + 2] = q.z;
          v[4 * h + 3] = q.w;
        }
        log1p_f32_vec(v, acc, tab);
#pragma unroll
        for (int h = 0; h < E / 4; ++h) {
          const f32x4 w = {v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w), ro, off + 16 * h,
                                                 0, 2);
        }
      }
    } else {
      for (int e = 0; e < E; ++e) {
        const int64_t i = base + (int64_t)t * E + e;
        if (i < p.n) {
          float v[1] = {p.x[i]};
          log1p_f32_vec(v, acc, tab);
          p.out[i] = v[0];
        }
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

// Default grid cap of the log1p kernel (measured on MI355X at 2^26 inputs:
// 8192 workgroups of 256 threads beat one workgroup per tile by 21%).
constexpr int64_t kLog1pMaxGrid = 8192;

template <int E>
hipError_t go_log1p(const Log1pParams& p, int block_threads, int64_t grid_blocks,
                    hipStream_t s) {
  if (grid_blocks == -1) grid_blocks = resident_blocks(k_log1p<E>, block_threads);
  // By default at most kLog1pMaxGrid workgroups, each looping over tiles:
  // the table is staged once per workgroup, not once per tile.
  int64_t g = grid_blocks > 0 ? grid_blocks : (p.tiles < kLog1pMaxGrid ? p.tiles : kLog1pMaxGrid);
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
