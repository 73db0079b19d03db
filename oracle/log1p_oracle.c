/*
 * CPU oracle for the launch-invariant binary32 log1p (test infrastructure).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the GPU library links, includes or
 * calls this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load it.  It shares no code with the HIP path.
 *
 * The ROCm/TransformerEngine issue "CP LSE merge switches compiled variants on
 * ROCm, breaking forward reproducibility" traces a forward mismatch to an
 * elementwise binary32 log1p whose result changes with the launch shape
 * ("Root cause": a scalar and a vectorised code path about one ULP apart,
 * both within the library's 2-ULP bound).  Its "Minimal reproducer" compares
 * two launch shapes bit for bit and measures each against a binary64 log1p.
 *
 * This oracle defines the result the GPU kernel must give: ln(1 + x) for the
 * binary32 input x, rounded once to the nearest binary32, ties to even.  A
 * correctly rounded function has exactly one result per input, so no launch
 * shape, vectorisation or contraction choice can change it.
 *
 * IEEE 754 special cases of log1p: log1p(+-0) = +-0, log1p(-1) = -Inf,
 * log1p(x) = NaN for x < -1 (with -Inf), log1p(+Inf) = +Inf, NaN -> NaN.
 *
 * orc_log1p_f32: every other input is evaluated by libquadmath's log1pq in
 * binary128 (113-bit significand) and rounded once to binary32.  The binary128
 * error, about 2^-112 relative, is 2^-88 of the binary32 rounding quantum.
 *
 * orc_log1p_f32_fast: the same results, faster, for sweeps over all 2^32
 * inputs.  glibc's binary64 log1p (documented within 1 ulp of binary64, i.e.
 * 2^-52 relative) decides the rounding whenever it lies farther than 2^-36
 * relative from both binary32 midpoints around its own binary32 rounding;
 * otherwise binary128 decides, as in orc_log1p_f32.
 *
 * orc_log1p_f64: the binary64 rounding of the binary128 value, the reference
 * for ULP-error measurements (the reproducer measures against a binary64
 * log1p).
 *
 * Build: gcc -O2 -std=gnu11 -ffp-contract=off, linked with -lquadmath -lm.
 */
#include <math.h>
#include <quadmath.h>
#include <stdint.h>

/* The IEEE special cases; returns 1 and sets *r when x is one of them. */
static int special_case(float x, float* r) {
  if (isnan(x)) {
    *r = x + x; /* quiet NaN */
    return 1;
  }
  if (x == 0.0f) {
    *r = x; /* keeps the sign of zero */
    return 1;
  }
  if (x == -1.0f) {
    *r = -INFINITY;
    return 1;
  }
  if (x < -1.0f) {
    *r = NAN;
    return 1;
  }
  if (isinf(x)) {
    *r = x; /* +Inf */
    return 1;
  }
  return 0;
}

static float log1p_by_quad(float x) {
  __float128 q = log1pq((__float128)x);
  return (float)q; /* one rounding, to nearest, ties to even */
}

int orc_log1p_f32(float* out, const float* x, int64_t n) {
  if (n < 0 || (n > 0 && (!out || !x))) return -1;
  for (int64_t i = 0; i < n; ++i) {
    float r;
    if (!special_case(x[i], &r)) r = log1p_by_quad(x[i]);
    out[i] = r;
  }
  return 0;
}

int orc_log1p_f64(double* out, const float* x, int64_t n) {
  if (n < 0 || (n > 0 && (!out || !x))) return -1;
  for (int64_t i = 0; i < n; ++i) {
    float r;
    if (special_case(x[i], &r))
      out[i] = (double)r;
    else
      out[i] = (double)log1pq((__float128)x[i]);
  }
  return 0;
}

/*
 * True when the binary64 value y, known to within 2^-52 relative of the exact
 * result, lies within 2^-36 relative of a midpoint between the binary32
 * rounding r of y and one of its binary32 neighbours.  (The average of two
 * adjacent binary32 numbers is exact in binary64.)
 */
static int near_midpoint(double y, float r) {
  const double tol = ldexp(fabs(y), -36);
  const float below = nextafterf(r, -INFINITY);
  const float above = nextafterf(r, INFINITY);
  const double m_lo = ((double)r + (double)below) * 0.5;
  const double m_hi = ((double)r + (double)above) * 0.5;
  return fabs(y - m_lo) <= tol || fabs(y - m_hi) <= tol;
}

int orc_log1p_f32_fast(float* out, const float* x, int64_t n, int64_t* escalated) {
  if (n < 0 || (n > 0 && (!out || !x))) return -1;
  int64_t esc = 0;
  for (int64_t i = 0; i < n; ++i) {
    float r;
    if (!special_case(x[i], &r)) {
      const double y = log1p((double)x[i]);
      r = (float)y;
      if (isinf(r) || near_midpoint(y, r)) {
        r = log1p_by_quad(x[i]);
        ++esc;
      }
    }
    out[i] = r;
  }
  if (escalated) *escalated = esc;
  return 0;
}
