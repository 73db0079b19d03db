/*
 * fp32 model of the library's arithmetic contract (test code).
 *
 * The binary64 oracle defines what the fused add + RMSNorm computes; this
 * model instead follows, step by step in IEEE binary32, the exact arithmetic
 * the library documents for its kernels, so that a GPU result can be checked
 * bit for bit rather than to within one bf16 ULP:
 *   acc_j      = fl32(x_j + r_j)
 *   segment s  = elements 8s .. 8s+7:  t = acc0*acc0, then t = fmaf(acck, acck, t);
 *                the last segment of a row whose hidden is not a multiple of 8
 *                is padded with +0 (which leaves the chain unchanged)
 *   S          = balanced pairwise sum of the segment sums in index order,
 *                padded with +0 to a power of two
 *   rinv       = 1 / sqrtf(S / hidden + eps)     (correctly rounded / and sqrt)
 *   out_j      = bf16_rne((acc_j * rinv) * w_j)
 * Plain RMSNorm (r and residual_out NULL): acc_j = fp32(x_j), no addition.
 * It shares no code with the GPU library.  Plain C, gcc -O2
 * -ffp-contract=off, SSE binary32 arithmetic with the default MXCSR (no
 * flush-to-zero); fmaf from the C library (correctly rounded).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static float f32_of(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static uint32_t bits_of(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

/* Nearest-even bf16 by comparing the dropped half with one half-ULP. */
static uint16_t round_bf16(float f) {
  uint32_t u = bits_of(f);
  if (isnan(f)) return (uint16_t)((u >> 16) | 0x40);
  uint32_t hi = u >> 16, lo = u & 0xFFFF;
  if (lo > 0x8000 || (lo == 0x8000 && (hi & 1))) hi += 1;
  return (uint16_t)hi;
}

/*
 * One row's fp32 pipeline up to rinv: acc (into acc[]), residual_out, the
 * tree sum of squares (returned through *sumsq) and rinv.
 */
static float row_rinv(float* acc, float* seg, int64_t padded, uint16_t* ro, const uint16_t* xr,
                      const uint16_t* rr, int64_t hidden, float eps, float* sumsq) {
  const int64_t segs = (hidden + 7) / 8;
  for (int64_t j = 0; j < hidden; ++j) {
    acc[j] = f32_of((uint32_t)xr[j] << 16);
    if (rr) acc[j] = acc[j] + f32_of((uint32_t)rr[j] << 16);
    if (ro) ro[j] = round_bf16(acc[j]);
  }
  for (int64_t s = 0; s < padded; ++s) {
    if (s >= segs) {
      seg[s] = 0.0f;
      continue;
    }
    float a[8];
    for (int k = 0; k < 8; ++k) a[k] = 8 * s + k < hidden ? acc[8 * s + k] : 0.0f;
    float t = a[0] * a[0];
    for (int k = 1; k < 8; ++k) t = fmaf(a[k], a[k], t);
    seg[s] = t;
  }
  for (int64_t width = padded; width > 1; width /= 2)
    for (int64_t k = 0; k < width / 2; ++k) seg[k] = seg[2 * k] + seg[2 * k + 1];
  const float S = seg[0];
  if (sumsq) *sumsq = S;
  const float m = S / (float)hidden;
  const float v = m + eps;
  return 1.0f / sqrtf(v);
}

/* Returns 0, or -1 on bad arguments. */
int model_add_rmsnorm(uint16_t* out, uint16_t* residual_out, float* sumsq_out,
                      const uint16_t* x, const uint16_t* r, const uint16_t* w, int64_t n_rows,
                      int64_t hidden, float eps) {
  if (hidden <= 0 || !r != !residual_out) return -1;
  int64_t padded = 1;
  while (padded < (hidden + 7) / 8) padded *= 2;
  float* seg = (float*)malloc(sizeof(float) * (size_t)padded);
  float* acc = (float*)malloc(sizeof(float) * (size_t)hidden);
  if (!seg || !acc) {
    free(seg);
    free(acc);
    return -1;
  }
  for (int64_t i = 0; i < n_rows; ++i) {
    const float rinv = row_rinv(acc, seg, padded, residual_out ? residual_out + i * hidden : NULL,
                                x + i * hidden, r ? r + i * hidden : NULL, hidden, eps,
                                sumsq_out ? sumsq_out + i : NULL);
    for (int64_t j = 0; j < hidden; ++j) {
      const float y = (acc[j] * rinv) * f32_of((uint32_t)w[j] << 16);
      out[i * hidden + j] = round_bf16(y);
    }
  }
  free(seg);
  free(acc);
  return 0;
}

/* NaN-propagating maximum: a NaN operand wins. */
static float max_nan(float m, float v) {
  if (isnan(m)) return m;
  if (isnan(v) || v > m) return v;
  return m;
}

/*
 * Quantised out: y_j = (acc_j * rinv) * w_j in fp32 as above, then
 * amax = max |y_j| (NaN wins), scale = amax / 127, inv = 127 / amax, and
 * codes q_j = nearbyintf(y_j * inv) within [-127, 127]; a row whose amax is
 * not in [2^-120, FLT_MAX] (0, tiny, Inf or NaN) gets all-zero codes (its
 * scale is still amax / 127).
 */
int model_add_rmsnorm_quant(int8_t* q, float* scale, uint16_t* residual_out, const uint16_t* x,
                            const uint16_t* r, const uint16_t* w, int64_t n_rows, int64_t hidden,
                            float eps) {
  if (hidden <= 0 || !r != !residual_out) return -1;
  int64_t padded = 1;
  while (padded < (hidden + 7) / 8) padded *= 2;
  float* seg = (float*)malloc(sizeof(float) * (size_t)padded);
  float* acc = (float*)malloc(sizeof(float) * (size_t)hidden);
  if (!seg || !acc) {
    free(seg);
    free(acc);
    return -1;
  }
  for (int64_t i = 0; i < n_rows; ++i) {
    const float rinv = row_rinv(acc, seg, padded, residual_out ? residual_out + i * hidden : NULL,
                                x + i * hidden, r ? r + i * hidden : NULL, hidden, eps, NULL);
    float amax = 0.0f;
    for (int64_t j = 0; j < hidden; ++j) {
      acc[j] = (acc[j] * rinv) * f32_of((uint32_t)w[j] << 16);
      amax = max_nan(amax, fabsf(acc[j]));
    }
    const float sc = amax / 127.0f;
    const float inv = 127.0f / amax;
    scale[i] = sc;
    const int ok = isfinite(amax) && amax >= ldexpf(1.0f, -120);
    for (int64_t j = 0; j < hidden; ++j) {
      int8_t code = 0;
      if (ok) {
        float t = nearbyintf(acc[j] * inv);
        if (t > 127.0f) t = 127.0f;
        if (t < -127.0f) t = -127.0f;
        code = (int8_t)t;
      }
      q[i * hidden + j] = code;
    }
  }
  free(seg);
  free(acc);
  return 0;
}

/*
 * OCP FP8 E4M3 code of a finite binary32 v with |v| < 464, nearest value with
 * ties to the even code, by bit arithmetic: below 2^-6 the values are
 * multiples of 2^-9 (nearbyintf of v * 2^9, exact scaling); from 2^-6 up the
 * binary32 exponent minus 120 and the top 3 mantissa bits, rounded at the
 * 20 dropped bits.  |v| >= 464 saturates to 448 (never reached below).
 */
static uint8_t e4m3_code(float v) {
  const uint32_t sign = (bits_of(v) >> 24) & 0x80;
  const float a = fabsf(v);
  uint32_t mag;
  if (!(a < 464.0f)) {
    mag = 0x7E;
  } else if (a < 0x1p-6f) {
    mag = (uint32_t)nearbyintf(a * 512.0f);
  } else {
    uint32_t b = bits_of(a);
    b += 0x7FFFF + ((b >> 20) & 1);
    mag = (b >> 20) - (120u << 3);
  }
  return (uint8_t)(sign | mag);
}

int model_e4m3_codes(uint8_t* out, const float* v, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_code(v[i]);
  return 0;
}

/*
 * FP8 E4M3 quantised out: as model_add_rmsnorm_quant with 448 in place of
 * 127 (scale = amax / 448, inv = 448 / amax), the threshold 2^-118, and
 * codes e4m3_code(y_j * inv).
 */
int model_add_rmsnorm_quant_fp8(uint8_t* q, float* scale, uint16_t* residual_out,
                                const uint16_t* x, const uint16_t* r, const uint16_t* w,
                                int64_t n_rows, int64_t hidden, float eps) {
  if (hidden <= 0 || !r != !residual_out) return -1;
  int64_t padded = 1;
  while (padded < (hidden + 7) / 8) padded *= 2;
  float* seg = (float*)malloc(sizeof(float) * (size_t)padded);
  float* acc = (float*)malloc(sizeof(float) * (size_t)hidden);
  if (!seg || !acc) {
    free(seg);
    free(acc);
    return -1;
  }
  for (int64_t i = 0; i < n_rows; ++i) {
    const float rinv = row_rinv(acc, seg, padded, residual_out ? residual_out + i * hidden : NULL,
                                x + i * hidden, r ? r + i * hidden : NULL, hidden, eps, NULL);
    float amax = 0.0f;
    for (int64_t j = 0; j < hidden; ++j) {
      acc[j] = (acc[j] * rinv) * f32_of((uint32_t)w[j] << 16);
      amax = max_nan(amax, fabsf(acc[j]));
    }
    const float inv = 448.0f / amax;
    scale[i] = amax / 448.0f;
    const int ok = isfinite(amax) && amax >= ldexpf(1.0f, -118);
    for (int64_t j = 0; j < hidden; ++j) q[i * hidden + j] = ok ? e4m3_code(acc[j] * inv) : 0;
  }
  free(seg);
  free(acc);
  return 0;
}
