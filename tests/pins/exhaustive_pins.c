/*
 * Exhaustive pins for the CPU oracle (test code; compiled by the test suite).
 *
 * Loads the oracle library given on the command line and checks it over every
 * input of a finite domain against formulas written independently here:
 *
 *   rne   For all 2^32 fp32 bit patterns u, the oracle's fp32 -> bf16 converter
 *         must equal
 *           (a) the closed form on the halves of the word: with hi = u >> 16
 *               and lo = u & 0xFFFF, the result is hi when lo < 0x8000, hi + 1
 *               when lo > 0x8000, and hi + (hi & 1) on the tie lo == 0x8000;
 *               NaN inputs must give a NaN of the same sign;
 *           (b) a nearest-candidate choice made on real values: the two bf16
 *               neighbours of the value, their distances computed exactly in
 *               binary64, nearer one wins, a tie goes to the even pattern;
 *         and the oracle's binary64 -> bf16 converter, fed the same value
 *         widened to binary64, must agree with both.
 *
 *   sum   For all 2^32 pairs of bf16 values (x, r), the residual_out of the
 *         oracle's fused op, which rounds the fp32 sum fl32(x + r), must equal
 *         the bf16 value nearest to the exact sum x + r (IEEE rules for NaN,
 *         infinities and the sign of zero).  This pins the claim that fp32
 *         accumulation loses nothing for one addition of two bf16 values.
 *
 * Exit status 0 when every input agrees; the first mismatches are printed.
 * An optional third argument k checks only every k-th block of the domain.
 */
#include <dlfcn.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef uint16_t (*rne16_fn)(uint32_t);
typedef uint16_t (*rne16_f64_fn)(double);
typedef void (*range_fn)(uint64_t, int64_t, uint16_t*);
typedef int (*fused_fn)(uint16_t*, uint16_t*, double*, const uint16_t*, const uint16_t*,
                        const uint16_t*, int64_t, int64_t, float, int);

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
static int is_nan16(uint16_t b) { return (b & 0x7F80) == 0x7F80 && (b & 0x7F) != 0; }

/* Closed form (a). Returns 0xFFFF for "must be NaN". */
static uint32_t closed_form(uint32_t u) {
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return 0xFFFFu;
  uint32_t hi = u >> 16, lo = u & 0xFFFFu;
  if (lo < 0x8000u) return hi;
  if (lo > 0x8000u) return hi + 1;
  return hi + (hi & 1u);
}

/*
 * Nearest bf16 to a finite nonzero binary64 magnitude a, by candidates.  With
 * a in [2^(e-1), 2^e), bf16's spacing there is q = 2^(max(e-1, -126) - 7);
 * the candidates are floor(a/q)*q and the next multiple up, both bf16 values
 * (the upper one may be 2^128, where IEEE rounding decides overflow).  Their
 * distances to a are exact in binary64; the nearer wins, a tie goes to the
 * even multiple.  Returns the magnitude pattern (0x7F80 means Inf).
 */
static uint32_t nearest_mag(double a) {
  int e;
  (void)frexp(a, &e);
  int ex = e - 1 < -126 ? -126 : e - 1;
  double q = ldexp(1.0, ex - 7);
  double k = floor(a / q);
  double lo = k * q, hi = (k + 1.0) * q;
  double dl = a - lo, dh = hi - a;
  double pick;
  if (dl < dh) pick = lo;
  else if (dh < dl) pick = hi;
  else pick = fmod(k, 2.0) == 0.0 ? lo : hi;
  return bits_of((float)pick) >> 16; /* exact; 2^128 and above become Inf */
}

static uint32_t nearest_signed(double s) {
  uint32_t sign = signbit(s) ? 0x8000u : 0u;
  if (s == 0.0) return sign;
  return sign | nearest_mag(fabs(s));
}

static int run_rne(void* L, int stride) {
  range_fn range = (range_fn)dlsym(L, "orc_rne16_range");
  rne16_f64_fn from64 = (rne16_f64_fn)dlsym(L, "orc_rne16_from_f64");
  if (!range || !from64) { fprintf(stderr, "missing symbols\n"); return 2; }
  const int64_t chunk = 1 << 20;
  long long bad = 0, checked = 0;
#pragma omp parallel for schedule(dynamic) reduction(+ : bad, checked)
  for (int64_t c = 0; c < (1LL << 32) / chunk; c += stride) {
    uint16_t* got = malloc(chunk * sizeof(uint16_t));
    uint64_t start = (uint64_t)c * chunk;
    range(start, chunk, got);
    for (int64_t i = 0; i < chunk; ++i) {
      uint32_t u = (uint32_t)(start + i);
      uint32_t cf = closed_form(u);
      uint16_t g = got[i];
      uint16_t g64 = from64((double)f32_of(u));
      int ok;
      if (cf == 0xFFFFu) {
        ok = is_nan16(g) && is_nan16(g64) && ((g >> 15) == (u >> 31));
      } else {
        uint32_t nc;
        float f = f32_of(u);
        if (isinf(f)) nc = (u >> 16);
        else nc = nearest_signed((double)f);
        ok = (g == cf) && (nc == cf) && (g64 == cf);
      }
      ++checked;
      if (!ok) {
        if (bad < 10)
#pragma omp critical
          fprintf(stderr, "rne mismatch u=%08x oracle=%04x f64path=%04x closed=%04x\n",
                  u, g, g64, cf);
        ++bad;
      }
    }
    free(got);
  }
  printf("rne: checked %lld patterns, %lld mismatches\n", checked, bad);
  return bad ? 1 : 0;
}

static int run_sum(void* L, int stride) {
  fused_fn fused = (fused_fn)dlsym(L, "orc_add_rmsnorm");
  if (!fused) { fprintf(stderr, "missing symbol\n"); return 2; }
  long long bad = 0, checked = 0;
  uint16_t* xs = malloc(65536 * sizeof(uint16_t));
  uint16_t* ws = malloc(65536 * sizeof(uint16_t));
  for (uint32_t i = 0; i < 65536; ++i) { xs[i] = (uint16_t)i; ws[i] = 0x3F80; }
#pragma omp parallel for schedule(dynamic) reduction(+ : bad, checked)
  for (int r = 0; r < 65536; r += stride) {
    uint16_t* rs = malloc(65536 * sizeof(uint16_t));
    uint16_t* out = malloc(65536 * sizeof(uint16_t));
    uint16_t* ro = malloc(65536 * sizeof(uint16_t));
    for (int i = 0; i < 65536; ++i) rs[i] = (uint16_t)r;
    if (fused(out, ro, NULL, xs, rs, ws, 1, 65536, 1e-6f, 0) != 0) ++bad;
    float rf = f32_of((uint32_t)r << 16);
    for (int i = 0; i < 65536; ++i) {
      float xf = f32_of((uint32_t)i << 16);
      uint16_t g = ro[i];
      int ok;
      if (isnan(xf) || isnan(rf) || (isinf(xf) && isinf(rf) && (signbit(xf) != signbit(rf)))) {
        ok = is_nan16(g);
      } else if (isinf(xf) || isinf(rf)) {
        float inf = isinf(xf) ? xf : rf;
        ok = g == (bits_of(inf) >> 16);
      } else {
        /* Exact sum: binary64 holds it whenever the exponents are within 45
         * of each other; beyond that the smaller term is below 2^-45 of the
         * larger, whose nearest bf16 is itself either way. */
        double s = (double)xf + (double)rf;
        uint32_t e;
        if (s == 0.0) {
          /* IEEE: an exact zero sum is +0 unless both terms are -0. */
          e = (signbit(xf) && signbit(rf)) ? 0x8000u : 0u;
        } else {
          e = nearest_signed(s);
        }
        ok = g == e;
      }
      ++checked;
      if (!ok) {
        if (bad < 10)
#pragma omp critical
          fprintf(stderr, "sum mismatch x=%04x r=%04x oracle=%04x\n", i, r, g);
        ++bad;
      }
    }
    free(rs);
    free(out);
    free(ro);
  }
  free(xs);
  free(ws);
  printf("sum: checked %lld pairs, %lld mismatches\n", checked, bad);
  return bad ? 1 : 0;
}

int main(int argc, char** argv) {
  if (argc != 3 && argc != 4) {
    fprintf(stderr, "usage: %s liboracle.so rne|sum [stride]\n", argv[0]);
    return 2;
  }
  /* stride > 1 checks every stride-th block only (quick sampled runs). */
  int stride = argc == 4 ? atoi(argv[3]) : 1;
  if (stride < 1) stride = 1;
  void* L = dlopen(argv[1], RTLD_NOW);
  if (!L) { fprintf(stderr, "dlopen: %s\n", dlerror()); return 2; }
  if (!strcmp(argv[2], "rne")) return run_rne(L, stride);
  if (!strcmp(argv[2], "sum")) return run_sum(L, stride);
  fprintf(stderr, "unknown mode %s\n", argv[2]);
  return 2;
}
