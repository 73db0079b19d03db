// Kernels of the fused residual-add + RMSNorm forward for gfx950 (MI355X).
//
// The operation is the reference() of the ROCm/aiter issue
// "rmsnorm2d_fwd_with_add truncates fp32->bf16 on gfx942, biasing
// residual_out and compounding across layers" ("Steps to Reproduce"), with
// both bf16 stores rounded to nearest, ties to even, as its "Cost of fixing"
// section asks for residual_out and as this library does for out too.
//
// Numerics shared by all three kernels (so that every path and every launch
// shape produces the same bits):
//   * bf16 -> fp32 widening is a 16-bit shift (exact).
//   * acc = x + r is one IEEE fp32 add per element.
//   * Both stores go through v_cvt_pk_bf16_f32, gfx950's packed fp32 -> bf16
//     conversion, which rounds to nearest-even under the default MODE and
//     keeps NaN a NaN (the aiter issue's Notes: on gfx942 the library's
//     fallback truncated; gfx950 has the instruction).
//   * The sum of squares follows one fixed tree that depends on hidden only.
//     A segment is 8 consecutive elements (one 16-byte load); its sum is
//     t = a0*a0, then t = fma(ak, ak, t) for k = 1..7.  Segment sums are then
//     added by a balanced pairwise tree in index order, padded with +0 to a
//     power of two.  Every subtree is an aligned block of segments, so a
//     wavefront that holds 64 consecutive segments (one per lane) computes
//     that block's subtree with a butterfly, and the block sums finish the
//     tree in registers or through LDS, whatever the workgroup size.  Padding
//     with more +0 leaves the result unchanged (x + 0 = x for the non-negative
//     partial sums), so the tree is the same for every padded size.
//   * rinv = 1 / sqrt(S / hidden + eps) with correctly rounded fp32 division
//     and square root (HIP's defaults; no fast-math), once per row.
//   * y = (acc * rinv) * w: two fp32 multiplies in that order; no contraction
//     (built with -ffp-contract=off).
//   * Quantised variant (template flag Q): instead of bf16 out, per-row int8
//     codes and an fp32 scale.  amax = max |y| over the row (a maximum is
//     exact, so its order is free; a NaN wins), scale = amax / 127 and
//     inv = 127 / amax (each correctly rounded, once per row), and
//     q = y * inv rounded to the nearest integer, ties to even, within
//     [-127, 127].  The inverse must be finite, so a row is quantised only
//     when 2^-120 <= amax <= FLT_MAX; other rows (amax 0, tiny, Inf or NaN)
//     get all-zero codes, and their scale is still amax / 127.
//     The same with OCP FP8 E4M3 codes (Q = 2): 448 (E4M3's largest finite
//     value) in place of 127, threshold 2^-118, and the code of y * inv is
//     its nearest E4M3 value, ties to even, from gfx950's packed fp32 -> fp8
//     conversion (v_cvt_pk_fp8_f32, OCP formats on this architecture).
//     |y * inv| <= 448 (1 + 2^-23) always rounds to at most 448, so no code
//     is NaN.
//   * Plain variant (template flag R false): RMSNorm without the residual
//     add.  acc = x exactly (no add at all: adding a zero would turn -0 into
//     +0), and there is no residual_out; everything after acc is the same.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <mutex>

#include "launch.h"

namespace addrms {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

#define DEV __device__ __forceinline__

struct Params {
  u32x4* out;           // bf16 out (plain variant)
  u32x2* qout;          // 1-byte codes, 8 per segment (quantised variants)
  float* qscale;        // per-row scale (quantised variant)
  u32x4* residual_out;
  const u32x4* x;
  const u32x4* residual;
  const u32x4* weight;
  int64_t n_rows;
  // Row strides, in 16-byte segments (the codes of the quantised variant are
  // always contiguous: C segments of 8 bytes per row).
  int64_t x_stride, r_stride, out_stride, ro_stride;
  int32_t segs;  // hidden / 8
  float hidden_f;
  float eps;
};

// ---------------------------------------------------------------- memory

// Streaming loads and stores: every byte of x, residual, out and residual_out
// is touched once, so they bypass cache retention (nontemporal).  The weight
// is re-read by every row and uses ordinary cached loads.
DEV u32x4 load_stream(const u32x4* p) { return __builtin_nontemporal_load(p); }
DEV void store_stream(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

// Buffer resource over one row of a tensor (row `row`, `stride` segments
// apart, `segs` segments long): offsets stay 32-bit whatever the tensor size,
// and the hardware range check (reads past num_records return 0) lets a
// prefetch run without a branch.  An unused tensor gets num_records = 0.  The
// last word selects 32-bit raw data (gfx9 layout).
DEV __amdgpu_buffer_rsrc_t row_rsrc(const u32x4* t, int64_t row, int64_t stride, int segs,
                                    bool valid) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4*>(t) + (valid ? row * stride : 0), 0,
                                           valid ? segs * 16 : 0, 0x00020000);
}

// Nontemporal (aux bit 1) 16-byte load of segment s through a row resource.
DEV u32x4 load_seg(__amdgpu_buffer_rsrc_t r, int s) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, s * 16, 0, 2);
}

// Nontemporal 16-byte store of segment s; stores past the row are dropped.
DEV void store_seg(__amdgpu_buffer_rsrc_t r, int s, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, s * 16, 0, 2);
}

// The same for a row of int8 codes (8 bytes per segment).
DEV __amdgpu_buffer_rsrc_t code_row_rsrc(u32x2* t, int64_t row, int segs) {
  return __builtin_amdgcn_make_buffer_rsrc(t + row * segs, 0, segs * 8, 0x00020000);
}
DEV void store_codes(__amdgpu_buffer_rsrc_t r, int s, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, s * 8, 0, 2);
}
DEV void store_codes_stream(u32x2* p, u32x2 v) { __builtin_nontemporal_store(v, p); }

// ---------------------------------------------------------------- numerics

DEV void unpack8(u32x4 q, float (&a)[8]) {
  a[0] = __builtin_bit_cast(float, q.x << 16);
  a[1] = __builtin_bit_cast(float, q.x & 0xFFFF0000u);
  a[2] = __builtin_bit_cast(float, q.y << 16);
  a[3] = __builtin_bit_cast(float, q.y & 0xFFFF0000u);
  a[4] = __builtin_bit_cast(float, q.z << 16);
  a[5] = __builtin_bit_cast(float, q.z & 0xFFFF0000u);
  a[6] = __builtin_bit_cast(float, q.w << 16);
  a[7] = __builtin_bit_cast(float, q.w & 0xFFFF0000u);
}

// Two fp32 values -> two bf16 in one word (first value in the low half), by
// the hardware's packed round-to-nearest-even conversion.
DEV uint32_t pack2_rne(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

DEV u32x4 pack8_rne(const float (&a)[8]) {
  u32x4 q;
  q.x = pack2_rne(a[0], a[1]);
  q.y = pack2_rne(a[2], a[3]);
  q.z = pack2_rne(a[4], a[5]);
  q.w = pack2_rne(a[6], a[7]);
  return q;
}

// Sum of squares of one segment, in element order.
DEV float seg_sumsq(const float (&a)[8]) {
  float t = a[0] * a[0];
#pragma unroll
  for (int k = 1; k < 8; ++k) t = __builtin_fmaf(a[k], a[k], t);
  return t;
}

// Row maxima of |y| are taken on bit patterns.  With the sign bit cleared,
// unsigned integer order is the numeric order of binary32 values, and every
// NaN pattern lies above +Inf, so a NaN anywhere makes the maximum a NaN.  An
// integer maximum is exact and order-free, NaN payloads included; it costs an
// AND and a max per element where a NaN-aware float maximum costs compares
// and selects.
DEV uint32_t abs_bits(float v) { return __builtin_bit_cast(uint32_t, v) & 0x7FFFFFFFu; }
DEV uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Cross-lane moves.  Each level adds two aligned sibling sub-blocks; once a
// sub-block holds one value in all its lanes, a mirror within the enclosing
// block reaches the sibling just as an xor would.
#define ADDRMS_DPP(v, ctrl) \
  __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, (v)), (ctrl), 0xF, 0xF, false))

// Sum of the 64 lanes' values as a balanced pairwise tree over lane index:
// (0,1) (2,3) ..., then aligned 4s, 8s, 16s, 32s, 64.  Returns the same bits
// in every lane.  Must be called with all 64 lanes active.
DEV float wave_block_sum(float v) {
  v = v + ADDRMS_DPP(v, 0xB1);   // quad_perm [1,0,3,2]: lane ^ 1
  v = v + ADDRMS_DPP(v, 0x4E);   // quad_perm [2,3,0,1]: lane ^ 2
  v = v + ADDRMS_DPP(v, 0x141);  // row_half_mirror: the other quad of the 8
  v = v + ADDRMS_DPP(v, 0x140);  // row_mirror: the other 8 of the 16
  // ds_swizzle, bit-mask mode (and 0x1F, or 0, xor 0x10): lane ^ 16 within 32.
  v = v + __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
  float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  return lo + hi;
}

// Unsigned maximum over the 64 lanes; the same in every lane.  Must be
// called with all 64 lanes active.
#define ADDRMS_DPP_U(v, ctrl) (uint32_t) __builtin_amdgcn_mov_dpp((int)(v), (ctrl), 0xF, 0xF, false)
DEV uint32_t wave_max(uint32_t v) {
  v = umax(v, ADDRMS_DPP_U(v, 0xB1));
  v = umax(v, ADDRMS_DPP_U(v, 0x4E));
  v = umax(v, ADDRMS_DPP_U(v, 0x141));
  v = umax(v, ADDRMS_DPP_U(v, 0x140));
  v = umax(v, (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F));
  return umax((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
              (uint32_t)__builtin_amdgcn_readlane((int)v, 32));
}

// Balanced pairwise tree over N (a power of two) values in index order.
template <int N>
DEV float pairwise_tree(float (&v)[N]) {
#pragma unroll
  for (int n = N; n > 1; n >>= 1) {
#pragma unroll
    for (int i = 0; i < n / 2; ++i) v[i] = v[2 * i] + v[2 * i + 1];
  }
  return v[0];
}

template <int N>
DEV float pairwise_tree_lds(const float* b) {
  float v[N];
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = b[i];
  return pairwise_tree<N>(v);
}

DEV float row_rinv(float sumsq, const Params& p) {
  return 1.0f / __builtin_sqrtf(sumsq / p.hidden_f + p.eps);
}

// y = (acc * rinv) * w for one segment.
DEV void scale8(const float (&acc)[8], float rinv, u32x4 wq, float (&y)[8]) {
  float w[8];
  unpack8(wq, w);
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = (acc[k] * rinv) * w[k];
}

// out = bf16((acc * rinv) * w) for one segment.
DEV u32x4 normalise8(const float (&acc)[8], float rinv, u32x4 wq) {
  float y[8];
  scale8(acc, rinv, wq, y);
  return pack8_rne(y);
}

// Running maximum of |y| over a segment, as bit patterns.
DEV uint32_t max_abs8(uint32_t m, const float (&y)[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) m = umax(m, abs_bits(y[k]));
  return m;
}

// Code formats of the quantised variants (template parameter Q): 1 int8,
// 2 OCP FP8 E4M3; 0 is the bf16-out variant.  Codes are bytes either way.
constexpr int kQInt8 = 1;
constexpr int kQFp8 = 2;

// The largest code magnitude: scale = amax / qmax, inv = qmax / amax.
template <int Q>
constexpr float qmax() {
  return Q == kQInt8 ? 127.0f : 448.0f;
}

// Whether a row's codes are taken from y * inv: qmax / amax must be finite,
// so 2^-120 (int8) or 2^-118 (E4M3) <= amax <= FLT_MAX (false for NaN).
template <int Q>
DEV bool quantisable(float amax) {
  return amax >= (Q == kQInt8 ? 0x1p-120f : 0x1p-118f) && amax <= 3.40282347e38f;
}

// Codes of one segment, for a quantisable row (|y| <= amax, so |y * inv| <=
// qmax (1 + 2^-24)^2 < qmax + 1/2).
//   int8: the nearest-even integer of t = y * inv, which is within [-127, 127]
//   by the bound above.  t + 1.5 * 2^23 lies in [2^23, 2^24), where binary32
//   steps by 1, so the add rounds t to the nearest integer n (ties to even,
//   the default mode) and the sum's bit pattern is 0x4B400000 + n: its low
//   byte is n's two's complement.  v_perm_b32 gathers four such bytes per word.
//   E4M3: the packed conversion of y * inv, two values per instruction.
template <int Q>
DEV u32x2 quant8(const float (&y)[8], float inv) {
  if constexpr (Q == kQInt8) {
    uint32_t g[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) g[k] = __builtin_bit_cast(uint32_t, y[k] * inv + 0x1.8p23f);
    const uint32_t a = __builtin_amdgcn_perm(g[1], g[0], 0x0C0C0400u);  // bytes g0, g1
    const uint32_t b = __builtin_amdgcn_perm(g[3], g[2], 0x0C0C0400u);  // bytes g2, g3
    const uint32_t c = __builtin_amdgcn_perm(g[5], g[4], 0x0C0C0400u);
    const uint32_t d = __builtin_amdgcn_perm(g[7], g[6], 0x0C0C0400u);
    return u32x2{__builtin_amdgcn_perm(b, a, 0x05040100u), __builtin_amdgcn_perm(d, c, 0x05040100u)};
  } else {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = y[k] * inv;
    uint32_t w0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
    w0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], (int)w0, true);
    uint32_t w1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false);
    w1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], (int)w1, true);
    return u32x2{w0, w1};
  }
}

// acc = x + r for one segment (acc = x in the plain variant), without the
// sum of squares.
template <bool R>
DEV void add8(u32x4 xq, u32x4 rq, float (&acc)[8]) {
  if constexpr (R) {
    float xa[8], ra[8];
    unpack8(xq, xa);
    unpack8(rq, ra);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = xa[k] + ra[k];
  } else {
    unpack8(xq, acc);
  }
}

// Hides a value from the optimiser.  The wavefront-per-row kernel keeps x and
// residual in their packed bf16 form across the reduction and adds them again
// afterwards (the same fp32 add, so the same bits): half the registers of
// keeping the fp32 sums.  Without this the compiler would merge the two adds
// and keep the sums live, or hoist loop-invariant LDS reads into registers.
template <typename T>
DEV T opaque(T v) {
  asm volatile("" : "+v"(v));
  return v;
}

// acc = x + r for one segment (acc = x in the plain variant); returns its
// sum of squares.
template <bool R>
DEV float add_segment(u32x4 xq, u32x4 rq, float (&acc)[8]) {
  add8<R>(xq, rq, acc);
  return seg_sumsq(acc);
}

// ---------------------------------------------------------------- wave per row

// WAVES rows per workgroup, one per wavefront; lane l holds segments
// l, l + 64, ..., l + 64 (J - 1).  Block j of 64 segments is summed by one
// butterfly; the J block sums finish the tree in registers.  The weight is
// staged once per workgroup in LDS (the waves share it), which keeps the
// per-lane register footprint small enough for more rows in flight per CU.
// Rows are read and written through per-row buffer resources: segments past
// the row read as zero and their stores are dropped, so nothing branches.
template <int WAVES, int J, int Q, bool R>
__global__ __launch_bounds__(WAVES * 64) void k_wave_row(Params p) {
  __shared__ u32x4 wl[64 * J];
  const int lane = threadIdx.x & 63;
  // The wave index is the same in all 64 lanes; saying so keeps the row and
  // its buffer resources in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int C = p.segs;
  for (int i = threadIdx.x; i < 64 * J; i += WAVES * 64)
    wl[i] = i < C ? p.weight[i] : u32x4{0, 0, 0, 0};
  __syncthreads();

  const int64_t stride = (int64_t)gridDim.x * WAVES;
  for (int64_t row = (int64_t)blockIdx.x * WAVES + wave; row < p.n_rows; row += stride) {
    const __amdgpu_buffer_rsrc_t rx = row_rsrc(p.x, row, p.x_stride, C, true);
    const __amdgpu_buffer_rsrc_t rr = row_rsrc(p.residual, row, p.r_stride, C, R);
    const __amdgpu_buffer_rsrc_t ro = row_rsrc(p.residual_out, row, p.ro_stride, C, R);
    const __amdgpu_buffer_rsrc_t oo = row_rsrc(p.out, row, p.out_stride, C, !Q);
    u32x4 xq[J], rq[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      xq[j] = load_seg(rx, lane + 64 * j);
      rq[j] = R ? load_seg(rr, lane + 64 * j) : u32x4{0, 0, 0, 0};
    }
    float blk[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      float acc[8];
      blk[j] = add_segment<R>(xq[j], rq[j], acc);
      if constexpr (R) store_seg(ro, lane + 64 * j, pack8_rne(acc));
    }
#pragma unroll
    for (int j = 0; j < J; ++j) blk[j] = wave_block_sum(blk[j]);
    const float rinv = row_rinv(pairwise_tree<J>(blk), p);
    if constexpr (!Q) {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        float acc[8];
        add8<R>(opaque(xq[j]), opaque(rq[j]), acc);
        store_seg(oo, lane + 64 * j, normalise8(acc, rinv, wl[opaque(lane + 64 * j)]));
      }
    } else {
      // y twice (the same fp32 operations, so the same values): once for the
      // row maximum, once for the codes.
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        float acc[8], y[8];
        add8<R>(opaque(xq[j]), opaque(rq[j]), acc);
        scale8(acc, rinv, wl[opaque(lane + 64 * j)], y);
        if (lane + 64 * j < C) m = max_abs8(m, y);
      }
      const float amax = __builtin_bit_cast(float, wave_max(m));
      const float scale = amax / qmax<Q>();
      const float inv = qmax<Q>() / amax;
      const bool ok = quantisable<Q>(amax);
      if (lane == 0) p.qscale[row] = scale;
      const __amdgpu_buffer_rsrc_t qo = code_row_rsrc(p.qout, row, C);
#pragma unroll
      for (int j = 0; j < J; ++j) {
        float acc[8], y[8];
        add8<R>(opaque(xq[j]), opaque(rq[j]), acc);
        scale8(acc, rinv, wl[opaque(lane + 64 * j)], y);
        store_codes(qo, lane + 64 * j, ok ? quant8<Q>(y, inv) : u32x2{0, 0});
      }
    }
  }
}

// ---------------------------------------------------------------- workgroup per row

// B threads per row; thread t holds segments t, t + B, ..., t + B (J - 1).
// For each j, wave w's butterfly yields the sum of block w + j * (B / 64);
// the B / 64 * J block sums meet in LDS and every thread finishes the tree.
// L (bf16 out only): the weight is not held in registers from the start but
// read again for each row after the row's barrier, where the out stores need
// it.  Measured on MI355X with one small workgroup per row (x and residual
// together at most 64 MiB): 4-14% faster than holding it, as the row's
// stores then follow its loads later (2048 x 4096: 12.0 against 13.1 us).
template <int B, int J, int Q, bool R, bool L, bool FB = false>
__global__ __launch_bounds__(B) void k_wg_row(Params p) {
  static_assert(!L || Q == 0, "the late weight read is built for bf16 out only");
  constexpr int W = B / 64;
  constexpr int NB = W * J;
  __shared__ float blk[2][NB];  // alternates by row so one barrier per row suffices
  __shared__ uint32_t mx[2][Q ? W : 1];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int C = p.segs;

  // A small call (the late-weight form) has nearly all its rows resident at
  // once: its waves issue their loads at raised priority, ahead of waves
  // already past their row's barrier, and drop it at the barrier (measured on
  // MI355X: 1-2.5% faster from 1024 x 4096 to 4096 x 4096, 1% slower at
  // 2048 x 2048; the same on a large call was 2-3% slower).
  if constexpr (L) __builtin_amdgcn_s_setprio(3);
  u32x4 wq[L ? 1 : J];
  if constexpr (!L) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int s = t + B * j;
      wq[j] = s < C ? p.weight[s] : u32x4{0, 0, 0, 0};
    }
  }

  // Plain quantised rows, and fused bf16 rows whose segments fill every
  // thread's J slots (FB), are read and written through per-row buffer
  // resources, as in k_wave_row: segments past the row read as zero and
  // their stores are dropped, so nothing branches on the row's end.
  // Measured on MI355X: 1-4% faster for plain quantised rows; for FB rows
  // the same at 4096 x 8192, 23.46 -> 22.68 us at 4096 x 4096, 12.06 ->
  // 11.94 us at 2048 x 4096, 7.17 -> 7.01 us at 1024 x 4096; for every fused
  // bf16 row, 5% slower at 4096 x 2560, where 37% of the slots lie past the
  // row (hence FB).  The
  // other forms use bounds-checked pointer accesses (measured 2% faster for
  // plain bf16).
  constexpr bool BUF = (Q != 0 && !R) || FB;
  int parity = 0;
  for (int64_t row = blockIdx.x; row < p.n_rows; row += gridDim.x, parity ^= 1) {
    u32x4 xq[J], rq[J];
    if constexpr (BUF) {
      const __amdgpu_buffer_rsrc_t rx = row_rsrc(p.x, row, p.x_stride, C, true);
      const __amdgpu_buffer_rsrc_t rr = row_rsrc(p.residual, row, p.r_stride, C, R);
#pragma unroll
      for (int j = 0; j < J; ++j) {
        xq[j] = load_seg(rx, t + B * j);
        rq[j] = R ? load_seg(rr, t + B * j) : u32x4{0, 0, 0, 0};
      }
    } else {
      const u32x4* xr = p.x + row * p.x_stride;
      const u32x4* rr = p.residual + (R ? row * p.r_stride : 0);
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int s = t + B * j;
        if (s < C) {
          xq[j] = load_stream(xr + s);
          rq[j] = R ? load_stream(rr + s) : u32x4{0, 0, 0, 0};
        } else {
          xq[j] = u32x4{0, 0, 0, 0};
          rq[j] = u32x4{0, 0, 0, 0};
        }
      }
    }
    float acc[J][8];
    float bs[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int s = t + B * j;
      bs[j] = add_segment<R>(xq[j], rq[j], acc[j]);
      if constexpr (R && BUF)
        store_seg(row_rsrc(p.residual_out, row, p.ro_stride, C, true), s, pack8_rne(acc[j]));
      else if (R && s < C)
        store_stream(p.residual_out + row * p.ro_stride + s, pack8_rne(acc[j]));
    }
#pragma unroll
    for (int j = 0; j < J; ++j) bs[j] = wave_block_sum(bs[j]);
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < J; ++j) blk[parity][wave + W * j] = bs[j];
    }
    if constexpr (L) __builtin_amdgcn_s_setprio(0);
    __syncthreads();
    const float rinv = row_rinv(pairwise_tree_lds<NB>(blk[parity]), p);
    if constexpr (!Q && BUF) {
      const __amdgpu_buffer_rsrc_t ro = row_rsrc(p.out, row, p.out_stride, C, true);
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int s = t + B * j;
        store_seg(ro, s, normalise8(acc[j], rinv, L ? p.weight[s < C ? s : 0] : wq[L ? 0 : j]));
      }
    } else if constexpr (!Q) {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int s = t + B * j;
        if (s < C)
          store_stream(p.out + row * p.out_stride + s,
                       normalise8(acc[j], rinv, L ? p.weight[s] : wq[L ? 0 : j]));
      }
    } else {
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        float y[8];
        scale8(acc[j], rinv, wq[L ? 0 : j], y);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[j][k] = y[k];
        if (t + B * j < C) m = max_abs8(m, y);
      }
      m = wave_max(m);
      if (lane == 0) mx[parity][wave] = m;
      __syncthreads();
      uint32_t mb = mx[parity][0];
#pragma unroll
      for (int i = 1; i < W; ++i) mb = umax(mb, mx[parity][i]);
      const float amax = __builtin_bit_cast(float, mb);
      const float scale = amax / qmax<Q>();
      const float inv = qmax<Q>() / amax;
      const bool ok = quantisable<Q>(amax);
      if (t == 0) p.qscale[row] = scale;
      if constexpr (BUF) {
        const __amdgpu_buffer_rsrc_t qo = code_row_rsrc(p.qout, row, C);
#pragma unroll
        for (int j = 0; j < J; ++j)
          store_codes(qo, t + B * j, ok ? quant8<Q>(acc[j], inv) : u32x2{0, 0});
      } else {
        const size_t base = (size_t)row * (size_t)C;
#pragma unroll
        for (int j = 0; j < J; ++j) {
          const int s = t + B * j;
          if (s < C) store_codes_stream(p.qout + base + s, ok ? quant8<Q>(acc[j], inv) : u32x2{0, 0});
        }
      }
    }
  }
}

// ---------------------------------------------------------------- LDS two-pass

// B threads per row.  Pass 1 walks the row in chunks of B segments: acc,
// residual_out, the segment's fp32 values staged in LDS (two planes of
// 16 bytes per segment, so a wavefront's accesses are contiguous), and one
// block sum per wave per chunk.  After one barrier every thread finishes the
// tree over NB padded block sums; pass 2 reads the staged values back (each
// thread only its own, so the staging needs no barrier of its own) and writes
// out.  The block sums (and the quantised variants' maxima) alternate by row
// parity, so one barrier per row suffices.
// Pass 1 issues the loads of U chunks at once before processing them, so
// each wavefront keeps U chunks of x and residual in flight.  Loads and the
// bf16 stores go through per-row buffer resources: segments past the row read
// as zero and their stores are dropped, without a branch.  The weight of the
// first U chunks is read once per workgroup, before its first row, into
// registers; further chunks read it in pass 2.  (Measured on MI355X at 2048 x 16384 against the weight read in
// pass 2 and a second barrier per row: 45.9 against 47.6 us.)
template <int B, int NB, int U, int Q, bool R>
__global__ __launch_bounds__(B) void k_lds_two_pass(Params p) {
  constexpr int W = B / 64;
  __shared__ float blk[2][NB];
  __shared__ uint32_t mx[2][Q ? W : 1];
  extern __shared__ float4 stage[];  // [2][C]: elements 0-3, then 4-7, of each segment
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int C = p.segs;
  const int chunks = (C + B - 1) / B;
  float4* lo = stage;
  float4* hi = stage + C;

  u32x4 wq[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int s = u * B + t;
    wq[u] = s < C ? p.weight[s] : u32x4{0, 0, 0, 0};
  }
  // Blocks past the row's last chunk are +0, in both parities; rows never
  // write them.  The first row's barrier orders these stores before any read.
  for (int i = t; i < 2 * NB; i += B)
    if (i % NB >= chunks * W) blk[i / NB][i % NB] = 0.0f;

  int parity = 0;
  for (int64_t row = blockIdx.x; row < p.n_rows; row += gridDim.x, parity ^= 1) {
    const size_t base = (size_t)row * (size_t)C;  // the codes
    const __amdgpu_buffer_rsrc_t rx = row_rsrc(p.x, row, p.x_stride, C, true);
    const __amdgpu_buffer_rsrc_t rr = row_rsrc(p.residual, row, p.r_stride, C, R);
    const __amdgpu_buffer_rsrc_t ro = row_rsrc(p.residual_out, row, p.ro_stride, C, R);
    const __amdgpu_buffer_rsrc_t oo = row_rsrc(p.out, row, p.out_stride, C, !Q);
    for (int c0 = 0; c0 < chunks; c0 += U) {
      u32x4 xq[U], rq[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        xq[u] = load_seg(rx, (c0 + u) * B + t);
        rq[u] = R ? load_seg(rr, (c0 + u) * B + t) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u;
        if (c >= chunks) break;  // uniform across the workgroup
        const int s = c * B + t;
        float acc[8];
        float bs = add_segment<R>(xq[u], rq[u], acc);
        if constexpr (R) store_seg(ro, s, pack8_rne(acc));  // dropped past the row
        if (s < C) {
          lo[s] = make_float4(acc[0], acc[1], acc[2], acc[3]);
          hi[s] = make_float4(acc[4], acc[5], acc[6], acc[7]);
        }
        bs = wave_block_sum(bs);
        if (lane == 0) blk[parity][c * W + wave] = bs;
      }
    }
    __syncthreads();
    const float rinv = row_rinv(pairwise_tree_lds<NB>(blk[parity]), p);
    // The staged fp32 values of segment s (the weight comes from registers
    // for the first U chunks, from memory beyond).
    auto staged = [&](int s, float (&acc)[8]) {
      const float4 l = lo[s], h = hi[s];
      acc[0] = l.x, acc[1] = l.y, acc[2] = l.z, acc[3] = l.w;
      acc[4] = h.x, acc[5] = h.y, acc[6] = h.z, acc[7] = h.w;
    };
    if constexpr (!Q) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int s = u * B + t;
        if (u < chunks && s < C) {
          float acc[8];
          staged(s, acc);
          store_seg(oo, s, normalise8(acc, rinv, wq[u]));
        }
      }
      for (int c = U; c < chunks; ++c) {
        const int s = c * B + t;
        if (s < C) {
          float acc[8];
          staged(s, acc);
          store_seg(oo, s, normalise8(acc, rinv, p.weight[s]));
        }
      }
    } else {
      // y from the staged sums twice: for the row maximum, then for the codes.
      uint32_t m = 0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int s = u * B + t;
        if (u < chunks && s < C) {
          float acc[8], y[8];
          staged(s, acc);
          scale8(acc, rinv, wq[u], y);
          m = max_abs8(m, y);
        }
      }
      for (int c = U; c < chunks; ++c) {
        const int s = c * B + t;
        if (s < C) {
          float acc[8], y[8];
          staged(s, acc);
          scale8(acc, rinv, p.weight[s], y);
          m = max_abs8(m, y);
        }
      }
      m = wave_max(m);
      if (lane == 0) mx[parity][wave] = m;
      __syncthreads();
      uint32_t mb = mx[parity][0];
#pragma unroll
      for (int i = 1; i < W; ++i) mb = umax(mb, mx[parity][i]);
      const float amax = __builtin_bit_cast(float, mb);
      const float scale = amax / qmax<Q>();
      const float inv = qmax<Q>() / amax;
      const bool ok = quantisable<Q>(amax);
      if (t == 0) p.qscale[row] = scale;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int s = u * B + t;
        if (u < chunks && s < C) {
          float acc[8], y[8];
          staged(s, acc);
          scale8(acc, rinv, wq[u], y);
          store_codes_stream(p.qout + base + s, ok ? quant8<Q>(y, inv) : u32x2{0, 0});
        }
      }
      for (int c = U; c < chunks; ++c) {
        const int s = c * B + t;
        if (s < C) {
          float acc[8], y[8];
          staged(s, acc);
          scale8(acc, rinv, p.weight[s], y);
          store_codes_stream(p.qout + base + s, ok ? quant8<Q>(y, inv) : u32x2{0, 0});
        }
      }
    }
  }
}

// ---------------------------------------------------------------- general shapes

// Any hidden in [1, 32768] and any row strides, 2-byte aligned.  Elements are
// loaded and stored one by one (16-bit), and the row is cut into the same
// 8-element segments as everywhere else: the last segment's missing elements
// are +0, which leaves its fma chain unchanged (fma(0, 0, t) = t for t >= 0),
// and segments past the row are +0 leaves of the tree.  So the sum of squares,
// and every result, is the same as the fast kernels give where both apply.
// One workgroup of B threads per row.  Loads and stores go one element per
// lane, consecutive lanes on consecutive elements (128 bytes per wavefront
// instruction); the fp32 sums are staged in LDS by element, and thread t then
// reads its segments t + B c from there for the tree, as the fast kernels
// hold them.  Normalisation reads LDS again and stores element by element.
struct GenParams {
  uint16_t* out;
  uint16_t* residual_out;
  const uint16_t* x;
  const uint16_t* residual;
  const uint16_t* weight;
  int64_t n_rows;
  int64_t x_stride, r_stride, out_stride, ro_stride;  // elements
  int32_t hidden;
  float hidden_f;
  float eps;
};

// Elements per thread loaded together by the general kernel.
constexpr int GU = 8;

DEV float bf16_at(const uint16_t* p, int j) { return __builtin_bit_cast(float, (uint32_t)p[j] << 16); }

// bf16 of one fp32 value by the same packed conversion as the fast kernels.
DEV uint16_t bf16_rne1(float v) { return (uint16_t)(pack2_rne(v, v) & 0xFFFFu); }

template <int B, int NB, bool R>
__global__ __launch_bounds__(B) void k_general(GenParams p) {
  constexpr int W = B / 64;
  __shared__ float blk[NB];
  extern __shared__ float4 stage4[];  // acc of element j at stage[j], padded to 8 * C
  float* stage = reinterpret_cast<float*>(stage4);
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int H = p.hidden;
  const int C = (H + 7) / 8;
  const int chunks = (C + B - 1) / B;

  for (int64_t row = blockIdx.x; row < p.n_rows; row += gridDim.x) {
    const uint16_t* xr = p.x + row * p.x_stride;
    const uint16_t* rr = R ? p.residual + row * p.r_stride : nullptr;
    uint16_t* ror = R ? p.residual_out + row * p.ro_stride : nullptr;
    uint16_t* orow = p.out + row * p.out_stride;
    // acc, one element per lane (consecutive lanes, consecutive elements),
    // residual_out stored the same way; the padding of the last segment is
    // +0.  GU elements per thread are loaded before any is used, so that
    // many loads are in flight.
    for (int j0 = t; j0 < 8 * C; j0 += GU * B) {
      float xv[GU], rv[GU];
#pragma unroll
      for (int u = 0; u < GU; ++u) {
        const int j = j0 + u * B;
        xv[u] = j < H ? bf16_at(xr, j) : 0.0f;
        if constexpr (R) rv[u] = j < H ? bf16_at(rr, j) : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < GU; ++u) {
        const int j = j0 + u * B;
        float a = xv[u];
        if constexpr (R) {
          a = a + rv[u];
          if (j < H) ror[j] = bf16_rne1(a);
        }
        if (j < 8 * C) stage[j] = j < H ? a : 0.0f;
      }
    }
    for (int i = chunks * W + t; i < NB; i += B) blk[i] = 0.0f;
    __syncthreads();
    // the segments' sums, thread t holding segments t + B c as everywhere
    for (int c = 0; c < chunks; ++c) {
      const int s = c * B + t;
      float acc[8];
      if (s < C) {
        const float4 l = stage4[2 * s];
        const float4 h = stage4[2 * s + 1];
        acc[0] = l.x; acc[1] = l.y; acc[2] = l.z; acc[3] = l.w;
        acc[4] = h.x; acc[5] = h.y; acc[6] = h.z; acc[7] = h.w;
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = 0.0f;
      }
      const float bs = wave_block_sum(seg_sumsq(acc));
      if (lane == 0) blk[c * W + wave] = bs;
    }
    __syncthreads();
    const float sumsq = pairwise_tree_lds<NB>(blk);
    const float rinv = 1.0f / __builtin_sqrtf(sumsq / p.hidden_f + p.eps);
    for (int j0 = t; j0 < H; j0 += GU * B) {
      float wv[GU];
#pragma unroll
      for (int u = 0; u < GU; ++u) wv[u] = j0 + u * B < H ? bf16_at(p.weight, j0 + u * B) : 0.0f;
#pragma unroll
      for (int u = 0; u < GU; ++u) {
        const int j = j0 + u * B;
        if (j < H) orow[j] = bf16_rne1((stage[j] * rinv) * wv[u]);
      }
    }
    __syncthreads();  // blk and the staged sums are rewritten by the next row
  }
}

// Register-resident general kernel: one workgroup of B threads per row,
// thread t holding segments t + B j (j < J) in registers, as k_wg_row does,
// with the same block sums and tree.  Loads and stores are 16-bit and
// coalesced: wavefront w reads the 512 elements of its segment block
// w + W j one element per lane (eight loads), then regroups them into one
// segment per lane through its own LDS slot, and sends residual_out and out
// back out the same way.  A wavefront's LDS accesses execute in order, so
// the regrouping needs no workgroup barrier; a wavefront-scope fence keeps
// the compiler from moving them across one another.  The weight is staged in
// LDS once per workgroup, in segment order, zero padded.
//
// Every row access goes through a buffer resource over the row, so the
// hardware range check, not a branch, handles the row's end.  With no
// branch around them the compiler counts how many accesses follow each
// prefetched load and waits for that load alone; with a branch per access
// it waited for every earlier access, the previous row's out stores
// included (measured on MI355X: 54.1 -> 52.3 us at 4096 x 8191, 58.1 -> 56.1
// us at 2048 x 16383, 67.1 -> 60.8 us at 4096 x 9001).
//
// A (line-aligned): each 16-bit access covers one whole 128-byte line
// instead of straddling two lines of a misaligned row, nine accesses per
// block instead of eight.  F: every block holds row elements; otherwise
// blocks past the row's end are skipped.  S (with A): all four tensors sit
// at one offset in their lines (checked on the host), so the sums and
// residual_out are formed where loaded, and each line that two blocks share
// is written whole, by the wavefront of the first block, after the row's
// barrier (so every wavefront has read the row, in place too; no wavefront
// writes that line before, so with two segments per thread its x and
// residual are read again there).
DEV void wave_fence() { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront"); }

// Stores a wavefront's block of 512 elements (first element b0 of the row)
// from its regrouping slot, one 16-bit element per lane and instruction,
// consecutive lanes at consecutive elements.  The slot is read whole before
// any store, so the eight LDS reads overlap (a read guarded by its store's
// own mask would wait for each in turn); only a block that ends past the
// row's end masks its stores.
DEV void store_block(uint16_t* dst, int b0, int h, const uint16_t* sl, int lane) {
  uint16_t v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = sl[64 * k + lane];
  if (b0 + 512 <= h) {
#pragma unroll
    for (int k = 0; k < 8; ++k) dst[b0 + 64 * k + lane] = v[k];
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (b0 + 64 * k + lane < h) dst[b0 + 64 * k + lane] = v[k];
  }
}

// A row's element offset within its 128-byte L2 line (0..63).
DEV int line_offset(const uint16_t* row) {
  return (int)((reinterpret_cast<uintptr_t>(row) >> 1) & 63);
}

// Buffer resource over one row of hidden h, starting o elements before the
// row (at its line in the line-aligned form below): the hardware range check
// drops stores and zeroes loads past the row's end, so no access needs a
// branch.  The last word selects 32-bit raw data (gfx9 layout).
DEV __amdgpu_buffer_rsrc_t gen_row_rsrc(const uint16_t* row, int o, int h) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(row - o), 0, 2 * (o + h),
                                           0x00020000);
}

template <int B, int J, bool R, bool A, bool F, bool S = false>
__global__ __launch_bounds__(B) void k_general_reg(GenParams p) {
  static_assert(!S || A, "shared line offsets are a case of the line-aligned form");
  constexpr int W = B / 64;
  constexpr int NB = W * J;
  constexpr int NW = A ? 9 : 8;     // 16-bit accesses per lane and block
  constexpr int PAD = A ? 64 : 0;   // slot elements on either side of the block
  constexpr int OOB = 1 << 30;      // a byte offset past every row resource
  // Cache policy of the row accesses: nontemporal in the line-aligned form
  // (measured on MI355X: 52.2 -> 49.2 us at 4096 x 8191, 17.9 -> 15.2 us at
  // 2048 x 4095, 43.7 -> 39.4 us at 4096 x 6143; nontemporal loads or stores
  // alone gained less), ordinary in the row-relative one, where nontemporal
  // accesses were slower (34.1 -> 38.0 us at 16384 x 1025, 56.1 -> 60.5 us at
  // 2048 x 16383).
  constexpr int CP = A ? 2 : 0;
  __shared__ float blk[2][NB];  // alternates by row so one barrier per row suffices
  // EW (row-relative form): x, residual and residual_out share the row's
  // layout, so the fp32 sums and residual_out are formed element by element
  // where loaded, and only the sums are regrouped, through an fp32 slot
  // (measured on MI355X: 60.9 -> 58.4 us at 4096 x 9001, 43.0 -> 38.0 us at
  // 16384 x 1025 with 512 threads; the line-aligned form, whose tensors may
  // sit at different offsets in their lines, was slower with it: 49.7 ->
  // 51.0 us at 4096 x 8191).  The 16-bit slot (out, and x and residual in
  // the other form) is the first half of the fp32 one.
  constexpr bool EW = !A || S;
  __shared__ float4 slotf4[W][S ? (512 + 2 * PAD) / 4 : EW ? 128 : (512 + 2 * PAD) / 8];
  extern __shared__ u32x4 wseg[];  // B * J segments of weight
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int H = p.hidden;
  uint16_t* wl = reinterpret_cast<uint16_t*>(wseg);
  for (int i = t; i < 8 * B * J; i += B) wl[i] = i < H ? p.weight[i] : (uint16_t)0;
  __syncthreads();
  uint16_t* sl = reinterpret_cast<uint16_t*>(slotf4[wave]) + PAD;  // sl[i]: element i of the block
  u32x4* sq = reinterpret_cast<u32x4*>(slotf4[wave]) + PAD / 8;    // sq[l]: segment l of the block
  float* slf = reinterpret_cast<float*>(slotf4[wave]) + (S ? PAD : 0);  // slf[i]: element i, fp32 (EW)

  // Access k of lane l in block b touches element 512 b + 64 k + l - o of
  // the row (o = 0 unless line-aligned), at byte 2 (512 b + 64 k + l) of the
  // row's resource; the first and last access drop the lanes outside the block.
  auto voff = [&](int o, int b, int k) {
    const int off = 2 * (512 * b + 64 * k + lane);
    if constexpr (A) {
      if (k == 0) return lane < o ? OOB : off;
      if (k == NW - 1) return lane < o ? off : OOB;
    }
    return off;
  };
  // S: the last access of a block reads its whole line (the next block's
  // first elements too), and a block after the first stores nothing of its
  // first line, which the block before it writes whole.
  auto voff_load = [&](int o, int b, int k) {
    if constexpr (S) {
      if (k == NW - 1) return 2 * (512 * b + 64 * k + lane);
    }
    return voff(o, b, k);
  };
  auto voff_store = [&](int o, int b, int k) {
    if constexpr (S) {
      if (k == 0 && b > 0) return OOB;
    }
    return voff(o, b, k);
  };
  uint16_t xv[J][NW], rv[J][NW];
  // In the line-aligned form a block's first and last lines are shared with
  // the neighbouring blocks (or rows), whose wavefronts read them too: those
  // two loads are ordinary, so the line stays in L2 for the second reader
  // (measured on MI355X: 15.3 -> 14.9 us at 2048 x 4095, 27.6 -> 26.8 us at
  // 8192 x 2047, 51.7 -> 50.9 us at 2048 x 16383, 48.4 -> 48.3 us at
  // 4096 x 8191).
  auto load_block = [&](__amdgpu_buffer_rsrc_t rs, int o, int b, uint16_t (&v)[NW]) {
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      if (A && (k == 0 || k == NW - 1))
        v[k] = __builtin_amdgcn_raw_buffer_load_b16(rs, voff_load(o, b, k), 0, 0);
      else
        v[k] = __builtin_amdgcn_raw_buffer_load_b16(rs, voff_load(o, b, k), 0, CP);
    }
  };
  // Element i of the block to sl[i]; lanes outside the block write the padding.
  auto to_slot = [&](const uint16_t (&v)[NW], int o) {
#pragma unroll
    for (int k = 0; k < NW; ++k) sl[64 * k + lane - o] = v[k];
  };
  // The block back out from the slot, all slot reads before any store (S:
  // all but its last line, which is written apart).
  auto store_block_rs = [&](__amdgpu_buffer_rsrc_t rs, int o, int b) {
    constexpr int NS = S ? NW - 1 : NW;
    uint16_t v[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) v[k] = sl[64 * k + lane - o];
    if (F || 512 * b < H) {
#pragma unroll
      for (int k = 0; k < NS; ++k)
        __builtin_amdgcn_raw_buffer_store_b16(v[k], rs, voff_store(o, b, k), 0, CP);
    }
  };
  // F: every block holds row elements, and no access has a branch.
  // Otherwise a block past the row's end is skipped whole, x and residual
  // under one branch (a branch per access would leave the waits for the
  // prefetched loads uncounted).  With J > 1 a skipped block's registers are
  // not zeroed, its processing is skipped instead (with a zero fill the
  // compiler packed the values in pairs, waiting for each load).
  auto load_row = [&](int64_t row) {
    const uint16_t* xr = p.x + row * p.x_stride;
    const int ox = A ? line_offset(xr) : 0;
    const auto xs = gen_row_rsrc(xr, ox, H);
    const uint16_t* rr = R ? p.residual + row * p.r_stride : nullptr;
    const int orr = A && R ? line_offset(rr) : 0;
    const auto rs = gen_row_rsrc(R ? rr : xr, orr, R ? H : 0);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (F || 512 * (wave + W * j) < H) {
        load_block(xs, ox, wave + W * j, xv[j]);
        if constexpr (R) load_block(rs, orr, wave + W * j, rv[j]);
      } else if constexpr (J == 1) {
#pragma unroll
        for (int k = 0; k < NW; ++k) xv[j][k] = rv[j][k] = 0;
      }
    }
  };
  // Each workgroup walks rows blockIdx.x, + gridDim.x, ...; the next row's
  // loads are issued before the current row's barrier and out stores
  // (measured on MI355X: 56.3 -> 54.8 us at 4096 x 8191, 64.3 -> 59.2 us at
  // 2048 x 16383).
  if ((int64_t)blockIdx.x < p.n_rows) load_row(blockIdx.x);
  int parity = 0;
  for (int64_t row = blockIdx.x; row < p.n_rows; row += gridDim.x, parity ^= 1) {
    const int ox = A ? line_offset(p.x + row * p.x_stride) : 0;
    const int orr = A && R ? line_offset(p.residual + row * p.r_stride) : 0;
    uint16_t* orow = p.out + row * p.out_stride;
    const int oo = A ? line_offset(orow) : 0;
    float acc[J][8];
    float bs[J];
    float a8[S && J == 1 ? J : 1];  // S: the fp32 sums of each block's last line, as loaded
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (!F && J > 1 && 512 * (wave + W * j) >= H) {
        // An empty block: its sum is +0 and nothing of it is stored.
        bs[j] = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[j][k] = 0.0f;
        continue;
      }
      if constexpr (EW) {
        float a[NW];
#pragma unroll
        for (int k = 0; k < NW; ++k) {
          a[k] = __builtin_bit_cast(float, (uint32_t)xv[j][k] << 16);
          if constexpr (R) a[k] = a[k] + __builtin_bit_cast(float, (uint32_t)rv[j][k] << 16);
        }
        if constexpr (R) {
          if (F || 512 * (wave + W * j) < H) {
            const auto ros = gen_row_rsrc(p.residual_out + row * p.ro_stride, ox, H);
#pragma unroll
            for (int k = 0; k < (S ? NW - 1 : NW); ++k)
              __builtin_amdgcn_raw_buffer_store_b16(bf16_rne1(a[k]), ros, voff_store(ox, wave + W * j, k),
                                                    0, CP);
          }
        }
        if constexpr (S && J == 1) a8[j] = a[NW - 1];
#pragma unroll
        for (int k = 0; k < NW; ++k) slf[64 * k + lane - ox] = a[k];
        wave_fence();
        constexpr int SP = S ? PAD / 4 : 0;  // the slot's padding, in float4
        const float4 l4 = slotf4[wave][SP + 2 * lane], h4 = slotf4[wave][SP + 2 * lane + 1];
        acc[j][0] = l4.x; acc[j][1] = l4.y; acc[j][2] = l4.z; acc[j][3] = l4.w;
        acc[j][4] = h4.x; acc[j][5] = h4.y; acc[j][6] = h4.z; acc[j][7] = h4.w;
        bs[j] = seg_sumsq(acc[j]);
        wave_fence();
        continue;
      }
      to_slot(xv[j], ox);
      wave_fence();
      const u32x4 xq = sq[lane];
      u32x4 rq = {0, 0, 0, 0};
      if constexpr (R) {
        wave_fence();
        to_slot(rv[j], orr);
        wave_fence();
        rq = sq[lane];
      }
      bs[j] = add_segment<R>(xq, rq, acc[j]);
      if constexpr (R) {
        uint16_t* ror = p.residual_out + row * p.ro_stride;
        const int oro = A ? line_offset(ror) : 0;
        wave_fence();
        sq[lane] = pack8_rne(acc[j]);
        wave_fence();
        store_block_rs(gen_row_rsrc(ror, oro, H), oro, wave + W * j);
      }
      wave_fence();
    }
    if (row + gridDim.x < p.n_rows) load_row(row + gridDim.x);
#pragma unroll
    for (int j = 0; j < J; ++j) bs[j] = wave_block_sum(bs[j]);
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < J; ++j) blk[parity][wave + W * j] = bs[j];
    }
    __syncthreads();
    const float sumsq = pairwise_tree_lds<NB>(blk[parity]);
    const float rinv = 1.0f / __builtin_sqrtf(sumsq / p.hidden_f + p.eps);
    const auto os = gen_row_rsrc(orow, oo, H);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const u32x4 wq = wseg[64 * (wave + W * j) + lane];
      sq[lane] = normalise8(acc[j], rinv, wq);
      wave_fence();
      store_block_rs(os, oo, wave + W * j);
      wave_fence();
      if constexpr (S) {
        // The block's last line, whole: its own last elements and the next
        // block's first ones (past the row's end the stores are dropped).
        const int b = wave + W * j;
        if (F || 512 * b < H) {
          const int e = min(512 * (b + 1) + lane - oo, 8 * B * J - 1);  // row element, in wl
          const float w = __builtin_bit_cast(float, (uint32_t)wl[e] << 16);
          const int off = 2 * (512 * b + 64 * (NW - 1) + lane);
          float s8;
          if constexpr (J == 1) {
            s8 = a8[j];
          } else {
            // read again (from L2): two segments per thread leave no
            // registers to keep the sums across the barrier
            const auto xs8 = gen_row_rsrc(p.x + row * p.x_stride, oo, H);
            const uint16_t x8 = __builtin_amdgcn_raw_buffer_load_b16(xs8, off, 0, 0);
            s8 = __builtin_bit_cast(float, (uint32_t)x8 << 16);
            if constexpr (R) {
              const auto rs8 = gen_row_rsrc(p.residual + row * p.r_stride, oo, H);
              const uint16_t r8 = __builtin_amdgcn_raw_buffer_load_b16(rs8, off, 0, 0);
              s8 = s8 + __builtin_bit_cast(float, (uint32_t)r8 << 16);
            }
          }
          __builtin_amdgcn_raw_buffer_store_b16(bf16_rne1((s8 * rinv) * w), os, off, 0, CP);
          if constexpr (R) {
            const auto ros = gen_row_rsrc(p.residual_out + row * p.ro_stride, oo, H);
            __builtin_amdgcn_raw_buffer_store_b16(bf16_rne1(s8), ros, off, 0, CP);
          }
        }
      }
    }
  }
}

// Long rows (above 16384 elements) of any alignment, 1024 threads per row:
// k_general's element-wise staging and arithmetic, thread t handling the G
// elements t + 1024 u of the row (u < G) in two halves of G / 2.  Every access
// goes through a buffer resource over its row (past the row: loads read +0,
// stores are dropped), so none sits under a branch.  The first half of the
// next row is loaded as soon as the current row's sums are staged in LDS,
// ahead of its reduction and out stores; its second half is loaded when the
// row starts, while the first half is added and staged.  Thread t stages and
// later reads back only its own elements, and the block sums are rewritten
// only after the next row's first barrier, so two barriers per row suffice
// (three in the line-aligned form below).
// (Measured on MI355X against k_general at 1024 threads: 168.2 -> 72.8 us at
// 1024 x 32767, 257.1 -> 102.6 us at 2048 x 24001, 248.0 -> 142.2 us at
// 4096 x 16385, bit-identical.  The weight staged in LDS beside the sums
// instead of read for each row was no faster: 102.6 -> 108.8 us at
// 2048 x 24001.)  A: when all tensors' rows sit at the same offset o in their
// 128-byte lines (checked on the host), thread t's element u is t + 1024 u - o
// and every access covers one whole line, nontemporal; this needs G elements
// per thread to cover o + the padded row, so rows above 32704 elements keep
// the row-relative form (measured, with its third barrier: 102.8 -> 84.4 us
// at 2048 x 24001, 142.2 -> 124.6 us at 4096 x 16385, 121.1 -> 98.8 us at
// 2048 x 28001).
template <int NB, int G, bool R, bool A>
__global__ __launch_bounds__(1024) void k_general_long(GenParams p) {
  constexpr int CP = A ? 2 : 0;  // nontemporal in the line-aligned form
  constexpr int OOB = 1 << 30;
  constexpr int B = 1024, W = B / 64;
  constexpr int G0 = (G + 1) / 2;  // accesses of the first half; G - G0 in the second
  auto in_half = [](int h, int u) { return u < (h ? G - G0 : G0); };
  __shared__ float blk[NB];
  extern __shared__ float4 stage4[];  // acc of element j at stage[j], padded to 8 * C
  float* stage = reinterpret_cast<float*>(stage4);
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int H = p.hidden;
  const int C = (H + 7) / 8;
  const int chunks = (C + B - 1) / B;
  // Element t + B u of a row: byte 2 t of the row's resource, plus 2 B u as
  // the (uniform) scalar offset, so no address register per element.  An
  // access wholly past the row (2 B u at or beyond the resource's size) takes
  // the size itself as its scalar offset: then it is out of range whether the
  // hardware adds the scalar offset to the checked offset or subtracts it
  // from the size, and no subtraction can wrap.  Only the last four accesses
  // can lie wholly past the row (G - 4 <= ceil(hidden / B), checked at
  // launch); the others keep constant offsets (clamping all of them cost
  // 1-2% on MI355X).
  const int vo = 2 * t;
  auto so = [&](int o, int u) { return u < G - 4 ? 2 * B * u : min(2 * B * u, 2 * (o + H)); };
  // A: every tensor's row starts o elements into its 128-byte line (checked
  // on the host); thread t's element u is t + B u - o, so each access covers
  // one whole line, and lanes with t + B u < o (before the row) are dropped.
  auto line_o = [&](int64_t row) { return A ? line_offset(p.x + row * p.x_stride) : 0; };
  auto vo0 = [&](int o) { return t < o ? OOB : vo; };  // the first access's offset
  // Loads of half h (elements u = G0 h .. G0 h + G0 - 1, below G) of a row.
  auto load_half = [&](int64_t row, int h, uint16_t (&xv)[G0], uint16_t (&rv)[G0]) {
    const int o = line_o(row);
    const auto xs = gen_row_rsrc(p.x + row * p.x_stride, o, H);
#pragma unroll
    for (int u = 0; u < G0; ++u)
      if (in_half(h, u))
        xv[u] = __builtin_amdgcn_raw_buffer_load_b16(xs, G0 * h + u == 0 ? vo0(o) : vo,
                                                     so(o, G0 * h + u), CP);
    if constexpr (R) {
      const auto rs = gen_row_rsrc(p.residual + row * p.r_stride, o, H);
#pragma unroll
      for (int u = 0; u < G0; ++u)
        if (in_half(h, u))
          rv[u] = __builtin_amdgcn_raw_buffer_load_b16(rs, G0 * h + u == 0 ? vo0(o) : vo,
                                                       so(o, G0 * h + u), CP);
    }
  };
  // acc by element (+0 past the row, as the loads there read +0) staged in
  // LDS, and residual_out stored the same way.
  auto stage_half = [&](int64_t row, int h, const uint16_t (&xv)[G0], const uint16_t (&rv)[G0]) {
    const int o = line_o(row);
    const auto ros = R ? gen_row_rsrc(p.residual_out + row * p.ro_stride, o, H)
                       : gen_row_rsrc(p.out, 0, 0);
#pragma unroll
    for (int u = 0; u < G0; ++u) {
      if (!in_half(h, u)) continue;
      const int j = t + B * (G0 * h + u) - o;
      float a = __builtin_bit_cast(float, (uint32_t)xv[u] << 16);
      if constexpr (R) {
        a = a + __builtin_bit_cast(float, (uint32_t)rv[u] << 16);
        __builtin_amdgcn_raw_buffer_store_b16(bf16_rne1(a), ros, G0 * h + u == 0 ? vo0(o) : vo,
                                              so(o, G0 * h + u), CP);
      }
      if (j >= 0 && j < 8 * C) stage[j] = a;
    }
  };
  uint16_t xa[G0], ra[G0], xb[G0], rb[G0];
  if ((int64_t)blockIdx.x < p.n_rows) load_half(blockIdx.x, 0, xa, ra);
  for (int64_t row = blockIdx.x; row < p.n_rows; row += gridDim.x) {
    load_half(row, 1, xb, rb);
    stage_half(row, 0, xa, ra);
    stage_half(row, 1, xb, rb);
    if (row + gridDim.x < p.n_rows) load_half(row + gridDim.x, 0, xa, ra);
    for (int i = chunks * W + t; i < NB; i += B) blk[i] = 0.0f;
    __syncthreads();
    // the segments' sums, thread t holding segments t + B c as everywhere
    for (int c = 0; c < chunks; ++c) {
      const int s = c * B + t;
      float acc[8];
      if (s < C) {
        const float4 l = stage4[2 * s];
        const float4 h = stage4[2 * s + 1];
        acc[0] = l.x; acc[1] = l.y; acc[2] = l.z; acc[3] = l.w;
        acc[4] = h.x; acc[5] = h.y; acc[6] = h.z; acc[7] = h.w;
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = 0.0f;
      }
      const float bs = wave_block_sum(seg_sumsq(acc));
      if (lane == 0) blk[c * W + wave] = bs;
    }
    __syncthreads();
    const float sumsq = pairwise_tree_lds<NB>(blk);
    const float rinv = 1.0f / __builtin_sqrtf(sumsq / p.hidden_f + p.eps);
    const int o = line_o(row);
    const auto os = gen_row_rsrc(p.out + row * p.out_stride, o, H);
    const auto ws = gen_row_rsrc(p.weight, o, H);  // the weight in the row's element order
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint16_t wv[G0];
#pragma unroll
      for (int u = 0; u < G0; ++u)
        if (in_half(h, u))
          wv[u] = __builtin_amdgcn_raw_buffer_load_b16(ws, G0 * h + u == 0 ? vo0(o) : vo,
                                                       so(o, G0 * h + u), 0);
#pragma unroll
      for (int u = 0; u < G0; ++u) {
        if (!in_half(h, u)) continue;
        const int j = t + B * (G0 * h + u) - o;
        const float a = j >= 0 && j < 8 * C ? stage[j] : 0.0f;
        const float w = __builtin_bit_cast(float, (uint32_t)wv[u] << 16);
        __builtin_amdgcn_raw_buffer_store_b16(bf16_rne1((a * rinv) * w), os, G0 * h + u == 0 ? vo0(o) : vo,
                                              so(o, G0 * h + u), CP);
      }
    }
    // In the line-aligned form a thread's elements move with the row's line
    // offset, so the next row's sums may land in slots other threads are
    // still reading.
    if constexpr (A) __syncthreads();
  }
}

// Wavefront-per-row general kernel for short rows (at most 64 J segments):
// WAVES rows per workgroup, each wavefront one row, its J segment blocks
// regrouped through its own LDS slot as in k_general_reg; the J block sums
// finish the tree in registers, so no barrier is needed after the weight is
// staged.  (Buffer-resource accesses with a next-row prefetch, as in
// k_general_reg, were slower here wherever the last block is short, since
// every access of it is issued: 26.8 -> 32.0 us at 65536 x 127, 32.3 -> 37.8
// us at 32768 x 513, against 30.4 -> 29.7 us at 16384 x 1001, measured on
// MI355X.)
template <int WAVES, int J, bool R>
__global__ __launch_bounds__(WAVES * 64) void k_general_wave(GenParams p) {
  __shared__ u32x4 slot[WAVES][64];
  __shared__ u32x4 wseg[64 * J];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int H = p.hidden;
  uint16_t* wl = reinterpret_cast<uint16_t*>(wseg);
  for (int i = t; i < 512 * J; i += WAVES * 64) wl[i] = i < H ? p.weight[i] : (uint16_t)0;
  __syncthreads();
  uint16_t* sl = reinterpret_cast<uint16_t*>(slot[wave]);

  const int64_t stride = (int64_t)gridDim.x * WAVES;
  for (int64_t row = (int64_t)blockIdx.x * WAVES + wave; row < p.n_rows; row += stride) {
    const uint16_t* xr = p.x + row * p.x_stride;
    const uint16_t* rr = R ? p.residual + row * p.r_stride : nullptr;
    uint16_t* ror = R ? p.residual_out + row * p.ro_stride : nullptr;
    uint16_t* orow = p.out + row * p.out_stride;
    uint16_t xv[J][8], rv[J][8];
#pragma unroll
    for (int j = 0; j < J; ++j) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int e = 512 * j + 64 * k + lane;
        xv[j][k] = e < H ? xr[e] : (uint16_t)0;
        if constexpr (R) rv[j][k] = e < H ? rr[e] : (uint16_t)0;
      }
    }
    float acc[J][8];
    float bs[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
#pragma unroll
      for (int k = 0; k < 8; ++k) sl[64 * k + lane] = xv[j][k];
      wave_fence();
      const u32x4 xq = slot[wave][lane];
      u32x4 rq = {0, 0, 0, 0};
      if constexpr (R) {
        wave_fence();
#pragma unroll
        for (int k = 0; k < 8; ++k) sl[64 * k + lane] = rv[j][k];
        wave_fence();
        rq = slot[wave][lane];
      }
      bs[j] = add_segment<R>(xq, rq, acc[j]);
      if constexpr (R) {
        wave_fence();
        slot[wave][lane] = pack8_rne(acc[j]);
        wave_fence();
        store_block(ror, 512 * j, H, sl, lane);
      }
      wave_fence();
    }
#pragma unroll
    for (int j = 0; j < J; ++j) bs[j] = wave_block_sum(bs[j]);
    const float sumsq = pairwise_tree<J>(bs);
    const float rinv = 1.0f / __builtin_sqrtf(sumsq / p.hidden_f + p.eps);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      slot[wave][lane] = normalise8(acc[j], rinv, wseg[64 * j + lane]);
      wave_fence();
      store_block(orow, 512 * j, H, sl, lane);
      wave_fence();
    }
  }
}

// ---------------------------------------------------------------- packed short rows

// Rows of at most 64 segments (hidden <= 512), several per wavefront: P lanes
// per row (the power of two >= the row's segments), 64 / P rows per
// wavefront, lane l holding segment l % P of row slot l / P.  The P-lane
// butterfly below is the canonical tree over the row's segments padded with
// +0 to P leaves; the levels from P up to 64 leaves would add only +0 to a
// sum of squares (never -0), which changes no bit, so every path gives the
// same sums.  Each wavefront takes U row groups of 64 / P rows per iteration,
// their loads issued together.
//
// Rows are addressed in two levels: row i of a group is head h = i % heads of
// token t = i / heads, at segment t * token_stride + h * segs of each tensor
// (a plain row tensor is one head per token).  Two groups, e.g. the q heads
// and the k heads of attention with their own weights, share one launch: the
// packed row index runs over group 0, padded to whole wavefront iterations,
// then group 1, so each wavefront iteration lies in one group.
struct PackGroup {
  u32x4* out;
  u32x2* qout;    // 1-byte codes, contiguous [n_rows][segs * 8] (quantised out)
  float* qscale;  // per-row scale (quantised out)
  u32x4* residual_out;
  const u32x4* x;
  const u32x4* residual;
  const u32x4* weight;
  int64_t x_ts, r_ts, out_ts, ro_ts;  // token strides, in segments
  uint32_t n_rows;                    // tokens * heads
  uint32_t heads;
  // ceil(2^64 / heads) for heads > 1, split in 32-bit halves: for i < 2^32,
  // the high 64 bits of i * magic are exactly i / heads.
  uint32_t magic_lo, magic_hi;
};

struct PackParams {
  PackGroup g[2];
  uint32_t first1;  // packed index of group 1's first row
  uint32_t total;   // first1 + group 1's rows
  int32_t segs;
  float hidden_f;
  float eps;
};

DEV uint32_t div_by_heads(uint32_t i, const PackGroup& g) {
  if (g.heads == 1) return i;
  const uint64_t a = (uint64_t)i * g.magic_hi + __umulhi(i, g.magic_lo);
  return (uint32_t)(a >> 32);
}

// Unsigned maximum over aligned blocks of P lanes; all 64 lanes active.
template <int P>
DEV uint32_t lane_block_max(uint32_t v) {
  if constexpr (P >= 2) v = umax(v, ADDRMS_DPP_U(v, 0xB1));
  if constexpr (P >= 4) v = umax(v, ADDRMS_DPP_U(v, 0x4E));
  if constexpr (P >= 8) v = umax(v, ADDRMS_DPP_U(v, 0x141));
  if constexpr (P >= 16) v = umax(v, ADDRMS_DPP_U(v, 0x140));
  if constexpr (P >= 32) v = umax(v, (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F));
  if constexpr (P >= 64)
    v = umax((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
             (uint32_t)__builtin_amdgcn_readlane((int)v, 32));
  return v;
}

// Sum over aligned blocks of P lanes (a power of two), the same bits in every
// lane of a block: the first levels of wave_block_sum.  All 64 lanes active.
template <int P>
DEV float lane_block_sum(float v) {
  if constexpr (P >= 2) v = v + ADDRMS_DPP(v, 0xB1);
  if constexpr (P >= 4) v = v + ADDRMS_DPP(v, 0x4E);
  if constexpr (P >= 8) v = v + ADDRMS_DPP(v, 0x141);
  if constexpr (P >= 16) v = v + ADDRMS_DPP(v, 0x140);
  if constexpr (P >= 32)
    v = v + __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
  if constexpr (P >= 64) {
    const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    v = lo + hi;
  }
  return v;
}

template <int WAVES, int P, int U, int Q, bool R>
__global__ __launch_bounds__(WAVES * 64) void k_pack_rows(PackParams p) {
  constexpr int RW = 64 / P;  // rows per wavefront per row group
  __shared__ u32x4 wl[2][P];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int C = p.segs;
  const int s = lane % P;
  const int slot = lane / P;
  for (int i = threadIdx.x; i < 2 * P; i += WAVES * 64) {
    const int g = i / P, k = i % P;
    const u32x4* w = g ? p.g[1].weight : p.g[0].weight;
    wl[g][k] = (k < C && w) ? w[k] : u32x4{0, 0, 0, 0};
  }
  __syncthreads();

  const int64_t step = (int64_t)gridDim.x * WAVES * RW * U;
  for (int64_t base = ((int64_t)blockIdx.x * WAVES + wave) * RW * U; base < p.total;
       base += step) {
    const int g = base >= p.first1 ? 1 : 0;
    const PackGroup G = g ? p.g[1] : p.g[0];
    const uint32_t row0 = (uint32_t)base - (g ? p.first1 : 0u);
    int64_t xo[U], oo[U], ro[U], rso[U];
    uint32_t row[U];
    bool valid[U];
    u32x4 xq[U], rq[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t i = row0 + (uint32_t)(u * RW + slot);
      row[u] = i;
      valid[u] = i < G.n_rows && s < C;
      const uint32_t t = div_by_heads(i, G);
      const int64_t hs = (int64_t)(i - t * G.heads) * C + s;
      xo[u] = (int64_t)t * G.x_ts + hs;
      oo[u] = (int64_t)t * G.out_ts + hs;
      ro[u] = (int64_t)t * G.r_ts + hs;
      rso[u] = (int64_t)t * G.ro_ts + hs;
      xq[u] = valid[u] ? load_stream(G.x + xo[u]) : u32x4{0, 0, 0, 0};
      rq[u] = (R && valid[u]) ? load_stream(G.residual + ro[u]) : u32x4{0, 0, 0, 0};
    }
    float sum[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float acc[8];
      sum[u] = add_segment<R>(xq[u], rq[u], acc);
      if constexpr (R)
        if (valid[u]) store_stream(G.residual_out + rso[u], pack8_rne(acc));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) sum[u] = lane_block_sum<P>(sum[u]);
    const u32x4 w = wl[g][s];
    if constexpr (!Q) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float rinv = 1.0f / __builtin_sqrtf(sum[u] / p.hidden_f + p.eps);
        float acc[8];
        add8<R>(opaque(xq[u]), opaque(rq[u]), acc);
        if (valid[u]) store_stream(G.out + oo[u], normalise8(acc, rinv, w));
      }
    } else {
      // y twice (the same fp32 operations, so the same values): once for the
      // row maximum over the row's lanes, once for the codes.  Codes are
      // contiguous per row, so a row's codes start at row * segs.
      float rinv[U];
      uint32_t m[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        rinv[u] = 1.0f / __builtin_sqrtf(sum[u] / p.hidden_f + p.eps);
        float acc[8], y[8];
        add8<R>(opaque(xq[u]), opaque(rq[u]), acc);
        scale8(acc, rinv[u], w, y);
        m[u] = valid[u] ? max_abs8(0u, y) : 0u;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) m[u] = lane_block_max<P>(m[u]);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float amax = __builtin_bit_cast(float, m[u]);
        const float inv = qmax<Q>() / amax;
        const bool ok = quantisable<Q>(amax);
        if (valid[u] && s == 0) G.qscale[row[u]] = amax / qmax<Q>();
        float acc[8], y[8];
        add8<R>(opaque(xq[u]), opaque(rq[u]), acc);
        scale8(acc, rinv[u], w, y);
        if (valid[u])
          store_codes_stream(G.qout + (int64_t)row[u] * C + s,
                             ok ? quant8<Q>(y, inv) : u32x2{0, 0});
      }
    }
  }
}

// ---------------------------------------------------------------- epilogue test

__global__ __launch_bounds__(256) void k_cvt_range(u32x4* out, uint32_t start, int64_t groups) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups; g += stride) {
    const uint32_t u0 = start + (uint32_t)(g * 8);
    float a[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) a[k] = __builtin_bit_cast(float, u0 + (uint32_t)k);
    out[g] = pack8_rne(a);
  }
}

// out[i] = E4M3 code of the fp32 with bit pattern start + i, through the
// quantised variant's code routine with inv = 1 (y * 1 = y exactly).
__global__ __launch_bounds__(256) void k_cvt_e4m3_range(u32x2* out, uint32_t start,
                                                        int64_t groups) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups; g += stride) {
    const uint32_t u0 = start + (uint32_t)(g * 8);
    float a[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) a[k] = __builtin_bit_cast(float, u0 + (uint32_t)k);
    out[g] = quant8<kQFp8>(a, 1.0f);
  }
}

// ---------------------------------------------------------------- copy reference

// Two streaming copies with the fused kernels' access pattern (16-byte
// nontemporal loads and stores) and no arithmetic: the reference rate for a
// 50/50 read/write stream of the same bytes.  Grid-stride over segments.
__global__ __launch_bounds__(256) void k_copy2(u32x4* d0, u32x4* d1, const u32x4* s0,
                                               const u32x4* s1, int64_t segs) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < segs; i += stride) {
    const u32x4 a = load_stream(s0 + i);
    const u32x4 b = load_stream(s1 + i);
    store_stream(d0 + i, a);
    store_stream(d1 + i, b);
  }
}

// The same copy with the fused kernels' row structure, and reads grouped:
// each workgroup of 512 threads takes R consecutive rows of hidden = 8 * segs
// elements (thread t holds segments t + 512 j, J of them), issues every load
// of its R rows, then every store.  With R = 1 it moves data exactly as one
// fused call's register kernel does; R = 2, 4 put longer same-direction
// bursts on each compute unit.  One workgroup per R rows.
template <int R, int J>
__global__ __launch_bounds__(512) void k_copy_rows(u32x4* d0, u32x4* d1, const u32x4* s0,
                                                 const u32x4* s1, int64_t n_rows, int segs) {
  const int t = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * R;
  u32x4 a[R][J], b[R][J];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const bool v = r0 + k < n_rows;
    const __amdgpu_buffer_rsrc_t ra = row_rsrc(s0, r0 + k, segs, segs, v);
    const __amdgpu_buffer_rsrc_t rb = row_rsrc(s1, r0 + k, segs, segs, v);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      a[k][j] = load_seg(ra, t + 512 * j);
      b[k][j] = load_seg(rb, t + 512 * j);
    }
  }
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const bool v = r0 + k < n_rows;
    const __amdgpu_buffer_rsrc_t wa = row_rsrc(d0, r0 + k, segs, segs, v);
    const __amdgpu_buffer_rsrc_t wb = row_rsrc(d1, r0 + k, segs, segs, v);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      store_seg(wa, t + 512 * j, a[k][j]);
      store_seg(wb, t + 512 * j, b[k][j]);
    }
  }
}

// One-directional streams with the same access pattern: read-only (the
// loaded words are folded together and written out only if they match a
// pattern no test data holds, so the loads stay live and almost nothing is
// written) and write-only.  With k_copy2 they bound what any mix of these
// loads and stores can reach on the device.
__global__ __launch_bounds__(256) void k_stream_read(u32x4* sink, const u32x4* src, int64_t segs) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 acc = {0, 0, 0, 0};
  for (int64_t i = t; i < segs; i += stride) acc ^= load_stream(src + i);
  if (t < segs && acc.x == 0x5EED5EEDu && acc.y == 0xC0FFEE00u && acc.z == 0x0BADF00Du &&
      acc.w == 0xFEEDFACEu)
    sink[t] = acc;  // within dst, which holds segs words
}

__global__ __launch_bounds__(256) void k_stream_write(u32x4* dst, int64_t segs) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  const u32x4 v = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < segs; i += stride)
    store_stream(dst + i, v);
}

// ---------------------------------------------------------------- launch helpers

Params make_params(const FwdArgs& a) {
  Params p;
  p.out = reinterpret_cast<u32x4*>(a.out);
  p.qout = reinterpret_cast<u32x2*>(a.qout);
  p.qscale = a.qscale;
  p.residual_out = reinterpret_cast<u32x4*>(a.residual_out);
  p.x = reinterpret_cast<const u32x4*>(a.x);
  p.residual = reinterpret_cast<const u32x4*>(a.residual);
  p.weight = reinterpret_cast<const u32x4*>(a.weight);
  p.n_rows = a.n_rows;
  p.segs = a.hidden / 8;
  p.x_stride = a.x_stride / 8;
  p.r_stride = a.r_stride / 8;
  p.out_stride = a.out_stride / 8;
  p.ro_stride = a.ro_stride / 8;
  p.hidden_f = (float)a.hidden;
  p.eps = a.eps;
  return p;
}

// Grid size: an explicit block count, else one workgroup per row group
// (capped; the kernels loop over any rows beyond the grid).
unsigned grid_for(int64_t grid_blocks, int64_t row_groups) {
  const int64_t cap = (int64_t)1 << 30;
  int64_t g = grid_blocks > 0 ? grid_blocks : row_groups;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return (unsigned)g;
}

// Resident-workgroup counts already asked of the runtime, by (device, kernel,
// workgroup size, LDS bytes): the occupancy query costs microseconds of host
// time, and its answer never changes for a kernel on a device.  Shared by all
// host threads.
struct ResidentKey {
  int dev;
  const void* kernel;
  int block_threads;
  size_t lds;
  bool operator<(const ResidentKey& o) const {
    if (dev != o.dev) return dev < o.dev;
    if (kernel != o.kernel) return kernel < o.kernel;
    if (block_threads != o.block_threads) return block_threads < o.block_threads;
    return lds < o.lds;
  }
};
std::mutex g_resident_mu;
std::map<ResidentKey, int64_t> g_resident;

// Workgroups of a kernel that fit on the current device at once; 0 if unknown.
template <typename K>
int64_t resident(K kernel, int block_threads, size_t lds) {
  int dev = 0, per_cu = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const ResidentKey key{dev, reinterpret_cast<const void*>(kernel), block_threads, lds};
  {
    std::lock_guard<std::mutex> g(g_resident_mu);
    const auto it = g_resident.find(key);
    if (it != g_resident.end()) return it->second;
  }
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block_threads, lds) !=
      hipSuccess)
    return 0;
  const int64_t n = (int64_t)per_cu * cus;
  if (n > 0) {
    std::lock_guard<std::mutex> g(g_resident_mu);
    g_resident[key] = n;
  }
  return n;
}

// Padded block count of the two-pass tree: 32 blocks of 64 segments cover
// hidden <= 16384, 64 cover the library's maximum.
int two_pass_nb(int hidden) { return hidden <= 16384 ? 32 : 64; }

// Chunks in flight per wavefront in the two-pass kernel: 2048 segments per
// batch at most (a whole 16384-wide row), and no more than 4.
template <int B>
constexpr int two_pass_batch() {
  return 2048 / B < 4 ? 2048 / B : 4;
}

// A kernel instance and its launch: `grid_blocks` -1 asks for the resident
// maximum, 0 for one workgroup per row group.
template <typename K>
hipError_t launch(K kernel, int block_threads, size_t lds, int64_t grid_blocks,
                  int64_t row_groups, const Params& p, hipStream_t s) {
  if (grid_blocks == -1) grid_blocks = resident(kernel, block_threads, lds);
  hipLaunchKernelGGL(kernel, dim3(grid_for(grid_blocks, row_groups)), dim3(block_threads), lds,
                     s, p);
  return hipGetLastError();
}

// Combinations that would not fit the register file (segments held per thread
// times threads per workgroup) are not built; wave_row_supported() and
// wg_row_supported() say which exist.
template <int Q, bool R, int WAVES>
hipError_t go_wave(const Params& p, int j, int64_t grid, hipStream_t s) {
  const int64_t groups = (p.n_rows + WAVES - 1) / WAVES;
  switch (j) {
    case 1: return launch(k_wave_row<WAVES, 1, Q, R>, WAVES * 64, 0, grid, groups, p, s);
    case 2: return launch(k_wave_row<WAVES, 2, Q, R>, WAVES * 64, 0, grid, groups, p, s);
    case 4: return launch(k_wave_row<WAVES, 4, Q, R>, WAVES * 64, 0, grid, groups, p, s);
    case 8:
      if constexpr (WAVES < 16)
        return launch(k_wave_row<WAVES, 8, Q, R>, WAVES * 64, 0, grid, groups, p, s);
      break;
  }
  return hipErrorInvalidValue;
}

template <int Q, bool R, int B, bool L, bool FB = false>
hipError_t go_wg(const Params& p, int j, int64_t grid, hipStream_t s) {
  switch (j) {
    case 1: return launch(k_wg_row<B, 1, Q, R, L, FB>, B, 0, grid, p.n_rows, p, s);
    case 2: return launch(k_wg_row<B, 2, Q, R, L, FB>, B, 0, grid, p.n_rows, p, s);
    case 4:
      if constexpr (B * 4 <= 2048)
        return launch(k_wg_row<B, 4, Q, R, L, FB>, B, 0, grid, p.n_rows, p, s);
      break;
    case 8:
      if constexpr (B * 8 <= 2048)
        return launch(k_wg_row<B, 8, Q, R, L, FB>, B, 0, grid, p.n_rows, p, s);
      break;
  }
  return hipErrorInvalidValue;
}

template <int Q, bool R, int B>
hipError_t go_wg_late(const Params& p, int j, int64_t grid, bool late, hipStream_t s) {
  if constexpr (Q == 0 && R) {
    // Fused bf16 rows whose segments fill every thread's slots.
    if (p.segs == B * j) {
      if (late) return go_wg<Q, R, B, true, true>(p, j, grid, s);
      return go_wg<Q, R, B, false, true>(p, j, grid, s);
    }
  }
  if constexpr (Q == 0) {
    if (late) return go_wg<Q, R, B, true>(p, j, grid, s);
  } else {
    if (late) return hipErrorInvalidValue;
  }
  return go_wg<Q, R, B, false>(p, j, grid, s);
}

template <int Q, bool R, int B>
hipError_t go_two_pass(const Params& p, int hidden, int64_t grid, hipStream_t s) {
  const size_t lds = (size_t)p.segs * 32;
  if (two_pass_nb(hidden) == 32)
    return launch(k_lds_two_pass<B, 32, two_pass_batch<B>(), Q, R>, B, lds, grid, p.n_rows, p,
                  s);
  return launch(k_lds_two_pass<B, 64, two_pass_batch<B>(), Q, R>, B, lds, grid, p.n_rows, p, s);
}

template <int Q, bool R>
hipError_t wave_by_block(const Params& p, int b, int j, int64_t grid, hipStream_t s) {
  switch (b) {
    case 64: return go_wave<Q, R, 1>(p, j, grid, s);
    case 128: return go_wave<Q, R, 2>(p, j, grid, s);
    case 256: return go_wave<Q, R, 4>(p, j, grid, s);
    case 512: return go_wave<Q, R, 8>(p, j, grid, s);
    case 1024: return go_wave<Q, R, 16>(p, j, grid, s);
  }
  return hipErrorInvalidValue;
}

template <int Q, bool R>
hipError_t wg_by_block(const Params& p, int b, int j, int64_t grid, bool late, hipStream_t s) {
  switch (b) {
    case 64: return go_wg_late<Q, R, 64>(p, j, grid, late, s);
    case 128: return go_wg_late<Q, R, 128>(p, j, grid, late, s);
    case 256: return go_wg_late<Q, R, 256>(p, j, grid, late, s);
    case 512: return go_wg_late<Q, R, 512>(p, j, grid, late, s);
    case 1024: return go_wg_late<Q, R, 1024>(p, j, grid, late, s);
  }
  return hipErrorInvalidValue;
}

template <int Q, bool R>
hipError_t two_pass_by_block(const Params& p, int b, int hidden, int64_t grid, hipStream_t s) {
  switch (b) {
    case 64: return go_two_pass<Q, R, 64>(p, hidden, grid, s);
    case 128: return go_two_pass<Q, R, 128>(p, hidden, grid, s);
    case 256: return go_two_pass<Q, R, 256>(p, hidden, grid, s);
    case 512: return go_two_pass<Q, R, 512>(p, hidden, grid, s);
    case 1024: return go_two_pass<Q, R, 1024>(p, hidden, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// ---------------------------------------------------------------- internal API

// Every tensor's rows start at one offset in their 128-byte lines: the same
// offset at the first row, and row strides equal modulo a line.
template <bool R>
bool shared_line_offsets(const GenParams& p) {
  auto off = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) >> 1) & 63; };
  return off(p.x) == off(p.out) && p.x_stride % 64 == p.out_stride % 64 &&
         (!R || (off(p.x) == off(p.residual) && off(p.x) == off(p.residual_out) &&
                 p.x_stride % 64 == p.r_stride % 64 && p.x_stride % 64 == p.ro_stride % 64));
}

template <int NB, int G, bool R, bool A = false>
hipError_t go_general_long(const GenParams& p, size_t lds, int64_t grid, hipStream_t s) {
  // the kernel clamps the scalar offsets of its last four accesses only
  if (G - 4 > (p.hidden + 1023) / 1024) return hipErrorInvalidValue;
  auto k = k_general_long<NB, G, R, A>;
  if (grid == -1) grid = resident(k, 1024, lds);
  hipLaunchKernelGGL(k, dim3(grid_for(grid, p.n_rows)), dim3(1024), lds, s, p);
  return hipGetLastError();
}

template <bool R, int B>
hipError_t go_general(const GenParams& p, int hidden, int64_t grid, hipStream_t s) {
  const size_t lds = (size_t)((hidden + 7) / 8) * 32;
  // Rows above 16384 at 1024 threads: the long-row kernel, with the fewest
  // elements per thread (of 18, 20, 24, 28, 32, and 33 for the line-aligned
  // form's extra line) that cover the row, in the line-aligned form when
  // every tensor's rows share their line offset.
  if constexpr (B == 1024) {
    const bool same = shared_line_offsets<R>(p);
    // Thread t's elements t + 1024 u - o (o <= 63) must cover the row padded
    // to whole segments.
    const int padded = (hidden + 7) / 8 * 8;
    if (same && hidden > 16384) {
      const int g = (padded + 63 + 1023) / 1024;
      if (g <= 18) return go_general_long<64, 18, R, true>(p, lds, grid, s);
      if (g <= 20) return go_general_long<64, 20, R, true>(p, lds, grid, s);
      if (g <= 24) return go_general_long<64, 24, R, true>(p, lds, grid, s);
      if (g <= 28) return go_general_long<64, 28, R, true>(p, lds, grid, s);
      if (g <= 32) return go_general_long<64, 32, R, true>(p, lds, grid, s);
      return go_general_long<64, 33, R, true>(p, lds, grid, s);
    }
    if (hidden > 16384 && hidden <= 32768) {
      const int g = (hidden + 1023) / 1024;
      if (g <= 18) return go_general_long<64, 18, R>(p, lds, grid, s);
      if (g <= 20) return go_general_long<64, 20, R>(p, lds, grid, s);
      if (g <= 24) return go_general_long<64, 24, R>(p, lds, grid, s);
      if (g <= 28) return go_general_long<64, 28, R>(p, lds, grid, s);
      return go_general_long<64, 32, R>(p, lds, grid, s);
    }
  }
  if (two_pass_nb(hidden) == 32) {
    auto k = k_general<B, 32, R>;
    if (grid == -1) grid = resident(k, B, lds);
    hipLaunchKernelGGL(k, dim3(grid_for(grid, p.n_rows)), dim3(B), lds, s, p);
  } else {
    auto k = k_general<B, 64, R>;
    if (grid == -1) grid = resident(k, B, lds);
    hipLaunchKernelGGL(k, dim3(grid_for(grid, p.n_rows)), dim3(B), lds, s, p);
  }
  return hipGetLastError();
}

template <int B, int J, bool R, bool A, bool F = false, bool S = false>
hipError_t go_general_reg_k(const GenParams& p, int64_t grid, hipStream_t s) {
  const size_t lds = (size_t)B * J * 16;
  auto k = k_general_reg<B, J, R, A, F, S>;
  if (grid == -1) grid = resident(k, B, lds);
  hipLaunchKernelGGL(k, dim3(grid_for(grid, p.n_rows)), dim3(B), lds, s, p);
  return hipGetLastError();
}

// The line-aligned accesses take rows whose last block holds more than 128
// elements, with one segment per thread, or with two when every block holds
// row elements.  Measured on MI355X before the line-aligned form's accesses
// became nontemporal: 32.3 -> 30.9 us at 8192 x 2047, 18.1 -> 17.6 us at
// 2048 x 4095, 57.2 -> 55.7 us at 8192 x 4095, 28.8 -> 28.3 us at
// 8192 x 1791, 81.6 -> 80.6 us at 8192 x 6143; with fewer elements they
// were slower: 27.2 -> 27.4 us at 8192 x 1663, 34.1 -> 35.9 us at
// 16384 x 1025.  With two segments per thread and nontemporal accesses:
// 56.3 -> 52.0 us at 2048 x 16383; with blocks past the row's end, slower
// (61.0 -> 66.1 us at 4096 x 9001, 80.5 -> 81.7 us at 4096 x 12287).
bool general_lines(int hidden) { return hidden % 512 == 0 || hidden % 512 > 128; }

template <bool R, int B>
hipError_t go_general_reg(const GenParams& p, int j, int64_t grid, hipStream_t s) {
  // Every one of the j * B / 64 blocks of 512 elements holds row elements:
  // the kernel without branches on the row's end.
  const bool full = 512 * (j * B / 64 - 1) < p.hidden;
  switch (j) {
    case 1:
      // Rows whose last block is short (row-relative form otherwise) take it
      // too when more than half of the blocks hold row elements, as with the
      // default workgroup (measured on MI355X: 27.1 -> 24.0 us at 8192 x
      // 1663, 34.0 -> 32.5 us at 16384 x 1025, 21.4 -> 18.8 us at 4096 x
      // 2600, 45.1 -> 40.1 us at 8192 x 3100; with most blocks empty, slower:
      // 37.5 -> 42.6 us at 16384 x 1025 with 512 threads).
      if ((general_lines(p.hidden) || 512 * (B / 128) < p.hidden) && shared_line_offsets<R>(p)) {
        // Writing the lines two blocks share whole pays once each workgroup
        // slot takes three or more rows.  Measured on MI355X (one segment
        // per thread, default launch): 49.9 -> 48.6 us at 4096 x 8191, 39.3
        // -> 38.2 at 4096 x 6143, 28.2 -> 27.6 at 8192 x 2047, 27.3 -> 26.9
        // at 4096 x 4095, within 1% at three rounds; with two rounds slower:
        // 15.1 -> 15.5 us at 1024 x 8191, 15.3 -> 15.5 at 2048 x 4095.
        auto ks = k_general_reg<B, 1, R, true, false, true>;
        const int64_t res = resident(ks, B, (size_t)B * 16);
        const int64_t slots = grid > 0 && grid < res ? grid : res;
        if (slots > 0 && p.n_rows >= 3 * slots)
          return go_general_reg_k<B, 1, R, true, false, true>(p, grid, s);
      }
      if (general_lines(p.hidden)) return go_general_reg_k<B, 1, R, true>(p, grid, s);
      return go_general_reg_k<B, 1, R, false>(p, grid, s);
    case 2:
      if (full && general_lines(p.hidden) && shared_line_offsets<R>(p)) {
        // As above (measured on MI355X: 52.2 -> 51.0 us at 2048 x 16383,
        // 98.3 -> 94.7 us at 4096 x 16383, 53.2 -> 51.4 us at 2048 x 16001).
        auto ks = k_general_reg<B, 2, R, true, true, true>;
        const int64_t res = resident(ks, B, (size_t)B * 32);
        const int64_t slots = grid > 0 && grid < res ? grid : res;
        if (slots > 0 && p.n_rows >= 3 * slots)
          return go_general_reg_k<B, 2, R, true, true, true>(p, grid, s);
      }
      if (full && general_lines(p.hidden)) return go_general_reg_k<B, 2, R, true, true>(p, grid, s);
      // Rows with blocks past their end keep the row-relative form, but with
      // every tensor at one line offset the whole-line form beats it
      // (measured on MI355X: 58.1 -> 56.1 us at 4096 x 9001, 80.0 -> 74.7 us
      // at 4096 x 12287, 36.0 -> 33.3 us at 2048 x 10001, 90.8 -> 83.8 us at
      // 4096 x 14001), also with a short last block when more than half of
      // the blocks hold row elements (43.7 -> 40.3 us at 2048 x 12289, 66.6
      // -> 63.6 us at 4096 x 10300, 49.6 -> 46.9 us at 2048 x 14400).
      if ((general_lines(p.hidden) || 512 * (B / 64) < p.hidden) && shared_line_offsets<R>(p)) {
        auto ks = k_general_reg<B, 2, R, true, false, true>;
        const int64_t res = resident(ks, B, (size_t)B * 32);
        const int64_t slots = grid > 0 && grid < res ? grid : res;
        if (slots > 0 && p.n_rows >= 3 * slots)
          return go_general_reg_k<B, 2, R, true, false, true>(p, grid, s);
      }
      if (full) return go_general_reg_k<B, 2, R, false, true>(p, grid, s);
      return go_general_reg_k<B, 2, R, false>(p, grid, s);
    case 4:
      if constexpr (B * 4 <= 2048) {
        if (full) return go_general_reg_k<B, 4, R, false, true>(p, grid, s);
        return go_general_reg_k<B, 4, R, false>(p, grid, s);
      }
      break;
  }
  return hipErrorInvalidValue;
}

template <bool R, int WAVES>
hipError_t go_general_wave(const GenParams& p, int j, int64_t grid, hipStream_t s) {
  const int64_t groups = (p.n_rows + WAVES - 1) / WAVES;
  if (j == 1) {
    auto k = k_general_wave<WAVES, 1, R>;
    if (grid == -1) grid = resident(k, WAVES * 64, 0);
    hipLaunchKernelGGL(k, dim3(grid_for(grid, groups)), dim3(WAVES * 64), 0, s, p);
  } else {
    auto k = k_general_wave<WAVES, 2, R>;
    if (grid == -1) grid = resident(k, WAVES * 64, 0);
    hipLaunchKernelGGL(k, dim3(grid_for(grid, groups)), dim3(WAVES * 64), 0, s, p);
  }
  return hipGetLastError();
}

template <bool R>
hipError_t general_wave_by_block(const GenParams& p, int b, int j, int64_t grid, hipStream_t s) {
  switch (b) {
    case 64: return go_general_wave<R, 1>(p, j, grid, s);
    case 128: return go_general_wave<R, 2>(p, j, grid, s);
    case 256: return go_general_wave<R, 4>(p, j, grid, s);
    case 512: return go_general_wave<R, 8>(p, j, grid, s);
    case 1024: return go_general_wave<R, 16>(p, j, grid, s);
  }
  return hipErrorInvalidValue;
}

template <bool R>
hipError_t general_reg_by_block(const GenParams& p, int b, int j, int64_t grid, hipStream_t s) {
  switch (b) {
    case 64: return go_general_reg<R, 64>(p, j, grid, s);
    case 128: return go_general_reg<R, 128>(p, j, grid, s);
    case 256: return go_general_reg<R, 256>(p, j, grid, s);
    case 512: return go_general_reg<R, 512>(p, j, grid, s);
    case 1024: return go_general_reg<R, 1024>(p, j, grid, s);
  }
  return hipErrorInvalidValue;
}

template <bool R>
hipError_t general_by_block(const GenParams& p, int b, int hidden, int64_t grid, hipStream_t s) {
  switch (b) {
    case 64: return go_general<R, 64>(p, hidden, grid, s);
    case 128: return go_general<R, 128>(p, hidden, grid, s);
    case 256: return go_general<R, 256>(p, hidden, grid, s);
    case 512: return go_general<R, 512>(p, hidden, grid, s);
    case 1024: return go_general<R, 1024>(p, hidden, grid, s);
  }
  return hipErrorInvalidValue;
}

// The variant is chosen by the arguments: quantised, in the format qfmt,
// when codes are requested, plain when there is no residual.
hipError_t launch_wave_row(const FwdArgs& a, int block_threads, int segs_per_lane,
                           int64_t grid_blocks, hipStream_t s) {
  const Params p = make_params(a);
  const int b = block_threads, j = segs_per_lane;
  if (a.qout && a.qfmt == kQInt8)
    return a.residual ? wave_by_block<kQInt8, true>(p, b, j, grid_blocks, s)
                      : wave_by_block<kQInt8, false>(p, b, j, grid_blocks, s);
  if (a.qout && a.qfmt == kQFp8)
    return a.residual ? wave_by_block<kQFp8, true>(p, b, j, grid_blocks, s)
                      : wave_by_block<kQFp8, false>(p, b, j, grid_blocks, s);
  if (a.qout) return hipErrorInvalidValue;
  return a.residual ? wave_by_block<0, true>(p, b, j, grid_blocks, s)
                    : wave_by_block<0, false>(p, b, j, grid_blocks, s);
}

hipError_t launch_wg_row(const FwdArgs& a, int block_threads, int segs_per_thread,
                         int64_t grid_blocks, bool late_weight, hipStream_t s) {
  const Params p = make_params(a);
  const int b = block_threads, j = segs_per_thread;
  const bool l = late_weight;
  if (a.qout && a.qfmt == kQInt8)
    return a.residual ? wg_by_block<kQInt8, true>(p, b, j, grid_blocks, l, s)
                      : wg_by_block<kQInt8, false>(p, b, j, grid_blocks, l, s);
  if (a.qout && a.qfmt == kQFp8)
    return a.residual ? wg_by_block<kQFp8, true>(p, b, j, grid_blocks, l, s)
                      : wg_by_block<kQFp8, false>(p, b, j, grid_blocks, l, s);
  if (a.qout) return hipErrorInvalidValue;
  return a.residual ? wg_by_block<0, true>(p, b, j, grid_blocks, l, s)
                    : wg_by_block<0, false>(p, b, j, grid_blocks, l, s);
}

hipError_t launch_lds_two_pass(const FwdArgs& a, int block_threads, int64_t grid_blocks,
                               hipStream_t s) {
  const Params p = make_params(a);
  const int b = block_threads, h = a.hidden;
  if (a.qout && a.qfmt == kQInt8)
    return a.residual ? two_pass_by_block<kQInt8, true>(p, b, h, grid_blocks, s)
                      : two_pass_by_block<kQInt8, false>(p, b, h, grid_blocks, s);
  if (a.qout && a.qfmt == kQFp8)
    return a.residual ? two_pass_by_block<kQFp8, true>(p, b, h, grid_blocks, s)
                      : two_pass_by_block<kQFp8, false>(p, b, h, grid_blocks, s);
  if (a.qout) return hipErrorInvalidValue;
  return a.residual ? two_pass_by_block<0, true>(p, b, h, grid_blocks, s)
                    : two_pass_by_block<0, false>(p, b, h, grid_blocks, s);
}

bool wave_row_supported(int block_threads, int segs_per_lane) {
  return !(block_threads == 1024 && segs_per_lane == 8);
}

bool wg_row_supported(int block_threads, int segs_per_thread) {
  return block_threads * segs_per_thread <= 2048;
}

size_t lds_two_pass_lds_bytes(int hidden) {
  return (size_t)(hidden / 8) * 32 + (size_t)two_pass_nb(hidden) * sizeof(float) + 64;
}

hipError_t launch_general(const FwdArgs& a, int block_threads, int64_t grid_blocks,
                          hipStream_t s) {
  GenParams p;
  p.out = a.out;
  p.residual_out = a.residual_out;
  p.x = a.x;
  p.residual = a.residual;
  p.weight = a.weight;
  p.n_rows = a.n_rows;
  p.x_stride = a.x_stride;
  p.r_stride = a.r_stride;
  p.out_stride = a.out_stride;
  p.ro_stride = a.ro_stride;
  p.hidden = a.hidden;
  p.hidden_f = (float)a.hidden;
  p.eps = a.eps;
  // Rows of at most 128 segments take one wavefront each; other rows that fit
  // in registers (at most 4 segments per thread and 2048 per workgroup) the
  // register-resident kernel, the rest the LDS one.  Rows of 65-128 segments
  // whose tensors all share a line offset, with a last block of more than
  // 128 elements, take the register kernel too, for its whole-line form
  // (measured on MI355X: 30.1 -> 27.7 us at 16384 x 1001, 56.4 -> 52.2 us at
  // 32768 x 1000, 111.0 -> 103.1 us at 65536 x 1000; with a short last block
  // slower: 36.3 -> 41.1 us at 32768 x 600).
  const int segs = (a.hidden + 7) / 8;
  const bool whole_lines = segs > 64 && general_lines(a.hidden) &&
                           (a.residual ? shared_line_offsets<true>(p) : shared_line_offsets<false>(p));
  if (segs <= 128 && !whole_lines) {
    const int jw = segs <= 64 ? 1 : 2;
    return a.residual ? general_wave_by_block<true>(p, block_threads, jw, grid_blocks, s)
                      : general_wave_by_block<false>(p, block_threads, jw, grid_blocks, s);
  }
  int j = 1;
  while (j * block_threads < segs) j *= 2;
  if (j <= 4 && j * block_threads <= 2048)
    return a.residual ? general_reg_by_block<true>(p, block_threads, j, grid_blocks, s)
                      : general_reg_by_block<false>(p, block_threads, j, grid_blocks, s);
  return a.residual ? general_by_block<true>(p, block_threads, a.hidden, grid_blocks, s)
                    : general_by_block<false>(p, block_threads, a.hidden, grid_blocks, s);
}

size_t general_lds_bytes(int hidden) {
  return (size_t)((hidden + 7) / 8) * 32 + (size_t)two_pass_nb(hidden) * 4 + 64;
}

namespace {

template <int P, int U, int Q, bool R>
hipError_t go_pack(const PackParams& p, int block_threads, int64_t grid_blocks, hipStream_t s) {
  const int64_t iters = ((int64_t)p.total + (64 / P) * U - 1) / ((64 / P) * U);
  const int waves = block_threads / 64;
  const int64_t groups = (iters + waves - 1) / waves;
  switch (block_threads) {
#define ADDRMS_PACK_CASE(B)                                                          \
  case B: {                                                                          \
    auto k = k_pack_rows<B / 64, P, U, Q, R>;                                        \
    const int64_t g = grid_blocks == -1 ? resident(k, B, 0) : grid_blocks;          \
    hipLaunchKernelGGL(k, dim3(grid_for(g, groups)), dim3(B), 0, s, p);              \
    return hipGetLastError();                                                        \
  }
    ADDRMS_PACK_CASE(64)
    ADDRMS_PACK_CASE(128)
    ADDRMS_PACK_CASE(256)
    ADDRMS_PACK_CASE(512)
    ADDRMS_PACK_CASE(1024)
#undef ADDRMS_PACK_CASE
  }
  return hipErrorInvalidValue;
}

template <int P, int Q, bool R>
hipError_t pack_by_u(const PackParams& p, int b, int u, int64_t grid, hipStream_t s) {
  switch (u) {
    case 1: return go_pack<P, 1, Q, R>(p, b, grid, s);
    case 2: return go_pack<P, 2, Q, R>(p, b, grid, s);
    case 4: return go_pack<P, 4, Q, R>(p, b, grid, s);
  }
  return hipErrorInvalidValue;
}

template <int Q, bool R>
hipError_t pack_by_p(const PackParams& p, int lanes, int b, int u, int64_t grid,
                     hipStream_t s) {
  switch (lanes) {
    case 1: return pack_by_u<1, Q, R>(p, b, u, grid, s);
    case 2: return pack_by_u<2, Q, R>(p, b, u, grid, s);
    case 4: return pack_by_u<4, Q, R>(p, b, u, grid, s);
    case 8: return pack_by_u<8, Q, R>(p, b, u, grid, s);
    case 16: return pack_by_u<16, Q, R>(p, b, u, grid, s);
    case 32: return pack_by_u<32, Q, R>(p, b, u, grid, s);
    case 64: return pack_by_u<64, Q, R>(p, b, u, grid, s);
  }
  return hipErrorInvalidValue;
}

PackGroup make_group(const PackTensors& t) {
  PackGroup g;
  g.out = reinterpret_cast<u32x4*>(t.out);
  g.qout = reinterpret_cast<u32x2*>(t.qout);
  g.qscale = t.qscale;
  g.residual_out = reinterpret_cast<u32x4*>(t.residual_out);
  g.x = reinterpret_cast<const u32x4*>(t.x);
  g.residual = reinterpret_cast<const u32x4*>(t.residual);
  g.weight = reinterpret_cast<const u32x4*>(t.weight);
  g.x_ts = t.x_token_stride / 8;
  g.r_ts = t.r_token_stride / 8;
  g.out_ts = t.out_token_stride / 8;
  g.ro_ts = t.ro_token_stride / 8;
  g.n_rows = (uint32_t)(t.n_tokens * t.heads);
  g.heads = t.heads > 0 ? (uint32_t)t.heads : 1u;
  const uint64_t m = g.heads > 1 ? ~0ull / g.heads + 1 : 0;
  g.magic_lo = (uint32_t)m;
  g.magic_hi = (uint32_t)(m >> 32);
  return g;
}

}  // namespace

hipError_t launch_pack_rows(const PackTensors& g0, const PackTensors& g1, int32_t hidden,
                            float eps, int qfmt, int block_threads, int rows_per_lane,
                            int64_t grid_blocks, hipStream_t s) {
  PackParams p;
  p.g[0] = make_group(g0);
  p.g[1] = make_group(g1);
  p.segs = hidden / 8;
  int lanes = 1;
  while (lanes < p.segs) lanes *= 2;
  const uint64_t per_iter = (uint64_t)(64 / lanes) * (uint64_t)rows_per_lane;
  const uint64_t first1 = ((uint64_t)p.g[0].n_rows + per_iter - 1) / per_iter * per_iter;
  p.first1 = (uint32_t)first1;
  p.total = (uint32_t)(first1 + p.g[1].n_rows);
  p.hidden_f = (float)hidden;
  p.eps = eps;
  const int b = block_threads, u = rows_per_lane;
  if (qfmt == kQInt8)
    return g0.residual ? pack_by_p<kQInt8, true>(p, lanes, b, u, grid_blocks, s)
                       : pack_by_p<kQInt8, false>(p, lanes, b, u, grid_blocks, s);
  if (qfmt == kQFp8)
    return g0.residual ? pack_by_p<kQFp8, true>(p, lanes, b, u, grid_blocks, s)
                       : pack_by_p<kQFp8, false>(p, lanes, b, u, grid_blocks, s);
  if (qfmt != 0) return hipErrorInvalidValue;
  return g0.residual ? pack_by_p<0, true>(p, lanes, b, u, grid_blocks, s)
                     : pack_by_p<0, false>(p, lanes, b, u, grid_blocks, s);
}

hipError_t launch_stream(uint16_t* dst, const uint16_t* src, int64_t count, int mode,
                         hipStream_t s) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t segs = count / 8;
  // The fastest grids of sweeps on MI355X: reads as launch_copy2; writes
  // with a few 16-byte stores per thread (5.9-6.2 TB/s, against 4.7 at 32
  // workgroups per CU).
  int64_t blocks = (int64_t)cus * (mode == 0 ? 32 : 512);
  const int64_t need = (segs + 255) / 256;
  if (blocks > need) blocks = need;
  if (blocks < 1) blocks = 1;
  if (mode == 0)
    hipLaunchKernelGGL(k_stream_read, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<u32x4*>(dst), reinterpret_cast<const u32x4*>(src), segs);
  else
    hipLaunchKernelGGL(k_stream_write, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<u32x4*>(dst), segs);
  return hipGetLastError();
}

hipError_t launch_copy2(uint16_t* d0, uint16_t* d1, const uint16_t* s0, const uint16_t* s1,
                        int64_t count, hipStream_t s) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t segs = count / 8;
  int64_t blocks = (int64_t)cus * 32;  // fastest grid of the copy sweeps on MI355X
  const int64_t need = (segs + 255) / 256;
  if (blocks > need) blocks = need;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_copy2, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<u32x4*>(d0),
                     reinterpret_cast<u32x4*>(d1), reinterpret_cast<const u32x4*>(s0),
                     reinterpret_cast<const u32x4*>(s1), segs);
  return hipGetLastError();
}

template <int R>
hipError_t go_copy_rows(u32x4* d0, u32x4* d1, const u32x4* s0, const u32x4* s1, int64_t n_rows,
                        int segs, hipStream_t s) {
  const int64_t g = (n_rows + R - 1) / R;
  const unsigned grid = (unsigned)(g < ((int64_t)1 << 30) ? g : ((int64_t)1 << 30));
  const int j = (segs + 511) / 512;
  if (g > ((int64_t)1 << 30)) return hipErrorInvalidValue;
  switch (j) {
    case 1: hipLaunchKernelGGL((k_copy_rows<R, 1>), dim3(grid), dim3(512), 0, s, d0, d1, s0, s1, n_rows, segs); break;
    case 2: hipLaunchKernelGGL((k_copy_rows<R, 2>), dim3(grid), dim3(512), 0, s, d0, d1, s0, s1, n_rows, segs); break;
    case 3:
    case 4: hipLaunchKernelGGL((k_copy_rows<R, 4>), dim3(grid), dim3(512), 0, s, d0, d1, s0, s1, n_rows, segs); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_copy_rows(uint16_t* d0, uint16_t* d1, const uint16_t* s0, const uint16_t* s1,
                            int64_t n_rows, int hidden, int rows_per_burst, hipStream_t s) {
  u32x4* a = reinterpret_cast<u32x4*>(d0);
  u32x4* b = reinterpret_cast<u32x4*>(d1);
  const u32x4* c = reinterpret_cast<const u32x4*>(s0);
  const u32x4* d = reinterpret_cast<const u32x4*>(s1);
  const int segs = hidden / 8;
  switch (rows_per_burst) {
    case 1: return go_copy_rows<1>(a, b, c, d, n_rows, segs, s);
    case 2: return go_copy_rows<2>(a, b, c, d, n_rows, segs, s);
    case 4: return go_copy_rows<4>(a, b, c, d, n_rows, segs, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_cvt_e4m3_range(uint8_t* out, uint32_t start, int64_t count, hipStream_t s) {
  const int64_t groups = count / 8;
  int64_t blocks = (groups + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_cvt_e4m3_range, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<u32x2*>(out), start, groups);
  return hipGetLastError();
}

hipError_t launch_cvt_range(uint16_t* out, uint32_t start, int64_t count, hipStream_t s) {
  const int64_t groups = count / 8;
  int64_t blocks = (groups + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_cvt_range, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<u32x4*>(out), start, groups);
  return hipGetLastError();
}

}  // namespace addrms
