// C entry points of the fused residual-add + RMSNorm forward, of plain
// RMSNorm (bf16 or int8 out) and of the correctly rounded binary32 log1p:
// argument validation (on the host, before anything is enqueued), kernel
// choice, launch on the caller's stream.  The contracts are documented in
// include/add_rmsnorm.h and include/log1p_f32.h.
#include "add_rmsnorm.h"
#include "log1p_f32.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>

#include "launch.h"

#ifndef ADD_RMSNORM_BUILD_INFO
#define ADD_RMSNORM_BUILD_INFO "unknown build"
#endif

namespace {

thread_local char g_hip_error[256] = "no HIP error recorded";

int hip_failure(hipError_t e) {
  std::snprintf(g_hip_error, sizeof g_hip_error, "%s: %s", hipGetErrorName(e),
                hipGetErrorString(e));
  return ADD_RMSNORM_EHIP;
}

bool overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uint64_t pa = reinterpret_cast<uintptr_t>(a);
  const uint64_t pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }
bool aligned16(const void* p) { return aligned(p, 16); }

bool valid_block(int b) { return b == 64 || b == 128 || b == 256 || b == 512 || b == 1024; }
bool valid_rows_per_lane(int u) { return u == 1 || u == 2 || u == 4; }

// Smallest of 1, 2, 4, 8 that is >= need (0 if none).
int pow2_at_least(int64_t need) {
  for (int j = 1; j <= 8; j *= 2)
    if (j >= need) return j;
  return 0;
}

// Default workgroup sizes per path.
constexpr int kPackThreads = 256;
constexpr int64_t kPackAutoMaxHidden = 256;
constexpr int64_t kPackAutoMaxHiddenQuant = 512;
constexpr int kPackRowsPerLane = 2;
constexpr int kWaveRowThreads = 256;
constexpr int kWgRowThreads = 512;
// The LDS two-pass kernel holds a whole row of fp32 sums in LDS (64 KiB at
// hidden 16384), so few workgroups fit on a CU; 1024 threads keep more
// wavefronts in flight than 512 (measured on MI355X: 1.5% faster at
// 2048 x 16384, 1.7% at 1024 x 32768, 0.3% slower at 4096 x 16384).
constexpr int kTwoPassThreads = 1024;

// Default launch of log1p_f32: 256 threads, 4 consecutive elements each.
constexpr int kLog1pThreads = 256;
constexpr int kLog1pElems = 4;

// Upper hidden sizes of the automatic choice.
constexpr int64_t kWaveRowMaxHidden = 2048;
constexpr int64_t kWgRowMaxHidden = 8192;
// Small fused bf16 calls: hidden in [2048, 8192], at most 4096 rows and x and
// residual together at most 64 MiB (2^24 elements each) take the register
// kernel with a small workgroup and the weight read after each row's barrier.
// Measured on MI355X against the large-call defaults: +3% at 2048 x 2048, +5%
// at 4096 x 2048, +14% at 1024 x 4096, +8% at 2048 x 4096, +4% at 3072 x
// 4096, +10% at 1024 x 8192, +4% at 2048 x 8192; within 1% at the edges of
// the range (4096 x 4096, 8192 x 2048) and slower beyond it.
constexpr int64_t kSmallCallMinHidden = 2048;
constexpr int64_t kSmallCallMaxRows = 4096;
constexpr int64_t kSmallCallMaxElems = (int64_t)1 << 24;

// Workgroup size of a small call: about 2^18 threads in all (the fastest
// totals measured), at least 64, at most 8 segments per thread and no more
// threads than segments.
int small_call_threads(int64_t n_rows, int64_t segs) {
  int b = 64;
  while (b < 1024 && (int64_t)b * 2 * n_rows <= ((int64_t)1 << 18)) b *= 2;
  while (b < 1024 && (int64_t)b * 8 < segs) b *= 2;
  while (b > 64 && b > segs) b /= 2;
  return b;
}
// ... for the quantised and plain variants, and their workgroup size up to
// hidden 2048.
constexpr int64_t kVariantWaveRowMaxHidden = 1024;
constexpr int64_t kVariantWgRowMaxHidden = 16384;
constexpr int kVariantWgRowSmallThreads = 128;
// Plain quantised out: two segments per thread (rather than four) up to this
// many elements per call, for hidden up to 8192.
constexpr int64_t kPlainQuantTwoSegMaxElems = (int64_t)1 << 25;
// Plain bf16 small calls: hidden 4096-8192 and at most 2^23 elements per call.
constexpr int64_t kPlainSmallMinHidden = 4096;
constexpr int64_t kPlainSmallMaxElems = (int64_t)1 << 23;

// The device's LDS limit per workgroup, asked of the runtime once per device
// (a device attribute never changes; the query costs host time per call).
constexpr int kMaxCachedDevices = 64;
std::atomic<int> g_max_lds[kMaxCachedDevices];  // 0: not asked yet

int device_max_lds(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_failure(e);
  if (dev >= 0 && dev < kMaxCachedDevices) {
    const int v = g_max_lds[dev].load(std::memory_order_relaxed);
    if (v > 0) {
      *out = v;
      return ADD_RMSNORM_OK;
    }
  }
  e = hipDeviceGetAttribute(out, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return hip_failure(e);
  if (dev >= 0 && dev < kMaxCachedDevices && *out > 0)
    g_max_lds[dev].store(*out, std::memory_order_relaxed);
  return ADD_RMSNORM_OK;
}

// Scalar arguments and the launch configuration, shared by both variants.
int check_scalars(int64_t n_rows, int64_t hidden, float eps,
                  const add_rmsnorm_launch_cfg* cfg, add_rmsnorm_launch_cfg* c) {
  if (n_rows < 0 || hidden <= 0 || !std::isfinite(eps) || eps < 0.0f) return ADD_RMSNORM_EINVAL;
  if (hidden % 8 != 0) return ADD_RMSNORM_EALIGN;
  if (hidden > ADD_RMSNORM_MAX_HIDDEN) return ADD_RMSNORM_ERANGE;
  *c = add_rmsnorm_launch_cfg{ADD_RMSNORM_PATH_AUTO, 0, 0, 0};
  if (cfg) *c = *cfg;
  if (c->grid_blocks < -1) return ADD_RMSNORM_EINVAL;
  if (c->path < ADD_RMSNORM_PATH_AUTO ||
      (c->path > ADD_RMSNORM_PATH_LDS_TWO_PASS && c->path != ADD_RMSNORM_PATH_PACKED))
    return ADD_RMSNORM_EINVAL;
  if (c->flags != 0 && !(c->path == ADD_RMSNORM_PATH_PACKED && valid_rows_per_lane(c->flags)))
    return ADD_RMSNORM_EINVAL;
  if (c->block_threads != 0 && !valid_block(c->block_threads)) return ADD_RMSNORM_EINVAL;
  return ADD_RMSNORM_OK;
}

// A bf16 output against the inputs and the weight: disjoint, or exactly x or
// residual (in place: every element is read and rewritten by the same thread,
// the stored value depending on the loaded one).
bool output_aliases_badly(const void* o, uint64_t t_bytes, const void* x, const void* residual,
                          const void* weight, uint64_t row_bytes) {
  if (overlap(o, t_bytes, weight, row_bytes)) return true;
  if (o != x && overlap(o, t_bytes, x, t_bytes)) return true;
  if (o != residual && overlap(o, t_bytes, residual, t_bytes)) return true;
  return false;
}

// Scalar arguments and launch configuration of the bf16-out entry points,
// which take any hidden in [1, ADD_RMSNORM_MAX_HIDDEN] and the general path.
int check_scalars_any_hidden(int64_t n_rows, int64_t hidden, float eps,
                             const add_rmsnorm_launch_cfg* cfg, add_rmsnorm_launch_cfg* c) {
  if (n_rows < 0 || hidden <= 0 || !std::isfinite(eps) || eps < 0.0f) return ADD_RMSNORM_EINVAL;
  if (hidden > ADD_RMSNORM_MAX_HIDDEN) return ADD_RMSNORM_ERANGE;
  *c = add_rmsnorm_launch_cfg{ADD_RMSNORM_PATH_AUTO, 0, 0, 0};
  if (cfg) *c = *cfg;
  if (c->grid_blocks < -1) return ADD_RMSNORM_EINVAL;
  if (c->path < ADD_RMSNORM_PATH_AUTO || c->path > ADD_RMSNORM_PATH_PACKED)
    return ADD_RMSNORM_EINVAL;
  if (c->flags != 0 && !(c->path == ADD_RMSNORM_PATH_PACKED && valid_rows_per_lane(c->flags)) &&
      !(c->path == ADD_RMSNORM_PATH_WG_ROW && c->flags == ADD_RMSNORM_FLAG_LATE_WEIGHT))
    return ADD_RMSNORM_EINVAL;
  if (c->block_threads != 0 && !valid_block(c->block_threads)) return ADD_RMSNORM_EINVAL;
  return ADD_RMSNORM_OK;
}

// A row-strided view: n rows of `width` bytes, `stride` bytes apart.
struct View {
  const void* p;
  uint64_t stride;
};

int64_t floor_div(int64_t a, int64_t b) {  // b > 0
  int64_t q = a / b;
  if ((a % b != 0) && (a < 0)) --q;
  return q;
}

// Whether two views of n rows of `width` bytes share a byte.  Views with one
// stride s meet exactly when some row difference q in [-(n-1), n-1] puts the
// base difference within a row width of q * s; views with different strides
// are taken to meet whenever their spans do.
bool views_overlap(View a, View b, int64_t n, uint64_t width) {
  const uint64_t span_a = (uint64_t)(n - 1) * a.stride + width;
  const uint64_t span_b = (uint64_t)(n - 1) * b.stride + width;
  if (!overlap(a.p, span_a, b.p, span_b)) return false;
  if (a.stride != b.stride) return true;
  const int64_t d = (int64_t)(reinterpret_cast<uintptr_t>(b.p) - reinterpret_cast<uintptr_t>(a.p));
  const int64_t s = (int64_t)a.stride;
  const int64_t q = floor_div(d, s);
  for (int64_t qq = q; qq <= q + 1; ++qq) {
    if (qq < -(n - 1) || qq > n - 1) continue;
    const int64_t r = d - qq * s;
    if (r > -(int64_t)width && r < (int64_t)width) return true;
  }
  return false;
}

// views_overlap for views of different widths (wa, wb bytes per row): with
// one stride s they meet exactly when some row difference q in [-(n-1), n-1]
// puts r = d + q s, d = b - a, inside (-wb, wa).  Different strides: as above.
bool views_overlap2(View a, uint64_t wa, View b, uint64_t wb, int64_t n) {
  const uint64_t span_a = (uint64_t)(n - 1) * a.stride + wa;
  const uint64_t span_b = (uint64_t)(n - 1) * b.stride + wb;
  if (!overlap(a.p, span_a, b.p, span_b)) return false;
  if (a.stride != b.stride) return true;
  const int64_t d = (int64_t)(reinterpret_cast<uintptr_t>(b.p) - reinterpret_cast<uintptr_t>(a.p));
  const int64_t s = (int64_t)a.stride;
  int64_t q_lo = floor_div(-(int64_t)wb - d, s) + 1;      // first q with r > -wb
  int64_t q_hi = -floor_div(-((int64_t)wa - d), s) - 1;  // last q with r < wa
  if (q_lo < -(n - 1)) q_lo = -(n - 1);
  if (q_hi > n - 1) q_hi = n - 1;
  return q_lo <= q_hi;
}

// Whether a view of n rows of `width` bytes shares a byte with the range
// [q, q + len): some row i in [0, n) with i s < d + len and i s + width > d,
// d = q - base.
bool view_meets_range(View v, int64_t n, uint64_t width, const void* q, uint64_t len) {
  const int64_t d = (int64_t)(reinterpret_cast<uintptr_t>(q) - reinterpret_cast<uintptr_t>(v.p));
  const int64_t s = (int64_t)v.stride;
  int64_t i_min = floor_div(d - (int64_t)width, s) + 1;  // first row ending after d
  int64_t i_max = -floor_div(-(d + (int64_t)len), s) - 1;  // last row starting before d + len
  if (i_min < 0) i_min = 0;
  if (i_max > n - 1) i_max = n - 1;
  return i_min <= i_max;
}

// An output view against an input view: the very same view (in place), or
// no shared byte.
bool output_meets_input(View o, View in, int64_t n, uint64_t width) {
  if (o.p == in.p && o.stride == in.stride) return false;
  return views_overlap(o, in, n, width);
}

// Kernel choice by hidden (or as forced) and launch.
int dispatch(const addrms::FwdArgs& a, const add_rmsnorm_launch_cfg& c,
             struct ihipStream_t* stream) {
  int path = c.path;
  int block = c.block_threads;
  const int64_t hidden = a.hidden;
  // The weight read after each row's barrier (bf16 out on the register kernel).
  bool late = path == ADD_RMSNORM_PATH_WG_ROW && c.flags == ADD_RMSNORM_FLAG_LATE_WEIGHT;
  // The quantised and plain variants keep rows in registers further: measured
  // on MI355X, one workgroup per row beats one wavefront per row at hidden
  // 2048 (by 5-13%) and the LDS two-pass kernel up to 16384 (by 7-25%).
  const bool variant = a.qout != nullptr || a.residual == nullptr;
  // Short rows pack several to a wavefront.  Measured on MI355X against one
  // wavefront per row: bf16 out 1.2-3.9x at hidden 64-256, and as fast or
  // slower at 512; quantised out 1.5-6x at 64-256 and 2-8% faster at 512.
  if (path == ADD_RMSNORM_PATH_AUTO &&
      hidden <= (a.qout ? kPackAutoMaxHiddenQuant : kPackAutoMaxHidden) &&
      a.n_rows < addrms::kPackMaxRows)
    path = ADD_RMSNORM_PATH_PACKED;
  // Plain bf16 small calls take one workgroup per row (see below).
  bool plain_small = false;
  if (path == ADD_RMSNORM_PATH_AUTO && variant) {
    if (hidden <= kVariantWaveRowMaxHidden) {
      path = ADD_RMSNORM_PATH_WAVE_ROW;
    } else if (hidden <= kVariantWgRowMaxHidden) {
      path = ADD_RMSNORM_PATH_WG_ROW;
      if (block == 0 && a.qout != nullptr && a.residual == nullptr) {
        // Plain quantised out: two segments per thread up to hidden 8192 and
        // 2^25 elements, four beyond (measured on MI355X against four
        // everywhere: 1-13% faster in that range, even at its edge, 3% slower
        // at 16384 x 4096 and 35-40% at hidden 16384).
        const int per = hidden <= kWgRowMaxHidden && a.n_rows * hidden <= kPlainQuantTwoSegMaxElems
                            ? 2 : 4;
        block = 64;
        while (block < 1024 && block * per * 8 < hidden) block *= 2;
      } else if (block == 0 && a.qout == nullptr && a.residual == nullptr &&
                 hidden >= kPlainSmallMinHidden && hidden <= kWgRowMaxHidden &&
                 a.n_rows * hidden <= kPlainSmallMaxElems) {
        // Plain bf16 small calls: the fused op's small-call workgroup, one
        // workgroup per row (measured on MI355X against the resident grid of
        // 512 threads: 1-14% faster from 512 x 4096 to 1024 x 8192; 9-13%
        // slower at 3072 x 8192 and 4096 x 4096, beyond the range).
        block = small_call_threads(a.n_rows, hidden / 8);
        plain_small = true;
      } else if (block == 0 && hidden <= kWaveRowMaxHidden) {
        block = kVariantWgRowSmallThreads;
      }
    } else {
      path = ADD_RMSNORM_PATH_LDS_TWO_PASS;
    }
  } else if (path == ADD_RMSNORM_PATH_AUTO) {
    if (hidden >= kSmallCallMinHidden && hidden <= kWgRowMaxHidden &&
        a.n_rows <= kSmallCallMaxRows && a.n_rows * hidden <= kSmallCallMaxElems) {
      path = ADD_RMSNORM_PATH_WG_ROW;
      late = true;
      if (block == 0) block = small_call_threads(a.n_rows, hidden / 8);
    } else {
      path = hidden <= kWaveRowMaxHidden ? ADD_RMSNORM_PATH_WAVE_ROW
             : hidden <= kWgRowMaxHidden ? ADD_RMSNORM_PATH_WG_ROW
                                         : ADD_RMSNORM_PATH_LDS_TWO_PASS;
    }
  }
  const int64_t segs = hidden / 8;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (path == ADD_RMSNORM_PATH_PACKED) {
    if (hidden > addrms::kPackMaxHidden || a.n_rows >= addrms::kPackMaxRows)
      return ADD_RMSNORM_ERANGE;
    const addrms::PackTensors g0 = {a.out, a.qout, a.qscale, a.residual_out, a.x, a.residual,
                                    a.weight, a.x_stride, a.r_stride, a.out_stride,
                                    a.ro_stride, a.n_rows, 1};
    const addrms::PackTensors g1 = {};
    e = addrms::launch_pack_rows(g0, g1, (int32_t)hidden, a.eps, a.qout ? a.qfmt : 0,
                                 block ? block : kPackThreads,
                                 c.flags ? c.flags : kPackRowsPerLane,
                                 c.grid_blocks ? c.grid_blocks : -1, s);
    return e != hipSuccess ? hip_failure(e) : ADD_RMSNORM_OK;
  }
  // Plain RMSNorm (bf16 or int8 out) launches, by default, as many
  // workgroups as fit, looping over rows: each workgroup then reads the
  // weight once, which for these rows is as many bytes as x itself (measured
  // 7-16% faster on MI355X; the fused kernels gain nothing from it).
  int64_t grid = c.grid_blocks;
  if (grid == 0 && a.residual == nullptr && path != ADD_RMSNORM_PATH_GENERAL && !plain_small)
    grid = -1;
  if (path == ADD_RMSNORM_PATH_GENERAL) {
    // Rows up to 1024 take one wavefront each, four rows per workgroup.
    // Longer rows take one workgroup each, by default with one segment per
    // thread (the fewest registers, so the most rows in flight): the smallest
    // workgroup that covers the row, 64 to 1024 threads; two segments per
    // thread at 1024 threads up to 16384, and the long-row kernel above.
    int b = c.block_threads;
    if (b == 0 && hidden <= 1024) {
      b = 256;
    } else if (b == 0) {
      b = 64;
      while (b < 1024 && b * 8 < hidden) b *= 2;
    }
    int max_lds = 0;
    const int rc = device_max_lds(&max_lds);
    if (rc != ADD_RMSNORM_OK) return rc;
    if (addrms::general_lds_bytes((int)hidden) > (size_t)max_lds) return ADD_RMSNORM_ERANGE;
    // By default as many workgroups as fit, looping over rows: the weight is
    // staged in LDS once per workgroup (measured +15-50% over one per row).
    e = addrms::launch_general(a, b, c.grid_blocks == 0 ? -1 : c.grid_blocks, s);
  } else if (path == ADD_RMSNORM_PATH_WAVE_ROW) {
    const int b = block ? block : kWaveRowThreads;
    const int j = pow2_at_least((segs + 63) / 64);
    if (j == 0 || !addrms::wave_row_supported(b, j)) return ADD_RMSNORM_ERANGE;
    e = addrms::launch_wave_row(a, b, j, grid, s);
  } else if (path == ADD_RMSNORM_PATH_WG_ROW) {
    const int b = block ? block : kWgRowThreads;
    const int j = pow2_at_least((segs + b - 1) / b);
    if (j == 0 || !addrms::wg_row_supported(b, j)) return ADD_RMSNORM_ERANGE;
    e = addrms::launch_wg_row(a, b, j, grid, late, s);
  } else {
    const int b = block ? block : kTwoPassThreads;
    int max_lds = 0;
    const int rc = device_max_lds(&max_lds);
    if (rc != ADD_RMSNORM_OK) return rc;
    if (addrms::lds_two_pass_lds_bytes((int)hidden) > (size_t)max_lds) return ADD_RMSNORM_ERANGE;
    e = addrms::launch_lds_two_pass(a, b, grid, s);
  }
  if (e != hipSuccess) return hip_failure(e);
  return ADD_RMSNORM_OK;
}

// The bf16-out forward over row-strided views (fused when `fused`, else
// plain RMSNorm with residual and residual_out unused).  Strides in elements.
int fwd_strided(uint16_t* out, int64_t out_stride, uint16_t* residual_out, int64_t ro_stride,
                const uint16_t* x, int64_t x_stride, const uint16_t* residual, int64_t r_stride,
                const uint16_t* weight, int64_t n_rows, int64_t hidden, float eps,
                const add_rmsnorm_launch_cfg* cfg, struct ihipStream_t* stream, bool fused) {
  add_rmsnorm_launch_cfg c;
  int rc = check_scalars_any_hidden(n_rows, hidden, eps, cfg, &c);
  if (rc != ADD_RMSNORM_OK) return rc;
  if (n_rows == 0) return ADD_RMSNORM_OK;

  if (!out || !x || !weight) return ADD_RMSNORM_EINVAL;
  if (fused && (!residual_out || !residual)) return ADD_RMSNORM_EINVAL;
  if (out_stride < hidden || x_stride < hidden) return ADD_RMSNORM_EINVAL;
  if (fused && (ro_stride < hidden || r_stride < hidden)) return ADD_RMSNORM_EINVAL;
  if (!aligned(out, 2) || !aligned(x, 2) || !aligned(weight, 2)) return ADD_RMSNORM_EALIGN;
  if (fused && (!aligned(residual_out, 2) || !aligned(residual, 2))) return ADD_RMSNORM_EALIGN;
  // Every view's span, (n_rows - 1) * stride + hidden elements, in bytes.
  const int64_t strides[4] = {out_stride, x_stride, fused ? ro_stride : hidden,
                              fused ? r_stride : hidden};
  for (int64_t st : strides)
    if ((uint64_t)(n_rows - 1) > ((uint64_t)INT64_MAX / 2 - (uint64_t)hidden) / (uint64_t)st)
      return ADD_RMSNORM_ERANGE;

  const uint64_t width = (uint64_t)hidden * 2;
  const View vo = {out, (uint64_t)out_stride * 2}, vx = {x, (uint64_t)x_stride * 2};
  const View vro = {residual_out, (uint64_t)ro_stride * 2}, vr = {residual, (uint64_t)r_stride * 2};
  // Outputs: disjoint from the weight and from each other; each either
  // disjoint from an input or exactly that input's view (in place).
  if (view_meets_range(vo, n_rows, width, weight, width)) return ADD_RMSNORM_EALIAS;
  if (output_meets_input(vo, vx, n_rows, width)) return ADD_RMSNORM_EALIAS;
  if (fused) {
    if (view_meets_range(vro, n_rows, width, weight, width)) return ADD_RMSNORM_EALIAS;
    if (views_overlap(vo, vro, n_rows, width)) return ADD_RMSNORM_EALIAS;
    if (output_meets_input(vo, vr, n_rows, width) || output_meets_input(vro, vx, n_rows, width) ||
        output_meets_input(vro, vr, n_rows, width))
      return ADD_RMSNORM_EALIAS;
  }

  // The fast kernels need hidden, every stride and every pointer on 8
  // elements (16 bytes); anything else takes the general kernel.
  bool fast = hidden % 8 == 0 && out_stride % 8 == 0 && x_stride % 8 == 0 && aligned16(out) &&
              aligned16(x) && aligned16(weight);
  if (fused)
    fast = fast && ro_stride % 8 == 0 && r_stride % 8 == 0 && aligned16(residual_out) &&
           aligned16(residual);
  if (!fast) {
    if (c.path == ADD_RMSNORM_PATH_AUTO) c.path = ADD_RMSNORM_PATH_GENERAL;
    if (c.path != ADD_RMSNORM_PATH_GENERAL) return ADD_RMSNORM_EALIGN;
  }
  addrms::FwdArgs a = {out, nullptr, nullptr, fused ? residual_out : nullptr, x,
                       fused ? residual : nullptr, weight, n_rows, (int32_t)hidden, eps,
                       x_stride, fused ? r_stride : 0, out_stride, fused ? ro_stride : 0};
  return dispatch(a, c, stream);
}

}  // namespace

extern "C" {

int add_rmsnorm_fwd_strided(uint16_t* out, int64_t out_stride, uint16_t* residual_out,
                            int64_t residual_out_stride, const uint16_t* x, int64_t x_stride,
                            const uint16_t* residual, int64_t residual_stride,
                            const uint16_t* weight, int64_t n_rows, int64_t hidden, float eps,
                            const struct add_rmsnorm_launch_cfg* cfg,
                            struct ihipStream_t* stream) {
  return fwd_strided(out, out_stride, residual_out, residual_out_stride, x, x_stride, residual,
                     residual_stride, weight, n_rows, hidden, eps, cfg, stream, true);
}

int add_rmsnorm_fwd_cfg(uint16_t* out, uint16_t* residual_out, const uint16_t* x,
                        const uint16_t* residual, const uint16_t* weight, int64_t n_rows,
                        int64_t hidden, float eps, const struct add_rmsnorm_launch_cfg* cfg,
                        struct ihipStream_t* stream) {
  return fwd_strided(out, hidden, residual_out, hidden, x, hidden, residual, hidden, weight,
                     n_rows, hidden, eps, cfg, stream, true);
}

int add_rmsnorm_fwd(uint16_t* out, uint16_t* residual_out, const uint16_t* x,
                    const uint16_t* residual, const uint16_t* weight, int64_t n_rows,
                    int64_t hidden, float eps, struct ihipStream_t* stream) {
  return add_rmsnorm_fwd_cfg(out, residual_out, x, residual, weight, n_rows, hidden, eps,
                             nullptr, stream);
}

}  // extern "C"

namespace {

// The quantised entry points, fused (residual set) or plain (residual and
// residual_out null), with codes in format fmt (1 int8, 2 E4M3).  x, residual
// and residual_out are row-strided views (strides in elements); codes and
// scales are contiguous.
int quant_fwd_strided(void* out_q, float* out_scale, uint16_t* residual_out, int64_t ro_stride,
                      const uint16_t* x, int64_t x_stride, const uint16_t* residual,
                      int64_t r_stride, const uint16_t* weight, int64_t n_rows, int64_t hidden,
                      float eps, const add_rmsnorm_launch_cfg* cfg, struct ihipStream_t* stream,
                      int fmt) {
  add_rmsnorm_launch_cfg c;
  int rc = check_scalars(n_rows, hidden, eps, cfg, &c);
  if (rc != ADD_RMSNORM_OK) return rc;
  if (n_rows == 0) return ADD_RMSNORM_OK;

  const bool fused = residual != nullptr || residual_out != nullptr;
  if (!out_q || !out_scale || !x || !weight || (fused && (!residual || !residual_out)))
    return ADD_RMSNORM_EINVAL;
  if (x_stride < hidden || (fused && (ro_stride < hidden || r_stride < hidden)))
    return ADD_RMSNORM_EINVAL;
  if (!aligned16(out_q) || !aligned(out_scale, 4) || !aligned16(x) || !aligned16(weight) ||
      x_stride % 8 != 0 ||
      (fused && (!aligned16(residual_out) || !aligned16(residual) || ro_stride % 8 != 0 ||
                 r_stride % 8 != 0)))
    return ADD_RMSNORM_EALIGN;
  const uint64_t row_bytes = (uint64_t)hidden * 2;
  if ((uint64_t)n_rows > (uint64_t)INT64_MAX / row_bytes) return ADD_RMSNORM_ERANGE;
  // Every view's span, (n_rows - 1) * stride + hidden elements, in bytes.
  const int64_t strides[3] = {x_stride, fused ? r_stride : hidden, fused ? ro_stride : hidden};
  for (int64_t st : strides)
    if ((uint64_t)(n_rows - 1) > ((uint64_t)INT64_MAX / 2 - (uint64_t)hidden) / (uint64_t)st)
      return ADD_RMSNORM_ERANGE;
  const uint64_t q_bytes = (uint64_t)n_rows * (uint64_t)hidden;
  const uint64_t s_bytes = (uint64_t)n_rows * 4;
  const View vx = {x, (uint64_t)x_stride * 2}, vr = {residual, (uint64_t)r_stride * 2};
  const View vro = {residual_out, (uint64_t)ro_stride * 2};
  // Codes and scales overlap nothing: each other, the weight, any view.
  if (overlap(out_q, q_bytes, out_scale, s_bytes)) return ADD_RMSNORM_EALIAS;
  if (overlap(out_q, q_bytes, weight, row_bytes) || overlap(out_scale, s_bytes, weight, row_bytes))
    return ADD_RMSNORM_EALIAS;
  const View* views[3] = {&vx, &vr, &vro};
  for (int i = 0; i < (fused ? 3 : 1); ++i)
    if (view_meets_range(*views[i], n_rows, row_bytes, out_q, q_bytes) ||
        view_meets_range(*views[i], n_rows, row_bytes, out_scale, s_bytes))
      return ADD_RMSNORM_EALIAS;
  // residual_out as in the bf16 variant: disjoint from the weight, and either
  // exactly an input's view (in place) or disjoint from it.
  if (fused && (view_meets_range(vro, n_rows, row_bytes, weight, row_bytes) ||
                output_meets_input(vro, vx, n_rows, row_bytes) ||
                output_meets_input(vro, vr, n_rows, row_bytes)))
    return ADD_RMSNORM_EALIAS;

  const addrms::FwdArgs a = {nullptr,  out_q,    out_scale, residual_out,
                             x,        residual, weight,    n_rows,
                             (int32_t)hidden, eps, x_stride, fused ? r_stride : 0,
                             hidden,   fused ? ro_stride : 0, fmt};
  return dispatch(a, c, stream);
}

int quant_fwd(void* out_q, float* out_scale, uint16_t* residual_out, const uint16_t* x,
              const uint16_t* residual, const uint16_t* weight, int64_t n_rows, int64_t hidden,
              float eps, const add_rmsnorm_launch_cfg* cfg, struct ihipStream_t* stream,
              int fmt) {
  return quant_fwd_strided(out_q, out_scale, residual_out, hidden, x, hidden, residual, hidden,
                           weight, n_rows, hidden, eps, cfg, stream, fmt);
}

constexpr int kFmtInt8 = 1;
constexpr int kFmtFp8 = 2;

}  // namespace

extern "C" {

int add_rmsnorm_quant_fwd_cfg(int8_t* out_q, float* out_scale, uint16_t* residual_out,
                              const uint16_t* x, const uint16_t* residual,
                              const uint16_t* weight, int64_t n_rows, int64_t hidden, float eps,
                              const struct add_rmsnorm_launch_cfg* cfg,
                              struct ihipStream_t* stream) {
  if (!residual || !residual_out) {
    add_rmsnorm_launch_cfg c;
    const int rc = check_scalars(n_rows, hidden, eps, cfg, &c);
    return rc != ADD_RMSNORM_OK ? rc : n_rows == 0 ? ADD_RMSNORM_OK : ADD_RMSNORM_EINVAL;
  }
  return quant_fwd(out_q, out_scale, residual_out, x, residual, weight, n_rows, hidden, eps, cfg,
                   stream, kFmtInt8);
}

int add_rmsnorm_quant_fwd(int8_t* out_q, float* out_scale, uint16_t* residual_out,
                          const uint16_t* x, const uint16_t* residual, const uint16_t* weight,
                          int64_t n_rows, int64_t hidden, float eps,
                          struct ihipStream_t* stream) {
  return add_rmsnorm_quant_fwd_cfg(out_q, out_scale, residual_out, x, residual, weight, n_rows,
                                   hidden, eps, nullptr, stream);
}

int add_rmsnorm_quant_fp8_fwd_cfg(uint8_t* out_q, float* out_scale, uint16_t* residual_out,
                                  const uint16_t* x, const uint16_t* residual,
                                  const uint16_t* weight, int64_t n_rows, int64_t hidden,
                                  float eps, const struct add_rmsnorm_launch_cfg* cfg,
                                  struct ihipStream_t* stream) {
  if (!residual || !residual_out) {
    add_rmsnorm_launch_cfg c;
    const int rc = check_scalars(n_rows, hidden, eps, cfg, &c);
    return rc != ADD_RMSNORM_OK ? rc : n_rows == 0 ? ADD_RMSNORM_OK : ADD_RMSNORM_EINVAL;
  }
  return quant_fwd(out_q, out_scale, residual_out, x, residual, weight, n_rows, hidden, eps, cfg,
                   stream, kFmtFp8);
}

int add_rmsnorm_quant_fp8_fwd(uint8_t* out_q, float* out_scale, uint16_t* residual_out,
                              const uint16_t* x, const uint16_t* residual,
                              const uint16_t* weight, int64_t n_rows, int64_t hidden, float eps,
                              struct ihipStream_t* stream) {
  return add_rmsnorm_quant_fp8_fwd_cfg(out_q, out_scale, residual_out, x, residual, weight,
                                       n_rows, hidden, eps, nullptr, stream);
}

int rmsnorm_fwd_strided(uint16_t* out, int64_t out_stride, const uint16_t* x, int64_t x_stride,
                        const uint16_t* weight, int64_t n_rows, int64_t hidden, float eps,
                        const struct add_rmsnorm_launch_cfg* cfg, struct ihipStream_t* stream) {
  return fwd_strided(out, out_stride, nullptr, 0, x, x_stride, nullptr, 0, weight, n_rows, hidden,
                     eps, cfg, stream, false);
}

int rmsnorm_fwd_cfg(uint16_t* out, const uint16_t* x, const uint16_t* weight, int64_t n_rows,
                    int64_t hidden, float eps, const struct add_rmsnorm_launch_cfg* cfg,
                    struct ihipStream_t* stream) {
  return fwd_strided(out, hidden, nullptr, 0, x, hidden, nullptr, 0, weight, n_rows, hidden, eps,
                     cfg, stream, false);
}

int rmsnorm_fwd(uint16_t* out, const uint16_t* x, const uint16_t* weight, int64_t n_rows,
                int64_t hidden, float eps, struct ihipStream_t* stream) {
  return rmsnorm_fwd_cfg(out, x, weight, n_rows, hidden, eps, nullptr, stream);
}

int rmsnorm_quant_fwd_cfg(int8_t* out_q, float* out_scale, const uint16_t* x,
                          const uint16_t* weight, int64_t n_rows, int64_t hidden, float eps,
                          const struct add_rmsnorm_launch_cfg* cfg, struct ihipStream_t* stream) {
  return quant_fwd(out_q, out_scale, nullptr, x, nullptr, weight, n_rows, hidden, eps, cfg,
                   stream, kFmtInt8);
}

int rmsnorm_quant_fwd(int8_t* out_q, float* out_scale, const uint16_t* x, const uint16_t* weight,
                      int64_t n_rows, int64_t hidden, float eps, struct ihipStream_t* stream) {
  return rmsnorm_quant_fwd_cfg(out_q, out_scale, x, weight, n_rows, hidden, eps, nullptr,
                               stream);
}

int rmsnorm_quant_fp8_fwd_cfg(uint8_t* out_q, float* out_scale, const uint16_t* x,
                              const uint16_t* weight, int64_t n_rows, int64_t hidden, float eps,
                              const struct add_rmsnorm_launch_cfg* cfg,
                              struct ihipStream_t* stream) {
  return quant_fwd(out_q, out_scale, nullptr, x, nullptr, weight, n_rows, hidden, eps, cfg,
                   stream, kFmtFp8);
}

int rmsnorm_quant_fp8_fwd(uint8_t* out_q, float* out_scale, const uint16_t* x,
                          const uint16_t* weight, int64_t n_rows, int64_t hidden, float eps,
                          struct ihipStream_t* stream) {
  return rmsnorm_quant_fp8_fwd_cfg(out_q, out_scale, x, weight, n_rows, hidden, eps, nullptr,
                                   stream);
}

int log1p_f32_cfg(float* out, const float* x, int64_t n, const struct log1p_launch_cfg* cfg,
                  struct ihipStream_t* stream) {
  log1p_launch_cfg c = {0, 0, 0, 0};
  if (cfg) c = *cfg;
  if (n < 0) return ADD_RMSNORM_EINVAL;
  if (c.block_threads != 0 && !valid_block(c.block_threads)) return ADD_RMSNORM_EINVAL;
  const int e = c.elems_per_thread;
  if (e != 0 && e != 1 && e != 2 && e != 4 && e != 8) return ADD_RMSNORM_EINVAL;
  if (c.grid_blocks < -1 || (c.flags & ~LOG1P_FLAG_ACCURATE_ONLY) != 0) return ADD_RMSNORM_EINVAL;
  if (n == 0) return ADD_RMSNORM_OK;
  if (!out || !x) return ADD_RMSNORM_EINVAL;
  if (!aligned16(out) || !aligned16(x)) return ADD_RMSNORM_EALIGN;
  if ((uint64_t)n > (uint64_t)INT64_MAX / 4) return ADD_RMSNORM_ERANGE;
  const uint64_t bytes = (uint64_t)n * 4;
  if (out != x && overlap(out, bytes, x, bytes)) return ADD_RMSNORM_EALIAS;
  const int b = c.block_threads ? c.block_threads : kLog1pThreads;
  hipError_t err = addrms::launch_log1p(out, x, n, b, e ? e : kLog1pElems, c.grid_blocks,
                                        (c.flags & LOG1P_FLAG_ACCURATE_ONLY) != 0,
                                        reinterpret_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_failure(err);
  return ADD_RMSNORM_OK;
}

int log1p_f32(float* out, const float* x, int64_t n, struct ihipStream_t* stream) {
  return log1p_f32_cfg(out, x, n, nullptr, stream);
}

int add_rmsnorm_test_cvt_range(uint16_t* out, uint32_t start, int64_t count,
                               struct ihipStream_t* stream) {
  if (count < 0) return ADD_RMSNORM_EINVAL;
  if (count % 8 != 0) return ADD_RMSNORM_EALIGN;
  if (count == 0) return ADD_RMSNORM_OK;
  if (!out) return ADD_RMSNORM_EINVAL;
  if (!aligned16(out)) return ADD_RMSNORM_EALIGN;
  hipError_t e = addrms::launch_cvt_range(out, start, count, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_failure(e);
  return ADD_RMSNORM_OK;
}

int add_rmsnorm_test_cvt_e4m3_range(uint8_t* out, uint32_t start, int64_t count,
                                    struct ihipStream_t* stream) {
  if (count < 0) return ADD_RMSNORM_EINVAL;
  if (count % 8 != 0) return ADD_RMSNORM_EALIGN;
  if (count == 0) return ADD_RMSNORM_OK;
  if (!out) return ADD_RMSNORM_EINVAL;
  if (!aligned16(out)) return ADD_RMSNORM_EALIGN;
  hipError_t e =
      addrms::launch_cvt_e4m3_range(out, start, count, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_failure(e);
  return ADD_RMSNORM_OK;
}

int add_rmsnorm_test_copy2(uint16_t* dst0, uint16_t* dst1, const uint16_t* src0,
                           const uint16_t* src1, int64_t count, struct ihipStream_t* stream) {
  if (count < 0) return ADD_RMSNORM_EINVAL;
  if (count % 8 != 0) return ADD_RMSNORM_EALIGN;
  if (count == 0) return ADD_RMSNORM_OK;
  if (!dst0 || !dst1 || !src0 || !src1) return ADD_RMSNORM_EINVAL;
  if (!aligned16(dst0) || !aligned16(dst1) || !aligned16(src0) || !aligned16(src1))
    return ADD_RMSNORM_EALIGN;
  const uint64_t n = (uint64_t)count * 2;
  if (overlap(dst0, n, dst1, n) || overlap(dst0, n, src0, n) || overlap(dst0, n, src1, n) ||
      overlap(dst1, n, src0, n) || overlap(dst1, n, src1, n))
    return ADD_RMSNORM_EALIAS;
  hipError_t e = addrms::launch_copy2(dst0, dst1, src0, src1, count,
                                      reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_failure(e);
  return ADD_RMSNORM_OK;
}

int add_rmsnorm_test_copy_rows(uint16_t* dst0, uint16_t* dst1, const uint16_t* src0,
                               const uint16_t* src1, int64_t n_rows, int64_t hidden,
                               int rows_per_burst, struct ihipStream_t* stream) {
  if (n_rows < 0 || hidden <= 0 || !(rows_per_burst == 1 || rows_per_burst == 2 ||
                                     rows_per_burst == 4))
    return ADD_RMSNORM_EINVAL;
  if (hidden % 8 != 0) return ADD_RMSNORM_EALIGN;
  if (hidden > 16384 || n_rows > ((int64_t)1 << 30)) return ADD_RMSNORM_ERANGE;
  if (n_rows == 0) return ADD_RMSNORM_OK;
  if (!dst0 || !dst1 || !src0 || !src1) return ADD_RMSNORM_EINVAL;
  if (!aligned16(dst0) || !aligned16(dst1) || !aligned16(src0) || !aligned16(src1))
    return ADD_RMSNORM_EALIGN;
  const uint64_t n = (uint64_t)n_rows * (uint64_t)hidden * 2;
  if (overlap(dst0, n, dst1, n) || overlap(dst0, n, src0, n) || overlap(dst0, n, src1, n) ||
      overlap(dst1, n, src0, n) || overlap(dst1, n, src1, n))
    return ADD_RMSNORM_EALIAS;
  hipError_t e = addrms::launch_copy_rows(dst0, dst1, src0, src1, n_rows, (int)hidden,
                                          rows_per_burst, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_failure(e);
  return ADD_RMSNORM_OK;
}

int add_rmsnorm_test_stream(uint16_t* dst, const uint16_t* src, int64_t count, int mode,
                            struct ihipStream_t* stream) {
  if (count < 0 || (mode != 0 && mode != 1)) return ADD_RMSNORM_EINVAL;
  if (count % 8 != 0) return ADD_RMSNORM_EALIGN;
  if (count == 0) return ADD_RMSNORM_OK;
  if (!dst || (mode == 0 && !src)) return ADD_RMSNORM_EINVAL;
  if (!aligned16(dst) || (mode == 0 && !aligned16(src))) return ADD_RMSNORM_EALIGN;
  const uint64_t n = (uint64_t)count * 2;
  if (mode == 0 && overlap(dst, n, src, n)) return ADD_RMSNORM_EALIAS;
  hipError_t e = addrms::launch_stream(dst, src, count, mode, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_failure(e);
  return ADD_RMSNORM_OK;
}

const char* add_rmsnorm_strerror(int status) {
  switch (status) {
    case ADD_RMSNORM_OK: return "success";
    case ADD_RMSNORM_EINVAL:
      return "invalid argument (null pointer, negative rows, hidden <= 0, bad eps or launch "
             "configuration)";
    case ADD_RMSNORM_EALIGN:
      return "a pointer is misaligned (2 bytes for bf16 data; 16 bytes with hidden % 8 == 0 "
             "for the quantised entry points and a forced fast path)";
    case ADD_RMSNORM_EALIAS:
      return "an output partly overlaps an input, or overlaps the weight or another output";
    case ADD_RMSNORM_ERANGE: return "hidden (or the problem size) is above what the path supports";
    case ADD_RMSNORM_EHIP: return "the HIP launch failed (see add_rmsnorm_last_hip_error)";
  }
  return "unknown status";
}

const char* add_rmsnorm_last_hip_error(void) { return g_hip_error; }

int add_rmsnorm_quant_fwd_strided(int8_t* out_q, float* out_scale, uint16_t* residual_out,
                                  int64_t residual_out_stride, const uint16_t* x,
                                  int64_t x_stride, const uint16_t* residual,
                                  int64_t residual_stride, const uint16_t* weight, int64_t n_rows,
                                  int64_t hidden, float eps,
                                  const struct add_rmsnorm_launch_cfg* cfg,
                                  struct ihipStream_t* stream) {
  if (!residual || !residual_out) {
    add_rmsnorm_launch_cfg c;
    const int rc = check_scalars(n_rows, hidden, eps, cfg, &c);
    return rc != ADD_RMSNORM_OK ? rc : n_rows == 0 ? ADD_RMSNORM_OK : ADD_RMSNORM_EINVAL;
  }
  return quant_fwd_strided(out_q, out_scale, residual_out, residual_out_stride, x, x_stride,
                           residual, residual_stride, weight, n_rows, hidden, eps, cfg, stream,
                           kFmtInt8);
}

int add_rmsnorm_quant_fp8_fwd_strided(uint8_t* out_q, float* out_scale, uint16_t* residual_out,
                                      int64_t residual_out_stride, const uint16_t* x,
                                      int64_t x_stride, const uint16_t* residual,
                                      int64_t residual_stride, const uint16_t* weight,
                                      int64_t n_rows, int64_t hidden, float eps,
                                      const struct add_rmsnorm_launch_cfg* cfg,
                                      struct ihipStream_t* stream) {
  if (!residual || !residual_out) {
    add_rmsnorm_launch_cfg c;
    const int rc = check_scalars(n_rows, hidden, eps, cfg, &c);
    return rc != ADD_RMSNORM_OK ? rc : n_rows == 0 ? ADD_RMSNORM_OK : ADD_RMSNORM_EINVAL;
  }
  return quant_fwd_strided(out_q, out_scale, residual_out, residual_out_stride, x, x_stride,
                           residual, residual_stride, weight, n_rows, hidden, eps, cfg, stream,
                           kFmtFp8);
}

int rmsnorm_quant_fwd_strided(int8_t* out_q, float* out_scale, const uint16_t* x,
                              int64_t x_stride, const uint16_t* weight, int64_t n_rows,
                              int64_t hidden, float eps, const struct add_rmsnorm_launch_cfg* cfg,
                              struct ihipStream_t* stream) {
  return quant_fwd_strided(out_q, out_scale, nullptr, 0, x, x_stride, nullptr, 0, weight, n_rows,
                           hidden, eps, cfg, stream, kFmtInt8);
}

int rmsnorm_quant_fp8_fwd_strided(uint8_t* out_q, float* out_scale, const uint16_t* x,
                                  int64_t x_stride, const uint16_t* weight, int64_t n_rows,
                                  int64_t hidden, float eps,
                                  const struct add_rmsnorm_launch_cfg* cfg,
                                  struct ihipStream_t* stream) {
  return quant_fwd_strided(out_q, out_scale, nullptr, 0, x, x_stride, nullptr, 0, weight, n_rows,
                           hidden, eps, cfg, stream, kFmtFp8);
}

int qk_rmsnorm_fwd_cfg(uint16_t* q_out, uint16_t* k_out, const uint16_t* q, const uint16_t* k,
                       const uint16_t* q_weight, const uint16_t* k_weight, int64_t n_tokens,
                       int64_t n_q_heads, int64_t n_k_heads, int64_t head_dim,
                       int64_t q_stride, int64_t k_stride, int64_t q_out_stride,
                       int64_t k_out_stride, float eps, const struct add_rmsnorm_launch_cfg* cfg,
                       struct ihipStream_t* stream) {
  if (n_tokens < 0 || n_q_heads < 0 || n_k_heads < 0 || head_dim <= 0 || !std::isfinite(eps) ||
      eps < 0.0f)
    return ADD_RMSNORM_EINVAL;
  add_rmsnorm_launch_cfg c = {ADD_RMSNORM_PATH_AUTO, 0, 0, 0};
  if (cfg) c = *cfg;
  if (c.path != ADD_RMSNORM_PATH_AUTO && c.path != ADD_RMSNORM_PATH_PACKED)
    return ADD_RMSNORM_EINVAL;
  if (c.grid_blocks < -1 || (c.flags != 0 && !valid_rows_per_lane(c.flags)) ||
      (c.block_threads != 0 && !valid_block(c.block_threads)))
    return ADD_RMSNORM_EINVAL;
  if (head_dim > ADD_RMSNORM_MAX_HIDDEN) return ADD_RMSNORM_ERANGE;
  if (head_dim % 8 != 0) return ADD_RMSNORM_EALIGN;
  if (n_tokens == 0) return ADD_RMSNORM_OK;

  struct Side {
    uint16_t* out;
    const uint16_t* in;
    const uint16_t* weight;
    int64_t heads, stride, out_stride;
  };
  const Side sides[2] = {{q_out, q, q_weight, n_q_heads, q_stride, q_out_stride},
                         {k_out, k, k_weight, n_k_heads, k_stride, k_out_stride}};
  int64_t rows = 0;
  bool too_many = false;
  for (const Side& d : sides) {
    if (d.heads == 0) continue;
    if (!d.out || !d.in || !d.weight) return ADD_RMSNORM_EINVAL;
    if (d.heads > addrms::kPackMaxRows) return ADD_RMSNORM_ERANGE;
    const int64_t width = d.heads * head_dim;
    if (d.stride < width || d.out_stride < width) return ADD_RMSNORM_EINVAL;
    if (!aligned16(d.out) || !aligned16(d.in) || !aligned16(d.weight) || d.stride % 8 != 0 ||
        d.out_stride % 8 != 0)
      return ADD_RMSNORM_EALIGN;
    if (n_tokens > 0 && d.heads > (addrms::kPackMaxRows - 1) / n_tokens) {
      too_many = true;
    } else {
      rows += n_tokens * d.heads;
    }
    for (int64_t st : {d.stride, d.out_stride})
      if (n_tokens > 0 &&
          (uint64_t)(n_tokens - 1) > ((uint64_t)INT64_MAX / 2 - (uint64_t)width) / (uint64_t)st)
        return ADD_RMSNORM_ERANGE;
  }
  if (n_q_heads == 0 && n_k_heads == 0) return ADD_RMSNORM_OK;

  // Outputs: each one either exactly its input's view (in place) or disjoint
  // from it; disjoint from the other tensor, the other output and the weights.
  const uint64_t hd_bytes = (uint64_t)head_dim * 2;
  for (int i = 0; i < 2; ++i) {
    const Side& d = sides[i];
    if (d.heads == 0) continue;
    const uint64_t width = (uint64_t)d.heads * hd_bytes;
    const View vo = {d.out, (uint64_t)d.out_stride * 2}, vi = {d.in, (uint64_t)d.stride * 2};
    if (output_meets_input(vo, vi, n_tokens, width)) return ADD_RMSNORM_EALIAS;
    for (const Side& e : sides) {
      if (e.heads == 0) continue;
      if (view_meets_range(vo, n_tokens, width, e.weight, hd_bytes)) return ADD_RMSNORM_EALIAS;
    }
    const Side& o = sides[1 - i];
    if (o.heads == 0) continue;
    const uint64_t owidth = (uint64_t)o.heads * hd_bytes;
    const View oo = {o.out, (uint64_t)o.out_stride * 2}, oi = {o.in, (uint64_t)o.stride * 2};
    if (views_overlap2(vo, width, oi, owidth, n_tokens)) return ADD_RMSNORM_EALIAS;
    if (i == 0 && views_overlap2(vo, width, oo, owidth, n_tokens)) return ADD_RMSNORM_EALIAS;
  }

  // Range limits last, so that a caller's views are checked whatever their size.
  if (head_dim > addrms::kPackMaxHidden || too_many || rows >= addrms::kPackMaxRows)
    return ADD_RMSNORM_ERANGE;

  addrms::PackTensors g[2] = {};
  for (int i = 0; i < 2; ++i) {
    const Side& d = sides[i];
    if (d.heads == 0) continue;
    g[i] = addrms::PackTensors{d.out, nullptr, nullptr, nullptr, d.in, nullptr, d.weight,
                               d.stride, 0, d.out_stride, 0, n_tokens, d.heads};
  }
  const hipError_t e = addrms::launch_pack_rows(
      g[0], g[1], (int32_t)head_dim, eps, 0, c.block_threads ? c.block_threads : kPackThreads,
      c.flags ? c.flags : kPackRowsPerLane, c.grid_blocks ? c.grid_blocks : -1,
      reinterpret_cast<hipStream_t>(stream));
  return e != hipSuccess ? hip_failure(e) : ADD_RMSNORM_OK;
}

int qk_rmsnorm_fwd(uint16_t* q_out, uint16_t* k_out, const uint16_t* q, const uint16_t* k,
                   const uint16_t* q_weight, const uint16_t* k_weight, int64_t n_tokens,
                   int64_t n_q_heads, int64_t n_k_heads, int64_t head_dim, int64_t q_stride,
                   int64_t k_stride, int64_t q_out_stride, int64_t k_out_stride, float eps,
                   struct ihipStream_t* stream) {
  return qk_rmsnorm_fwd_cfg(q_out, k_out, q, k, q_weight, k_weight, n_tokens, n_q_heads,
                            n_k_heads, head_dim, q_stride, k_stride, q_out_stride, k_out_stride,
                            eps, nullptr, stream);
}

int add_rmsnorm_abi_version(void) { return ADD_RMSNORM_ABI_VERSION; }

const char* add_rmsnorm_build_info(void) { return ADD_RMSNORM_BUILD_INFO; }

}  // extern "C"
