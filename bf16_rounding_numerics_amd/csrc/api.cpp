// C entry points of the fused residual-add + RMSNorm forward, of plain
// RMSNorm (bf16 or int8 out) and of the correctly rounded binary32 log1p:
// argument validation (on the host, before anything is enqueued), kernel
// choice, launch on the caller's stream.  The contracts are documented in
// include/add_rmsnorm.h and include/log1p_f32.h.
#include "add_rmsnorm.h"
#include "log1p_f32.h"

#include <hip/hip_runtime.h>

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

// Smallest of 1, 2, 4, 8 that is >= need (0 if none).
int pow2_at_least(int64_t need) {
  for (int j = 1; j <= 8; j *= 2)
    if (j >= need) return j;
  return 0;
}

// Default workgroup sizes per path.
constexpr int kWaveRowThreads = 256;
constexpr int kWgRowThreads = 512;
constexpr int kTwoPassThreads = 512;

// Default launch of log1p_f32: 256 threads, 4 consecutive elements each.
constexpr int kLog1pThreads = 256;
constexpr int kLog1pElems = 4;

// Upper hidden sizes of the automatic choice.
constexpr int64_t kWaveRowMaxHidden = 2048;
constexpr int64_t kWgRowMaxHidden = 8192;

int device_max_lds(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_failure(e);
  e = hipDeviceGetAttribute(out, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return hip_failure(e);
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
  if (c->flags != 0 || c->grid_blocks < -1) return ADD_RMSNORM_EINVAL;
  if (c->path < ADD_RMSNORM_PATH_AUTO || c->path > ADD_RMSNORM_PATH_LDS_TWO_PASS)
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

// Kernel choice by hidden (or as forced) and launch.
int dispatch(const addrms::FwdArgs& a, const add_rmsnorm_launch_cfg& c,
             struct ihipStream_t* stream) {
  int path = c.path;
  const int64_t hidden = a.hidden;
  if (path == ADD_RMSNORM_PATH_AUTO) {
    path = hidden <= kWaveRowMaxHidden ? ADD_RMSNORM_PATH_WAVE_ROW
           : hidden <= kWgRowMaxHidden ? ADD_RMSNORM_PATH_WG_ROW
                                       : ADD_RMSNORM_PATH_LDS_TWO_PASS;
  }
  const int64_t segs = hidden / 8;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (path == ADD_RMSNORM_PATH_WAVE_ROW) {
    const int b = c.block_threads ? c.block_threads : kWaveRowThreads;
    const int j = pow2_at_least((segs + 63) / 64);
    if (j == 0 || !addrms::wave_row_supported(b, j)) return ADD_RMSNORM_ERANGE;
    e = addrms::launch_wave_row(a, b, j, c.grid_blocks, s);
  } else if (path == ADD_RMSNORM_PATH_WG_ROW) {
    const int b = c.block_threads ? c.block_threads : kWgRowThreads;
    const int j = pow2_at_least((segs + b - 1) / b);
    if (j == 0 || !addrms::wg_row_supported(b, j)) return ADD_RMSNORM_ERANGE;
    e = addrms::launch_wg_row(a, b, j, c.grid_blocks, s);
  } else {
    const int b = c.block_threads ? c.block_threads : kTwoPassThreads;
    int max_lds = 0;
    const int rc = device_max_lds(&max_lds);
    if (rc != ADD_RMSNORM_OK) return rc;
    if (addrms::lds_two_pass_lds_bytes((int)hidden) > (size_t)max_lds) return ADD_RMSNORM_ERANGE;
    e = addrms::launch_lds_two_pass(a, b, c.grid_blocks, s);
  }
  if (e != hipSuccess) return hip_failure(e);
  return ADD_RMSNORM_OK;
}

}  // namespace

extern "C" {

int add_rmsnorm_fwd_cfg(uint16_t* out, uint16_t* residual_out, const uint16_t* x,
                        const uint16_t* residual, const uint16_t* weight, int64_t n_rows,
                        int64_t hidden, float eps, const struct add_rmsnorm_launch_cfg* cfg,
                        struct ihipStream_t* stream) {
  add_rmsnorm_launch_cfg c;
  int rc = check_scalars(n_rows, hidden, eps, cfg, &c);
  if (rc != ADD_RMSNORM_OK) return rc;
  if (n_rows == 0) return ADD_RMSNORM_OK;

  if (!out || !residual_out || !x || !residual || !weight) return ADD_RMSNORM_EINVAL;
  if (!aligned16(out) || !aligned16(residual_out) || !aligned16(x) || !aligned16(residual) ||
      !aligned16(weight))
    return ADD_RMSNORM_EALIGN;
  const uint64_t row_bytes = (uint64_t)hidden * 2;
  if ((uint64_t)n_rows > (uint64_t)INT64_MAX / row_bytes) return ADD_RMSNORM_ERANGE;
  const uint64_t t_bytes = (uint64_t)n_rows * row_bytes;
  // The outputs are disjoint from each other and from the weight; each is
  // either disjoint from an input or exactly that input (in place).
  if (overlap(out, t_bytes, residual_out, t_bytes)) return ADD_RMSNORM_EALIAS;
  if (output_aliases_badly(out, t_bytes, x, residual, weight, row_bytes) ||
      output_aliases_badly(residual_out, t_bytes, x, residual, weight, row_bytes))
    return ADD_RMSNORM_EALIAS;

  const addrms::FwdArgs a = {out, nullptr, nullptr, residual_out, x, residual, weight,
                             n_rows, (int32_t)hidden, eps};
  return dispatch(a, c, stream);
}

int add_rmsnorm_fwd(uint16_t* out, uint16_t* residual_out, const uint16_t* x,
                    const uint16_t* residual, const uint16_t* weight, int64_t n_rows,
                    int64_t hidden, float eps, struct ihipStream_t* stream) {
  return add_rmsnorm_fwd_cfg(out, residual_out, x, residual, weight, n_rows, hidden, eps,
                             nullptr, stream);
}

int add_rmsnorm_quant_fwd_cfg(int8_t* out_q, float* out_scale, uint16_t* residual_out,
                              const uint16_t* x, const uint16_t* residual,
                              const uint16_t* weight, int64_t n_rows, int64_t hidden, float eps,
                              const struct add_rmsnorm_launch_cfg* cfg,
                              struct ihipStream_t* stream) {
  add_rmsnorm_launch_cfg c;
  int rc = check_scalars(n_rows, hidden, eps, cfg, &c);
  if (rc != ADD_RMSNORM_OK) return rc;
  if (n_rows == 0) return ADD_RMSNORM_OK;

  if (!out_q || !out_scale || !residual_out || !x || !residual || !weight)
    return ADD_RMSNORM_EINVAL;
  if (!aligned16(out_q) || !aligned(out_scale, 4) || !aligned16(residual_out) || !aligned16(x) ||
      !aligned16(residual) || !aligned16(weight))
    return ADD_RMSNORM_EALIGN;
  const uint64_t row_bytes = (uint64_t)hidden * 2;
  if ((uint64_t)n_rows > (uint64_t)INT64_MAX / row_bytes) return ADD_RMSNORM_ERANGE;
  const uint64_t t_bytes = (uint64_t)n_rows * row_bytes;
  const uint64_t q_bytes = (uint64_t)n_rows * (uint64_t)hidden;
  const uint64_t s_bytes = (uint64_t)n_rows * 4;
  // Codes and scales overlap nothing; residual_out as in the bf16 variant.
  const void* ins[3] = {x, residual, weight};
  const uint64_t in_bytes[3] = {t_bytes, t_bytes, row_bytes};
  if (overlap(out_q, q_bytes, out_scale, s_bytes) ||
      overlap(out_q, q_bytes, residual_out, t_bytes) ||
      overlap(out_scale, s_bytes, residual_out, t_bytes))
    return ADD_RMSNORM_EALIAS;
  for (int i = 0; i < 3; ++i)
    if (overlap(out_q, q_bytes, ins[i], in_bytes[i]) ||
        overlap(out_scale, s_bytes, ins[i], in_bytes[i]))
      return ADD_RMSNORM_EALIAS;
  if (output_aliases_badly(residual_out, t_bytes, x, residual, weight, row_bytes))
    return ADD_RMSNORM_EALIAS;

  const addrms::FwdArgs a = {nullptr, out_q, out_scale, residual_out, x, residual, weight,
                             n_rows, (int32_t)hidden, eps};
  return dispatch(a, c, stream);
}

int add_rmsnorm_quant_fwd(int8_t* out_q, float* out_scale, uint16_t* residual_out,
                          const uint16_t* x, const uint16_t* residual, const uint16_t* weight,
                          int64_t n_rows, int64_t hidden, float eps,
                          struct ihipStream_t* stream) {
  return add_rmsnorm_quant_fwd_cfg(out_q, out_scale, residual_out, x, residual, weight, n_rows,
                                   hidden, eps, nullptr, stream);
}

int rmsnorm_fwd_cfg(uint16_t* out, const uint16_t* x, const uint16_t* weight, int64_t n_rows,
                    int64_t hidden, float eps, const struct add_rmsnorm_launch_cfg* cfg,
                    struct ihipStream_t* stream) {
  add_rmsnorm_launch_cfg c;
  int rc = check_scalars(n_rows, hidden, eps, cfg, &c);
  if (rc != ADD_RMSNORM_OK) return rc;
  if (n_rows == 0) return ADD_RMSNORM_OK;

  if (!out || !x || !weight) return ADD_RMSNORM_EINVAL;
  if (!aligned16(out) || !aligned16(x) || !aligned16(weight)) return ADD_RMSNORM_EALIGN;
  const uint64_t row_bytes = (uint64_t)hidden * 2;
  if ((uint64_t)n_rows > (uint64_t)INT64_MAX / row_bytes) return ADD_RMSNORM_ERANGE;
  const uint64_t t_bytes = (uint64_t)n_rows * row_bytes;
  // out is disjoint from the weight, and disjoint from x or exactly x.
  if (output_aliases_badly(out, t_bytes, x, x, weight, row_bytes)) return ADD_RMSNORM_EALIAS;

  const addrms::FwdArgs a = {out, nullptr, nullptr, nullptr, x, nullptr, weight,
                             n_rows, (int32_t)hidden, eps};
  return dispatch(a, c, stream);
}

int rmsnorm_fwd(uint16_t* out, const uint16_t* x, const uint16_t* weight, int64_t n_rows,
                int64_t hidden, float eps, struct ihipStream_t* stream) {
  return rmsnorm_fwd_cfg(out, x, weight, n_rows, hidden, eps, nullptr, stream);
}

int rmsnorm_quant_fwd_cfg(int8_t* out_q, float* out_scale, const uint16_t* x,
                          const uint16_t* weight, int64_t n_rows, int64_t hidden, float eps,
                          const struct add_rmsnorm_launch_cfg* cfg, struct ihipStream_t* stream) {
  add_rmsnorm_launch_cfg c;
  int rc = check_scalars(n_rows, hidden, eps, cfg, &c);
  if (rc != ADD_RMSNORM_OK) return rc;
  if (n_rows == 0) return ADD_RMSNORM_OK;

  if (!out_q || !out_scale || !x || !weight) return ADD_RMSNORM_EINVAL;
  if (!aligned16(out_q) || !aligned(out_scale, 4) || !aligned16(x) || !aligned16(weight))
    return ADD_RMSNORM_EALIGN;
  const uint64_t row_bytes = (uint64_t)hidden * 2;
  if ((uint64_t)n_rows > (uint64_t)INT64_MAX / row_bytes) return ADD_RMSNORM_ERANGE;
  const uint64_t t_bytes = (uint64_t)n_rows * row_bytes;
  const uint64_t q_bytes = (uint64_t)n_rows * (uint64_t)hidden;
  const uint64_t s_bytes = (uint64_t)n_rows * 4;
  // Codes and scales overlap nothing.
  if (overlap(out_q, q_bytes, out_scale, s_bytes) || overlap(out_q, q_bytes, x, t_bytes) ||
      overlap(out_q, q_bytes, weight, row_bytes) || overlap(out_scale, s_bytes, x, t_bytes) ||
      overlap(out_scale, s_bytes, weight, row_bytes))
    return ADD_RMSNORM_EALIAS;

  const addrms::FwdArgs a = {nullptr, out_q, out_scale, nullptr, x, nullptr, weight,
                             n_rows, (int32_t)hidden, eps};
  return dispatch(a, c, stream);
}

int rmsnorm_quant_fwd(int8_t* out_q, float* out_scale, const uint16_t* x, const uint16_t* weight,
                      int64_t n_rows, int64_t hidden, float eps, struct ihipStream_t* stream) {
  return rmsnorm_quant_fwd_cfg(out_q, out_scale, x, weight, n_rows, hidden, eps, nullptr,
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

const char* add_rmsnorm_strerror(int status) {
  switch (status) {
    case ADD_RMSNORM_OK: return "success";
    case ADD_RMSNORM_EINVAL:
      return "invalid argument (null pointer, negative rows, hidden <= 0, bad eps or launch "
             "configuration)";
    case ADD_RMSNORM_EALIGN: return "a pointer is misaligned, or hidden % 8 != 0";
    case ADD_RMSNORM_EALIAS:
      return "an output partly overlaps an input, or overlaps the weight or another output";
    case ADD_RMSNORM_ERANGE: return "hidden (or the problem size) is above what the path supports";
    case ADD_RMSNORM_EHIP: return "the HIP launch failed (see add_rmsnorm_last_hip_error)";
  }
  return "unknown status";
}

const char* add_rmsnorm_last_hip_error(void) { return g_hip_error; }

int add_rmsnorm_abi_version(void) { return ADD_RMSNORM_ABI_VERSION; }

const char* add_rmsnorm_build_info(void) { return ADD_RMSNORM_BUILD_INFO; }

}  // extern "C"
