/*
 * log1p_f32.h -- launch-invariant binary32 log1p for MI355X (gfx950).
 *
 * The ROCm/TransformerEngine issue "CP LSE merge switches compiled variants on
 * ROCm, breaking forward reproducibility" ("Root cause", "Minimal reproducer")
 * finds an elementwise binary32 log1p whose results depend on the launch
 * shape (block size, elements per thread): two code paths about one ULP
 * apart.  These entry points compute out[i] = ln(1 + x[i]) rounded once to
 * the nearest binary32, ties to even, for every input.  A correctly rounded
 * result is unique, so it is the same bit pattern for every launch
 * configuration, every run and every build of this library.
 *
 * IEEE 754 special cases: log1p(+-0) = +-0, log1p(-1) = -Inf,
 * log1p(x < -1) = NaN (also for -Inf), log1p(+Inf) = +Inf, NaN -> NaN.
 *
 * Conventions as in add_rmsnorm.h: device pointers owned by the caller, work
 * enqueued on `stream` without synchronisation, argument errors returned on
 * the host as ADD_RMSNORM_* status codes before anything is enqueued
 * (add_rmsnorm_strerror gives their text).
 */
#ifndef LOG1P_F32_H
#define LOG1P_F32_H

#include <stdint.h>

#include "add_rmsnorm.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * out[i] = log1p(x[i]) for 0 <= i < n, correctly rounded binary32.
 *   out, x  device pointers to n floats, each 16-byte aligned; out may be x
 *           itself (in place); any other overlap is ADD_RMSNORM_EALIAS.
 *   n >= 0  (0 enqueues nothing and returns OK; pointers are not checked).
 * Errors: ADD_RMSNORM_EINVAL (n < 0, null pointer), ADD_RMSNORM_EALIGN,
 * ADD_RMSNORM_EALIAS, ADD_RMSNORM_EHIP.
 */
int log1p_f32(float* out, const float* x, int64_t n, struct ihipStream_t* stream);

/* Bits of log1p_launch_cfg.flags. */
#define LOG1P_FLAG_ACCURATE_ONLY 1 /* every element by the double-double path (testing) */

/*
 * Launch configuration, for tests and benchmarks that must show the result
 * does not depend on it.  0 in a field means the library's choice.
 *   block_threads     64, 128, 256, 512 or 1024.
 *   elems_per_thread  1, 2, 4 or 8 consecutive elements per thread.
 *   grid_blocks       0: one workgroup per tile of block_threads *
 *                     elems_per_thread elements, at most 8192 workgroups
 *                     (which then loop over tiles); > 0: that many
 *                     workgroups, looping over tiles; -1: as many as fit on
 *                     the device.
 *   flags             0 or LOG1P_FLAG_ACCURATE_ONLY.
 */
struct log1p_launch_cfg {
  int32_t block_threads;
  int32_t elems_per_thread;
  int32_t grid_blocks;
  int32_t flags;
};

/* log1p_f32 with an explicit launch configuration (cfg may be NULL); the
 * result is the same for every configuration.  A bad field is
 * ADD_RMSNORM_EINVAL. */
int log1p_f32_cfg(float* out, const float* x, int64_t n, const struct log1p_launch_cfg* cfg,
                  struct ihipStream_t* stream);

#ifdef __cplusplus
}
#endif

#endif /* LOG1P_F32_H */
