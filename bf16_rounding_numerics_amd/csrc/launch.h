// Internal interface between the C entry points (api.cpp) and the kernels
// (kernels.hip).  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace addrms {

struct FwdArgs {
  uint16_t* out;           // bf16 out, or null for the quantised variant
  void* qout;              // 1-byte codes (quantised variants), else null
  float* qscale;           // per-row scale (quantised variants), else null
  uint16_t* residual_out;  // null for plain RMSNorm
  const uint16_t* x;
  const uint16_t* residual;  // null for plain RMSNorm (acc = x, no residual_out)
  const uint16_t* weight;
  int64_t n_rows;
  int32_t hidden;
  float eps;
  // Row strides in elements (>= hidden).  The three fast kernels need hidden,
  // the strides and every pointer aligned to 8 elements (16 bytes); the
  // general kernel takes any hidden and any 2-byte aligned layout.
  int64_t x_stride, r_stride, out_stride, ro_stride;
  int32_t qfmt;  // code format when qout is set: 1 int8, 2 OCP FP8 E4M3
};

// Largest number of 8-element segments any row can have.
constexpr int kMaxSegments = 32768 / 8;

// One wavefront per row, block_threads / 64 rows per workgroup.  The row's
// segments are spread over the 64 lanes, segs_per_lane (1, 2, 4 or 8) each.
// grid_blocks > 0 launches that many workgroups, which loop over the rows;
// -1 launches as many as fit on the device at once; 0 one per row group.
// The quantised variants run when FwdArgs::qout is set, plain RMSNorm when
// FwdArgs::residual is null.
hipError_t launch_wave_row(const FwdArgs& a, int block_threads, int segs_per_lane,
                           int64_t grid_blocks, hipStream_t stream);

// One workgroup of block_threads per row, the row in registers:
// segs_per_thread (1, 2, 4 or 8) segments per thread.  late_weight (bf16 out
// only; hipErrorInvalidValue for codes): the weight is read for each row after
// the row's barrier instead of once per workgroup into registers.
hipError_t launch_wg_row(const FwdArgs& a, int block_threads, int segs_per_thread,
                         int64_t grid_blocks, bool late_weight, hipStream_t stream);

// One workgroup per row; pass 1 streams the row in chunks of block_threads
// segments, storing residual_out and staging fp32 sums in LDS; pass 2
// normalises from LDS.  lds_two_pass_lds_bytes() gives its LDS size.
hipError_t launch_lds_two_pass(const FwdArgs& a, int block_threads, int64_t grid_blocks,
                               hipStream_t stream);
size_t lds_two_pass_lds_bytes(int hidden);

// Any hidden in [1, 32768], any row strides, 2-byte aligned pointers
// (bf16 out only): element-wise loads and stores, the same reduction tree.
// general_lds_bytes() gives its LDS size.
hipError_t launch_general(const FwdArgs& a, int block_threads, int64_t grid_blocks,
                          hipStream_t stream);
size_t general_lds_bytes(int hidden);

// One tensor group of the packed short-row kernel: n_tokens * heads rows of
// `hidden` elements each, row (t, h) at element t * token_stride + h * hidden
// of each tensor.  residual and residual_out are null for plain RMSNorm (then
// in both groups).  heads == 0 or n_tokens == 0: no rows.
struct PackTensors {
  uint16_t* out;       // bf16 out, or null for quantised out
  void* qout;          // 1-byte codes, contiguous [rows][hidden] (quantised out), else null
  float* qscale;       // per-row scale (quantised out), else null
  uint16_t* residual_out;
  const uint16_t* x;
  const uint16_t* residual;
  const uint16_t* weight;
  int64_t x_token_stride, r_token_stride, out_token_stride, ro_token_stride;
  int64_t n_tokens;
  int64_t heads;
};

// Rows of hidden <= 512 packed several to a wavefront (the power of two P >=
// hidden / 8 lanes per row), two groups in one launch (g1 may be empty).
// qfmt 0: bf16 out; 1 int8, 2 E4M3 codes with a per-row scale (the rows'
// codes contiguous per group, row i at i * hidden bytes).  Needs hidden % 8
// == 0, every pointer and token stride on 16 bytes, and fewer than 2^31 rows
// in all.  rows_per_lane (1, 2 or 4): row groups each wavefront loads
// together; grid_blocks as launch_wave_row.
hipError_t launch_pack_rows(const PackTensors& g0, const PackTensors& g1, int32_t hidden,
                            float eps, int qfmt, int block_threads, int rows_per_lane,
                            int64_t grid_blocks, hipStream_t stream);
constexpr int64_t kPackMaxHidden = 512;
constexpr int64_t kPackMaxRows = (int64_t)1 << 31;

// Which (workgroup size, segments per thread) pairs are built: those whose
// per-thread row share fits the register file without spilling.
bool wave_row_supported(int block_threads, int segs_per_lane);
bool wg_row_supported(int block_threads, int segs_per_thread);

// Correctly rounded binary32 log1p of n elements (log1p.hip): E =
// elems_per_thread (1, 2, 4 or 8) consecutive elements per thread,
// block_threads * E per tile; grid_blocks as above (0: one workgroup per
// tile, at most 8192).  accurate_only sends every element through the double-double path.
hipError_t launch_log1p(float* out, const float* x, int64_t n, int block_threads,
                        int elems_per_thread, int64_t grid_blocks, bool accurate_only,
                        hipStream_t stream);

// Reference streams: mode 0 reads count 16-bit elements of src (dst must hold
// count elements; at most one 16-byte word per thread is ever written),
// mode 1 writes count elements to dst.
hipError_t launch_stream(uint16_t* dst, const uint16_t* src, int64_t count, int mode,
                         hipStream_t stream);

// Reference copy: d0 <- s0 and d1 <- s1, count 16-bit elements each.
hipError_t launch_copy2(uint16_t* d0, uint16_t* d1, const uint16_t* s0, const uint16_t* s1,
                        int64_t count, hipStream_t stream);

// Reference copy with row structure: d0 <- s0 and d1 <- s1, n_rows rows of
// hidden elements (hidden a multiple of 8, at most 16384), one workgroup of
// 512 threads per rows_per_burst (1, 2 or 4) rows, all loads of its rows
// issued before any store.
hipError_t launch_copy_rows(uint16_t* d0, uint16_t* d1, const uint16_t* s0, const uint16_t* s1,
                            int64_t n_rows, int hidden, int rows_per_burst, hipStream_t stream);

// Test hook: the store epilogue applied to consecutive fp32 bit patterns.
hipError_t launch_cvt_range(uint16_t* out, uint32_t start, int64_t count, hipStream_t stream);

// E4M3 codes of count consecutive fp32 bit patterns (the quantised variant's
// code routine with inv = 1); count a multiple of 8.
hipError_t launch_cvt_e4m3_range(uint8_t* out, uint32_t start, int64_t count,
                                 hipStream_t stream);

}  // namespace addrms
