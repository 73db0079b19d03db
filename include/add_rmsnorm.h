/*
 * add_rmsnorm.h -- fused residual-add + RMSNorm forward for MI355X (gfx950),
 * bf16 storage, round-to-nearest-even on both stores.
 *
 * The operation is the one the ROCm/aiter issue "rmsnorm2d_fwd_with_add
 * truncates fp32->bf16 on gfx942, biasing residual_out and compounding across
 * layers" defines in the reference() function of its "Steps to Reproduce"
 * script, with the rounding that its "Cost of fixing" and "Additional
 * Information" sections ask for (round to nearest, ties to even, never
 * truncation).  Per row i of n_rows and column j of hidden:
 *
 *   acc_j          = fp32(x[i,j]) + fp32(residual[i,j])          (IEEE fp32 add)
 *   residual_out_j = bf16_rne(acc_j)
 *   S              = sum_j acc_j^2                                 (fp32, fixed tree)
 *   rinv           = 1 / sqrt(S / hidden + eps)                    (fp32, correctly rounded)
 *   out[i,j]       = bf16_rne((acc_j * rinv) * fp32(weight[j]))
 *
 * Results are bit-identical across runs, launch configurations and kernel
 * paths: the sum of squares always follows one reduction tree that depends on
 * hidden only (8-element segments summed in order by fused multiply-add, then
 * a balanced pairwise tree over the segments in index order, padded with +0
 * to a power of two).  residual_out equals the correctly rounded bf16 of the
 * exact x + residual; out is within one bf16 ULP of the correctly rounded
 * real value.
 *
 * Conventions shared by every entry point below:
 *   - Tensors are raw bf16 bit patterns (uint16_t), row-major: x, residual,
 *     out, residual_out are [n_rows, hidden] (contiguous, or with row strides
 *     for the *_strided entry points), weight is [hidden].
 *   - All tensor pointers are DEVICE pointers (HIP device memory, or memory
 *     the device can address).  The caller owns them; the
 *     library never allocates, frees or synchronises, keeps no state between
 *     calls, and is safe to call from several host threads.
 *   - Work is enqueued on `stream` (NULL = the null stream) and the call
 *     returns without waiting.  The caller synchronises before reading.
 *   - Argument errors are detected on the host, before anything is enqueued,
 *     and returned as a negative status; nothing is written then.  NaN and
 *     Inf in the data are not errors: they propagate per IEEE arithmetic.
 */
#ifndef ADD_RMSNORM_H
#define ADD_RMSNORM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* hipStream_t is a pointer to this opaque struct. */
struct ihipStream_t;

/* Declared below; named here so that every prototype refers to the one
 * file-scope type (in C a struct first named in a parameter list would be
 * local to that prototype). */
struct add_rmsnorm_launch_cfg;

#define ADD_RMSNORM_ABI_VERSION 10

/* Largest supported hidden size. */
#define ADD_RMSNORM_MAX_HIDDEN 32768

/* Status codes. */
#define ADD_RMSNORM_OK 0
#define ADD_RMSNORM_EINVAL (-1) /* null pointer, n_rows < 0, hidden <= 0, eps < 0 or not finite, bad cfg */
#define ADD_RMSNORM_EALIGN (-2) /* a pointer misaligned (see each entry point), or a forced fast path on a shape it cannot take */
#define ADD_RMSNORM_EALIAS (-3) /* an output partly overlaps an input, or overlaps the weight or another output */
#define ADD_RMSNORM_ERANGE (-4) /* hidden above the maximum (of the library, the chosen path or the device) */
#define ADD_RMSNORM_EHIP (-5)   /* the HIP launch failed; add_rmsnorm_last_hip_error() has the detail */

/*
 * The fused forward.
 *   out           [n_rows, hidden] bf16, written: the normalised, weighted rows.
 *   residual_out  [n_rows, hidden] bf16, written: x + residual.
 *   x, residual   [n_rows, hidden] bf16, read.
 *   weight        [hidden] bf16, read.
 *   n_rows >= 0 (0 enqueues nothing and returns OK; pointers are not checked),
 *   1 <= hidden <= ADD_RMSNORM_MAX_HIDDEN,
 *   eps finite and >= 0, added to the mean of squares inside the square root.
 * Pointers need only 2-byte alignment.  When hidden % 8 == 0 and every
 * pointer is 16-byte aligned one of the fast kernels below runs;
 * otherwise the general kernel (element-wise loads and stores, the same
 * reduction tree, so the same results).
 * In place: an output may be the very same buffer as x or residual (e.g.
 * out == x and residual_out == residual, the usual residual-stream update);
 * any other overlap of an output with an input, the weight or the other
 * output is rejected with ADD_RMSNORM_EALIAS.
 * The fast kernel is chosen by hidden: up to 256, several rows per
 * wavefront (the power of two >= hidden / 8 lanes per row); one wavefront
 * per row up to 2048, one workgroup per row with the row held in registers
 * up to 8192, and above that one workgroup per row that stages the row's
 * fp32 sums in LDS and normalises in a second pass over LDS.  Small calls
 * with hidden in [2048, 8192] (at most 4096 rows and 2^24 elements per
 * tensor) take the register kernel with a smaller workgroup that reads the
 * weight after each row's barrier (ADD_RMSNORM_FLAG_LATE_WEIGHT).
 * Returns ADD_RMSNORM_OK or a negative status.
 */
int add_rmsnorm_fwd(uint16_t* out, uint16_t* residual_out, const uint16_t* x,
                    const uint16_t* residual, const uint16_t* weight, int64_t n_rows,
                    int64_t hidden, float eps, struct ihipStream_t* stream);

/*
 * The fused forward over row-strided views, for rows that are slices of wider
 * matrices.  Row i of each tensor starts `*_stride` elements after row i - 1
 * (strides >= hidden, in elements; the weight stays contiguous).  Results are
 * those of add_rmsnorm_fwd on the same rows.  The fast kernels run when
 * hidden, every stride and every pointer are multiples of 8 elements (16
 * bytes), the general kernel otherwise.  An output may be exactly an input's
 * view (same pointer and stride: in place); any other shared element between
 * an output and an input, the other output or the weight is
 * ADD_RMSNORM_EALIAS.  Views with equal strides are tested element by element
 * (so interleaved column blocks of one matrix are fine); views with unequal
 * strides must not share any byte of their spans.  cfg may be NULL.
 */
int add_rmsnorm_fwd_strided(uint16_t* out, int64_t out_stride, uint16_t* residual_out,
                            int64_t residual_out_stride, const uint16_t* x, int64_t x_stride,
                            const uint16_t* residual, int64_t residual_stride,
                            const uint16_t* weight, int64_t n_rows, int64_t hidden, float eps,
                            const struct add_rmsnorm_launch_cfg* cfg,
                            struct ihipStream_t* stream);

/* Kernel paths for add_rmsnorm_fwd_cfg. */
#define ADD_RMSNORM_PATH_AUTO 0
#define ADD_RMSNORM_PATH_WAVE_ROW 1     /* hidden <= 4096 (2048 with 1024 threads) when forced */
#define ADD_RMSNORM_PATH_WG_ROW 2       /* hidden <= min(64 * block_threads, 16384) when forced */
#define ADD_RMSNORM_PATH_LDS_TWO_PASS 3 /* any supported hidden */
#define ADD_RMSNORM_PATH_GENERAL 4      /* any hidden, strides and 2-byte alignment (bf16 out only) */
#define ADD_RMSNORM_PATH_PACKED 5       /* hidden <= 512, several rows per wavefront */

/* flags value on ADD_RMSNORM_PATH_WG_ROW (bf16-out entry points only): the
 * weight is read for each row after the row's barrier rather than held in
 * registers from the workgroup's start.  The same results. */
#define ADD_RMSNORM_FLAG_LATE_WEIGHT 1

/*
 * Launch configuration, for tests and benchmarks that must show that results
 * do not depend on it.  Every field 0 means "the library's choice".
 *   path           one of ADD_RMSNORM_PATH_*.
 *   block_threads  workgroup size: 64, 128, 256, 512 or 1024 (the wave path
 *                  runs block_threads / 64 rows per workgroup, the packed
 *                  path block_threads / 64 wavefronts of several rows each).
 *   grid_blocks    0: the library's choice: one workgroup per row (per row
 *                  group on the wave path) for the fused fast kernels and for
 *                  small plain bf16 calls (hidden 4096-8192, at most 2^23
 *                  elements), as many as fit on the device for other plain
 *                  RMSNorm calls, the packed path and the general kernels;
 *                  > 0: exactly that many
 *                  workgroups, each looping over rows (a persistent grid);
 *                  -1: as many as fit on the device at once.
 *   flags          0, or on ADD_RMSNORM_PATH_PACKED the row groups each
 *                  wavefront loads together: 1, 2 or 4, or on
 *                  ADD_RMSNORM_PATH_WG_ROW for bf16 out
 *                  ADD_RMSNORM_FLAG_LATE_WEIGHT.
 */
struct add_rmsnorm_launch_cfg {
  int32_t path;
  int32_t block_threads;
  int32_t grid_blocks;
  int32_t flags;
};

/*
 * add_rmsnorm_fwd with an explicit launch configuration (cfg may be NULL,
 * meaning all defaults).  Same arguments, results and errors as
 * add_rmsnorm_fwd; a configuration the chosen path cannot run returns
 * ADD_RMSNORM_EINVAL (bad field), ADD_RMSNORM_ERANGE (hidden too large for
 * that path) or ADD_RMSNORM_EALIGN (a fast path forced on a shape or
 * alignment only the general path takes).  The numerical result is the same
 * for every configuration, the general path included.
 */
int add_rmsnorm_fwd_cfg(uint16_t* out, uint16_t* residual_out, const uint16_t* x,
                        const uint16_t* residual, const uint16_t* weight, int64_t n_rows,
                        int64_t hidden, float eps, const struct add_rmsnorm_launch_cfg* cfg,
                        struct ihipStream_t* stream);

/*
 * Quantised variant: the same row computation with out replaced by per-row
 * symmetric int8 codes, the FUSE_QUANT sibling of the fused kernel in the
 * aiter issue ("Cost of fixing": in the quantised configurations out goes
 * through a scaled cast instead of the bf16 conversion; the cast itself is
 * not given there, this is the plain per-row int8 reading).  With
 * y_j = (acc_j * rinv) * w_j as above (fp32):
 *   amax          = max_j |y_j|                       (exact; NaN wins)
 *   out_scale[i]  = amax / 127                        (fp32, correctly rounded)
 *   inv           = 127 / amax                        (fp32, correctly rounded)
 *   out_q[i, j]   = y_j * inv (fp32) rounded to the nearest integer, ties to
 *                   even, within [-127, 127]
 * inv must be finite, so a row is quantised only when 2^-120 <= amax <=
 * FLT_MAX; any other row (amax 0, tiny, Inf or NaN) gets all-zero codes, and
 * its scale is still amax / 127.  residual_out is exactly as in
 * add_rmsnorm_fwd and may be residual itself (in place).
 *   out_q      [n_rows, hidden] int8, written, 16-byte aligned.
 *   out_scale  [n_rows] fp32, written, 4-byte aligned.
 * Codes and scales must not overlap any other buffer (ADD_RMSNORM_EALIAS).
 * Unlike add_rmsnorm_fwd, the quantised entry points need hidden % 8 == 0
 * and 16-byte aligned rows (ADD_RMSNORM_EALIGN otherwise) and take no general
 * path; everything else (sizes, errors, stream) as add_rmsnorm_fwd.  Rows up
 * to hidden 512 take the packed kernel (several rows per wavefront).
 */
int add_rmsnorm_quant_fwd(int8_t* out_q, float* out_scale, uint16_t* residual_out,
                          const uint16_t* x, const uint16_t* residual, const uint16_t* weight,
                          int64_t n_rows, int64_t hidden, float eps, struct ihipStream_t* stream);

/* add_rmsnorm_quant_fwd with an explicit launch configuration (same results). */
int add_rmsnorm_quant_fwd_cfg(int8_t* out_q, float* out_scale, uint16_t* residual_out,
                              const uint16_t* x, const uint16_t* residual,
                              const uint16_t* weight, int64_t n_rows, int64_t hidden, float eps,
                              const struct add_rmsnorm_launch_cfg* cfg,
                              struct ihipStream_t* stream);

/*
 * FP8 quantised variant: add_rmsnorm_quant_fwd with OCP FP8 E4M3 codes
 * ("e4m3fn": 1 sign, 4 exponent (bias 7) and 3 mantissa bits, largest finite
 * value 448, no infinities), the fp8 scaled cast among the aiter issue's
 * quantised configurations ("Cost of fixing"; the cast itself is not given
 * there, this is the per-row reading with E4M3's range).  Per row:
 *   out_scale[i]  = amax / 448                        (fp32, correctly rounded)
 *   inv           = 448 / amax                        (fp32, correctly rounded)
 *   out_q[i, j]   = the E4M3 value nearest to y_j * inv (fp32), ties to the
 *                   even code; |y_j * inv| never rounds past 448, so no code
 *                   is NaN
 * A row is quantised only when 2^-118 <= amax <= FLT_MAX (448 / amax
 * finite); other rows get all-zero codes and the scale amax / 448.  Codes
 * are bytes (0x80 is -0).  Arguments, alignment, aliasing and errors exactly
 * as add_rmsnorm_quant_fwd.
 */
int add_rmsnorm_quant_fp8_fwd(uint8_t* out_q, float* out_scale, uint16_t* residual_out,
                              const uint16_t* x, const uint16_t* residual,
                              const uint16_t* weight, int64_t n_rows, int64_t hidden, float eps,
                              struct ihipStream_t* stream);

/* add_rmsnorm_quant_fp8_fwd with an explicit launch configuration (same results). */
int add_rmsnorm_quant_fp8_fwd_cfg(uint8_t* out_q, float* out_scale, uint16_t* residual_out,
                                  const uint16_t* x, const uint16_t* residual,
                                  const uint16_t* weight, int64_t n_rows, int64_t hidden,
                                  float eps, const struct add_rmsnorm_launch_cfg* cfg,
                                  struct ihipStream_t* stream);

/*
 * Plain RMSNorm: the row computation above without the residual add, for the
 * other norms with bf16 stores that the aiter issue's "Notes" list beside the
 * fused kernel (the q/k norms, the norm kernel used above hidden 8192).  Per
 * row: acc_j = fp32(x[i,j]) exactly (no addition, so -0 stays -0), then S,
 * rinv and out as in add_rmsnorm_fwd, with the same fixed reduction tree and
 * round-to-nearest-even store.  The result is bit for bit add_rmsnorm_fwd's
 * out with a residual of all -0 (x + -0 = x in IEEE arithmetic).
 *   out     [n_rows, hidden] bf16, written; may be x itself (in place), any
 *           other overlap with x or the weight is ADD_RMSNORM_EALIAS.
 *   x       [n_rows, hidden] bf16, read.  weight [hidden] bf16, read.
 * Sizes, alignment, eps, errors, kernel choice and stream as add_rmsnorm_fwd.
 */
int rmsnorm_fwd(uint16_t* out, const uint16_t* x, const uint16_t* weight, int64_t n_rows,
                int64_t hidden, float eps, struct ihipStream_t* stream);

/* rmsnorm_fwd with an explicit launch configuration (same results). */
int rmsnorm_fwd_cfg(uint16_t* out, const uint16_t* x, const uint16_t* weight, int64_t n_rows,
                    int64_t hidden, float eps, const struct add_rmsnorm_launch_cfg* cfg,
                    struct ihipStream_t* stream);

/* rmsnorm_fwd over row-strided views, as add_rmsnorm_fwd_strided (out may
 * be exactly x's view). */
int rmsnorm_fwd_strided(uint16_t* out, int64_t out_stride, const uint16_t* x, int64_t x_stride,
                        const uint16_t* weight, int64_t n_rows, int64_t hidden, float eps,
                        const struct add_rmsnorm_launch_cfg* cfg, struct ihipStream_t* stream);

/*
 * Plain RMSNorm with int8 out: rmsnorm_fwd's row computation followed by the
 * per-row quantisation of add_rmsnorm_quant_fwd (same scale, inverse scale,
 * rounding and zero-code rule).  Codes and scales must not overlap x, the
 * weight or each other (ADD_RMSNORM_EALIAS).  Like add_rmsnorm_quant_fwd it
 * needs hidden % 8 == 0 and 16-byte aligned x and weight.
 *   out_q      [n_rows, hidden] int8, written, 16-byte aligned.
 *   out_scale  [n_rows] fp32, written, 4-byte aligned.
 */
int rmsnorm_quant_fwd(int8_t* out_q, float* out_scale, const uint16_t* x, const uint16_t* weight,
                      int64_t n_rows, int64_t hidden, float eps, struct ihipStream_t* stream);

/* rmsnorm_quant_fwd with an explicit launch configuration (same results). */
int rmsnorm_quant_fwd_cfg(int8_t* out_q, float* out_scale, const uint16_t* x,
                          const uint16_t* weight, int64_t n_rows, int64_t hidden, float eps,
                          const struct add_rmsnorm_launch_cfg* cfg, struct ihipStream_t* stream);

/*
 * Plain RMSNorm with FP8 E4M3 out: rmsnorm_quant_fwd with the codes, scale
 * and zero-code rule of add_rmsnorm_quant_fp8_fwd.  Arguments as
 * rmsnorm_quant_fwd.
 */
int rmsnorm_quant_fp8_fwd(uint8_t* out_q, float* out_scale, const uint16_t* x,
                          const uint16_t* weight, int64_t n_rows, int64_t hidden, float eps,
                          struct ihipStream_t* stream);

/* rmsnorm_quant_fp8_fwd with an explicit launch configuration (same results). */
int rmsnorm_quant_fp8_fwd_cfg(uint8_t* out_q, float* out_scale, const uint16_t* x,
                              const uint16_t* weight, int64_t n_rows, int64_t hidden, float eps,
                              const struct add_rmsnorm_launch_cfg* cfg,
                              struct ihipStream_t* stream);

/*
 * The four quantised entry points over row-strided views of x, residual and
 * residual_out (rows that are slices of wider matrices): row i of each view
 * starts `*_stride` elements after row i - 1 (strides >= hidden, multiples of
 * 8; ADD_RMSNORM_EINVAL below hidden, ADD_RMSNORM_EALIGN off 8).  Codes and
 * scales stay contiguous ([n_rows, hidden] bytes and [n_rows] fp32) and
 * overlap nothing.  residual_out may be exactly residual's or x's view (same
 * pointer and stride: in place); any other shared element with an input or
 * the weight is ADD_RMSNORM_EALIAS (with different strides, any overlap of
 * the views' spans).  Results are those of the contiguous entry points on the
 * same rows; everything else as there.  cfg may be NULL.
 */
int add_rmsnorm_quant_fwd_strided(int8_t* out_q, float* out_scale, uint16_t* residual_out,
                                  int64_t residual_out_stride, const uint16_t* x,
                                  int64_t x_stride, const uint16_t* residual,
                                  int64_t residual_stride, const uint16_t* weight, int64_t n_rows,
                                  int64_t hidden, float eps,
                                  const struct add_rmsnorm_launch_cfg* cfg,
                                  struct ihipStream_t* stream);
int add_rmsnorm_quant_fp8_fwd_strided(uint8_t* out_q, float* out_scale, uint16_t* residual_out,
                                      int64_t residual_out_stride, const uint16_t* x,
                                      int64_t x_stride, const uint16_t* residual,
                                      int64_t residual_stride, const uint16_t* weight,
                                      int64_t n_rows, int64_t hidden, float eps,
                                      const struct add_rmsnorm_launch_cfg* cfg,
                                      struct ihipStream_t* stream);
int rmsnorm_quant_fwd_strided(int8_t* out_q, float* out_scale, const uint16_t* x,
                              int64_t x_stride, const uint16_t* weight, int64_t n_rows,
                              int64_t hidden, float eps, const struct add_rmsnorm_launch_cfg* cfg,
                              struct ihipStream_t* stream);
int rmsnorm_quant_fp8_fwd_strided(uint8_t* out_q, float* out_scale, const uint16_t* x,
                                  int64_t x_stride, const uint16_t* weight, int64_t n_rows,
                                  int64_t hidden, float eps,
                                  const struct add_rmsnorm_launch_cfg* cfg,
                                  struct ihipStream_t* stream);

/*
 * Per-head RMSNorm of attention queries and keys, bf16 out.  The aiter
 * issue's notes list a fused q/k norm kernel among those whose bf16 stores
 * were not audited for rounding; the page does not spell out its arithmetic.
 * This entry point takes the reading of the q/k normalisation in the decoder
 * the issue's RL run uses (Qwen3-8B): every head vector of head_dim elements
 * is one rmsnorm_fwd row over head_dim, q heads with q_weight and k heads
 * with k_weight, the same eps, each out element rounded once to bf16 (nearest,
 * ties to even).  Results are bit for bit rmsnorm_fwd's on the same rows, and
 * do not depend on the launch.  Both tensors go in one launch.
 *
 * Layout: token t, head h of q is the head_dim elements at
 * q + t * q_stride + h * head_dim (heads contiguous within a token, tokens
 * q_stride elements apart: q may be a column slice of a fused qkv
 * projection).  k, q_out and k_out likewise with their own token strides.
 *   q_out, k_out  written; q_out may be exactly q's view (same pointer and
 *                 stride: in place), k_out exactly k's; any other overlap of
 *                 an output with an input, the other output or a weight is
 *                 ADD_RMSNORM_EALIAS.
 *   q, k          read.  q_weight, k_weight [head_dim] bf16, read.
 *   n_tokens >= 0 (0: a no-op, nothing checked beyond the scalars);
 *   n_q_heads, n_k_heads >= 0 (a tensor with no heads is not touched and its
 *   pointers may be NULL); strides in elements, each at least
 *   heads * head_dim.
 * Requirements: head_dim in [8, 512] and a multiple of 8, every pointer
 * 16-byte aligned and every stride a multiple of 8 (else ADD_RMSNORM_EALIGN;
 * head_dim above 512 is ADD_RMSNORM_ERANGE), fewer than 2^31 head rows in
 * all (else ADD_RMSNORM_ERANGE).  eps finite and >= 0.  Other errors,
 * ownership and stream as add_rmsnorm_fwd.
 */
int qk_rmsnorm_fwd(uint16_t* q_out, uint16_t* k_out, const uint16_t* q, const uint16_t* k,
                   const uint16_t* q_weight, const uint16_t* k_weight, int64_t n_tokens,
                   int64_t n_q_heads, int64_t n_k_heads, int64_t head_dim, int64_t q_stride,
                   int64_t k_stride, int64_t q_out_stride, int64_t k_out_stride, float eps,
                   struct ihipStream_t* stream);

/* qk_rmsnorm_fwd with an explicit launch configuration (path AUTO or
 * ADD_RMSNORM_PATH_PACKED; same results). */
int qk_rmsnorm_fwd_cfg(uint16_t* q_out, uint16_t* k_out, const uint16_t* q, const uint16_t* k,
                       const uint16_t* q_weight, const uint16_t* k_weight, int64_t n_tokens,
                       int64_t n_q_heads, int64_t n_k_heads, int64_t head_dim,
                       int64_t q_stride, int64_t k_stride, int64_t q_out_stride,
                       int64_t k_out_stride, float eps, const struct add_rmsnorm_launch_cfg* cfg,
                       struct ihipStream_t* stream);

/*
 * Test hook for the store epilogue: out[i] = bf16_rne of the fp32 whose bit
 * pattern is (start + i) mod 2^32, for 0 <= i < count, converted by the same
 * device routine that rounds both stores of the fused kernels.  out is a
 * device pointer to count uint16_t, 16-byte aligned; count >= 0 and a
 * multiple of 8.  Enqueued on stream like the forward.
 */
int add_rmsnorm_test_cvt_range(uint16_t* out, uint32_t start, int64_t count,
                               struct ihipStream_t* stream);

/*
 * Test hook for the FP8 code routine: out[i] = the E4M3 code (as stored by
 * the fp8 quantised entry points, with inv = 1) of the fp32 whose bit
 * pattern is (start + i) mod 2^32.  Meaningful for |value| < 464 (beyond,
 * the conversion's out-of-range result, which the quantised entry points
 * never reach).  out: device pointer to count bytes, 16-byte aligned; count
 * >= 0 and a multiple of 8.  Enqueued on stream.
 */
int add_rmsnorm_test_cvt_e4m3_range(uint8_t* out, uint32_t start, int64_t count,
                                    struct ihipStream_t* stream);

/*
 * Measurement hook: dst0 <- src0 and dst1 <- src1, count 16-bit elements
 * each, with the fused kernels' memory access pattern (16-byte nontemporal
 * loads and stores) and no arithmetic.  Moving the same bytes as one fused
 * call, it gives the streaming rate that call can at best reach on the
 * device.  Device pointers, 16-byte aligned, count a multiple of 8; no
 * buffer may overlap another (ADD_RMSNORM_EALIAS).  Enqueued on stream.
 */
int add_rmsnorm_test_copy2(uint16_t* dst0, uint16_t* dst1, const uint16_t* src0,
                           const uint16_t* src1, int64_t count, struct ihipStream_t* stream);

/*
 * Measurement hook: the copy of add_rmsnorm_test_copy2 with the fused
 * kernels' row structure: dst0 <- src0 and dst1 <- src1, n_rows contiguous
 * rows of hidden 16-bit elements each.  One workgroup of 512 threads takes
 * rows_per_burst (1, 2 or 4) consecutive rows and issues every load of them
 * before any store, so each compute unit's traffic comes in same-direction
 * bursts (with 1, exactly the register kernel's access pattern).  hidden a
 * multiple of 8 (ADD_RMSNORM_EALIGN) and at most 16384, n_rows at most 2^30
 * (ADD_RMSNORM_ERANGE); device pointers, 16-byte aligned; no buffer may
 * overlap another (ADD_RMSNORM_EALIAS).  Enqueued on stream.
 */
int add_rmsnorm_test_copy_rows(uint16_t* dst0, uint16_t* dst1, const uint16_t* src0,
                               const uint16_t* src1, int64_t n_rows, int64_t hidden,
                               int rows_per_burst, struct ihipStream_t* stream);

/*
 * Measurement hook: one-directional streams with the same access pattern as
 * add_rmsnorm_test_copy2.  mode 0 reads count 16-bit elements of src and
 * writes (almost) nothing; dst must hold count elements and not overlap src.
 * mode 1 writes count elements of dst (bf16 1.0) and reads nothing; src is
 * unused.  With the copy they give the device's read-only, write-only and
 * 50/50 streaming rates, the bounds of the fused kernels' traffic mix.
 * Device pointers, 16-byte aligned, count a multiple of 8.  Enqueued on
 * stream.
 */
int add_rmsnorm_test_stream(uint16_t* dst, const uint16_t* src, int64_t count, int mode,
                            struct ihipStream_t* stream);

/* Human-readable text of a status code (static storage). */
const char* add_rmsnorm_strerror(int status);

/* Text of the HIP error behind the last ADD_RMSNORM_EHIP on this thread. */
const char* add_rmsnorm_last_hip_error(void);

/* ADD_RMSNORM_ABI_VERSION of the built library; bindings refuse a mismatch. */
int add_rmsnorm_abi_version(void);

/* Target architecture, compiler flags and source digest of the build. */
const char* add_rmsnorm_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* ADD_RMSNORM_H */
