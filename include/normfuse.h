/*
 * normfuse.h -- C ABI of the fused LayerNorm / RMSNorm library for AMD
 * Instinct MI355X (gfx950).
 *
 * Operations
 *  ln_fwd / rms_fwd : fused (bias +) residual + LayerNorm / RMSNorm forward
 *      with an optional FP8-scaling amax of the normalised output.  The
 *      operation is the one spelled out in nvFuser issue #1660 ("performance
 *      optimization for moving distributive reduction operation across
 *      broadcast dimensions"), layernorm + amax comment:
 *          out1 = (x + bias) + residual, viewed as rows of the hidden size N
 *          out2 = layer_norm(out1, gamma, beta, eps)
 *          amax = max |out2|, overwriting the amax tensor.
 *      The same comment asks for the amax to be split so that its first
 *      stage runs inside the normalisation kernel; IREE issue #9139
 *      ("Investigate a fusion opportunity on Layer Normalization") asks for
 *      mean, variance and normalisation to read the source data once.  Both
 *      hold here: every [M, N] input is read once and every output written
 *      once, in one kernel.
 *  ln_bwd / rms_bwd : backward.  PyTorch PR #165370 (Inductor mix-order
 *      reduction), PR description: the dx reduction runs over the hidden
 *      dimension and the dgamma / dbeta reduction over all B x T rows; both
 *      read dy and x, which are loaded once here, and the outer reduction
 *      ends with a down-cast when dgamma / dbeta are low precision.  The
 *      optional dbias is the backward of the forward's fused add (the
 *      nvFuser comment's out1 = (x + bias) + residual): a third reduction
 *      over the rows, of dx, in the same pass; x and residual receive dx.
 *
 * Definitions (the pages call PyTorch's layer_norm; these are its semantics)
 *   u      = round_io((x + bias) + residual)          (absent terms are 0)
 *   LN     : mean = sum(u)/N, var = sum((u-mean)^2)/N, rstd = 1/sqrt(var+eps)
 *            y = (u - mean) * rstd * gamma + beta
 *   RMS    : rstd = 1/sqrt(sum(u^2)/N + eps),  y = u * rstd * gamma (+ beta)
 *   amax   = max over all elements of |y| as stored (after rounding)
 *   bwd    : xhat = (x-mean)*rstd (LN) or x*rstd (RMS), g = dy*gamma,
 *            dx = rstd*(g - mean_j(g) - xhat*mean_j(g*xhat))   (LN)
 *            dx = rstd*(g - xhat*mean_j(g*xhat))                (RMS)
 *            dgamma_j = sum_i dy_ij*xhat_ij,  dbeta_j = sum_i dy_ij,
 *            dbias_j = sum_i dx_ij (dx before rounding)
 *   Arithmetic is fp32 throughout; round_io rounds to the I/O dtype to
 *   nearest, ties to even.  The normalisation reads the rounded u, which is
 *   also what residual_out holds.
 *
 * Conventions shared by every entry point
 *   Layout   : [M, N] tensors are dense row-major (row stride N elements);
 *              M is every leading dimension flattened.  [N] vectors (bias,
 *              gamma, beta, dgamma, dbeta) are dense.  mean / rstd are fp32
 *              [M].
 *   Memory   : every pointer is device memory owned by the caller.  The
 *              library allocates nothing, frees nothing and keeps no pointer
 *              after a call returns.  ln_bwd / rms_bwd take a caller-owned
 *              workspace whose size norm_bwd_workspace_size reports.
 *   Streams  : all work is enqueued on `stream` (a hipStream_t; NULL is the
 *              default stream) and the call returns without synchronising.
 *              Work of one call is ordered by that stream.
 *   Errors   : arguments are checked before anything is enqueued; on an
 *              error the call returns a status other than NORM_OK and
 *              enqueues nothing.  NORM_ERR_LAUNCH reports a failed launch;
 *              faults during execution appear at the caller's next
 *              synchronisation, as in HIP.
 *   Aliasing : an [M, N] output may be the very tensor (same pointer) of an
 *              [M, N] input of the same call: y or residual_out over x or
 *              residual, dx over dy or x, softmax's y over x (every row group
 *              is loaded before the same workgroup stores its outputs, and no
 *              other workgroup reads those rows).  FP8 codes may not overlap
 *              an input.  No other overlap between tensors is allowed, nor
 *              between outputs.
 *   Threads  : calls are thread-safe; the library keeps no state between
 *              calls.
 *   Results  : deterministic: the same inputs give bit-identical outputs.
 *              The kernel shape, the grid and every summation order follow
 *              from M, N, the dtypes and the pointers' alignment alone.
 *   Tuning   : this library reads no environment variables.  Its test
 *              build, libnormfuse_tuning.so (same kernels and entry points),
 *              also honours tuning overrides read at every call, for tests
 *              that cross-check kernel shapes against each other and for
 *              measurements: NORMFUSE_FWD_SHAPE / _BWD_SHAPE
 *              ("LPRxVPL[xTEAMS]"; the forward's also for softmax),
 *              NORMFUSE_FWD_GROUPS_PER_WG /
 *              _BWD_GROUPS_PER_WG, NORMFUSE_FWD_INTERLEAVE / _BWD_INTERLEAVE
 *              (results stay within the same tolerances, but column sums
 *              may round differently), NORMFUSE_WT_BYTES (output bytes,
 *              counted from the end of a call, stored write-through: a cache
 *              policy, values do not change; NORMFUSE_FWD_WT_BYTES /
 *              _BWD_WT_BYTES for one direction), NORMFUSE_BWD_SPLIT=0 / 1
 *              (turns off / forces the backward's split of rows along N)
 *              and NORMFUSE_PAIRS=0 (turns the odd-row kernels below off:
 *              such rows then take the narrower vectors N allows).
 *   Alignment: pointers must be aligned to their element size.  Each call
 *              takes the widest vector access of 16, 8 or 4 bytes (fp32: 16
 *              or 8) that N is a multiple of (in elements) and that every
 *              [M, N] / [N] pointer is aligned to, else single elements.
 *              Rows whose N is an odd multiple of a unit U of 1, 2 or
 *              (bf16) 4 elements, with [M, N] pointers aligned to 2U
 *              elements (an FP8 output to 2U bytes), are read in aligned
 *              vectors of 2U elements from each row's first such element,
 *              plus one unit by itself ("odd-row" kernels; 2U elements are
 *              wider than the rule above allows).  The forward and softmax
 *              take them up to NORM_N_MAX (the fp32 forward up to 8193 /
 *              8194 for U = 1 / 2), the backward up to 8193 (U = 1), 8194
 *              (U = 2) or 8196 (U = 4); for U = 2 and 4 the
 *              backward takes a row across several waves only where that
 *              leaves fewer lanes idle than the vector kernel (on teams of
 *              256 lanes, also where 70% of them are busy).  All give
 *              results within the same tolerances, fastest with 16-byte
 *              aligned tensors and N a multiple of 8 (bf16) or 4 (fp32).
 *   Sizes    : 0 <= M; 1 <= N <= NORM_N_MAX.  M = 0 enqueues only what
 *              defines the outputs (amax = 0, dgamma = dbeta = dbias = 0), and then
 *              the [M, N] and [M] pointers may be NULL.
 */
#ifndef NORMFUSE_H
#define NORMFUSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of tensors (the "I/O dtype") and of dgamma / dbeta. */
#define NORM_F32 0  /* IEEE binary32 */
#define NORM_BF16 1 /* bfloat16 (upper half of a binary32) */

/* Status codes. */
typedef int32_t norm_status_t;
#define NORM_OK 0
#define NORM_ERR_NULL 1      /* a required pointer is NULL */
#define NORM_ERR_SHAPE 2     /* M < 0, N < 1 or N > NORM_N_MAX */
#define NORM_ERR_ARG 3       /* eps negative or NaN, or an argument the op does not take */
#define NORM_ERR_DTYPE 4     /* unknown dtype code */
#define NORM_ERR_ALIGN 5     /* a pointer is not aligned to its element size */
#define NORM_ERR_WORKSPACE 6 /* workspace NULL or smaller than norm_bwd_workspace_size */
#define NORM_ERR_LAUNCH 7    /* a kernel launch failed */
#define NORM_ERR_DEVICE 8    /* no usable HIP device, or a device query failed */

/* Largest row length any entry point accepts. */
#define NORM_N_MAX 16384

/*
 * Option bits (`flags` of every compute entry point; others: NORM_ERR_ARG).
 * NORM_ZERO_CENTERED_GAMMA -- gamma is stored around 0 and the weight is
 *     w = 1 + gamma, formed in the I/O dtype: the `zero_centered_gamma`
 *     branch of the nvFuser issue's layernorm + amax comment.  An absent
 *     gamma is then a weight of 1.  In the backward, dx uses w and dgamma
 *     (= dL/dw) keeps its form.
 * NORM_DPARAM_MEAN (backward only) -- dgamma / dbeta / dbias are the mean
 *     over the M rows instead of the sum: the "division for mean" epilogue of
 *     the outer reduction in PyTorch PR #165370 (description, step 3).
 */
#define NORM_ZERO_CENTERED_GAMMA 1u
#define NORM_DPARAM_MEAN 2u

/*
 * ln_fwd -- fused (bias +) residual + LayerNorm forward.
 *   x            [M,N] dtype   required
 *   bias         [N]   dtype   optional (NULL: no bias)
 *   residual     [M,N] dtype   optional (NULL: no residual)
 *   gamma        [N]   dtype   optional (NULL: 1)
 *   beta         [N]   dtype   optional (NULL: 0)
 *   eps          >= 0, finite
 *   y            [M,N] dtype   required
 *   residual_out [M,N] dtype   optional: u, the rounded sum that was normalised
 *   mean, rstd   [M]   fp32    optional
 *   amax         [1]   fp32    optional: overwritten with max |y| (0 when M = 0)
 *   amax_ws      NORM_AMAX_WS_BYTES of device memory, 4-byte aligned, optional
 *                (ignored without amax).  Without it the call zeroes amax with
 *                a one-thread kernel before the forward kernel, whose
 *                workgroups then combine their maxima into it; with it the
 *                forward kernel alone produces amax: the workgroups combine
 *                their maxima in the workspace and the last one to finish
 *                writes amax.  The workspace must hold zeros before its first
 *                use (e.g. hipMemset once after allocation); every call leaves
 *                it zero-filled again when it completes, so it can be reused
 *                by calls ordered on one stream.  Calls that may run at the
 *                same time must not share one.  A call that did not complete
 *                (a fault) can leave it non-zero.
 *   flags        0 or NORM_ZERO_CENTERED_GAMMA
 *   stream       hipStream_t
 */
#define NORM_AMAX_WS_BYTES 4160
norm_status_t ln_fwd(const void *x, const void *bias, const void *residual, const void *gamma,
                     const void *beta, float eps, int64_t M, int64_t N, int32_t dtype, void *y,
                     void *residual_out, float *mean, float *rstd, float *amax, void *amax_ws,
                     uint32_t flags, void *stream);

/*
 * rms_fwd -- fused (bias +) residual + RMSNorm forward.  Arguments as ln_fwd;
 * `mean` must be NULL (RMSNorm has no mean; NORM_ERR_ARG otherwise).  beta is
 * an optional additive shift after the scale.
 */
norm_status_t rms_fwd(const void *x, const void *bias, const void *residual, const void *gamma,
                      const void *beta, float eps, int64_t M, int64_t N, int32_t dtype, void *y,
                      void *residual_out, float *mean, float *rstd, float *amax, void *amax_ws,
                      uint32_t flags, void *stream);

/*
 * ln_fwd_fp8 / rms_fwd_fp8 -- the same forward with y emitted as OCP FP8
 * E4M3 codes for a following FP8 matrix product: the output the nvFuser
 * issue's layernorm + amax comment obtains the scaling amax for.  Arguments
 * as ln_fwd / rms_fwd, except:
 *   y_scale      [1]   fp32    device memory, required when M > 0: each
 *                              output is y * (*y_scale) (a scale that can
 *                              come from a previous call's amax, e.g.
 *                              448 / amax, without a host round trip)
 *   y_fp8        [M,N] uint8   required when M > 0: E4M3 codes (sign, 4-bit
 *                              exponent with bias 7, 3-bit mantissa) of
 *                              round_io(y) * (*y_scale), the product rounded
 *                              to fp32 and then to nearest E4M3, ties to
 *                              even; magnitudes beyond 448 saturate to 448.
 *                              Any alignment; 16 / sizeof(dtype)-byte
 *                              alignment keeps the vectorised kernels.
 *   amax         as ln_fwd: max |round_io(y)|, before the scale.
 * residual_out, mean, rstd and amax are bit-identical to those of ln_fwd /
 * rms_fwd on the same inputs when both calls take the same kernels (their
 * pointers fall in the same alignment class).
 */
norm_status_t ln_fwd_fp8(const void *x, const void *bias, const void *residual,
                         const void *gamma, const void *beta, float eps, int64_t M, int64_t N,
                         int32_t dtype, const float *y_scale, void *y_fp8, void *residual_out,
                         float *mean, float *rstd, float *amax, void *amax_ws, uint32_t flags,
                         void *stream);
norm_status_t rms_fwd_fp8(const void *x, const void *bias, const void *residual,
                          const void *gamma, const void *beta, float eps, int64_t M, int64_t N,
                          int32_t dtype, const float *y_scale, void *y_fp8, void *residual_out,
                          float *mean, float *rstd, float *amax, void *amax_ws, uint32_t flags,
                          void *stream);

/*
 * softmax_fwd -- row softmax in one read of x: per row, the max, the sum of
 * exp(x - max), and y = exp(x - max) / sum.  The other normalisation IREE
 * issue #9139 ("Investigate a fusion opportunity on Layer Normalization")
 * walks through fusing into a single dispatch; here it runs on the same
 * row kernels as the LayerNorm forward.
 *   x            [M,N] dtype   required (finite values)
 *   y            [M,N] dtype   required
 *   flags        0 (reserved)
 * Conventions as above (M = 0: nothing to do).
 */
norm_status_t softmax_fwd(const void *x, int64_t M, int64_t N, int32_t dtype, void *y,
                          uint32_t flags, void *stream);

/*
 * norm_bwd_workspace_size -- bytes of device workspace ln_bwd / rms_bwd need
 * for an [M, N] problem of the given dtype on the current device (the
 * per-workgroup dgamma / dbeta / dbias column partials, and for rows split
 * along N their per-chunk row sums; the size covers a call that asks for
 * dbias).  Writes 0 when none is needed.  (In the test build, query it
 * under the same tuning overrides as the call.)  The workspace
 * needs no initialisation and may be reused by calls ordered on one stream.
 */
norm_status_t norm_bwd_workspace_size(int64_t M, int64_t N, int32_t dtype, size_t *bytes);

/*
 * ln_bwd -- LayerNorm backward with the mix-order (one-load) reduction.
 *   dy           [M,N] dtype   required
 *   x            [M,N] dtype   required: the tensor that was normalised
 *                              (the forward's residual_out when it fused an add)
 *   gamma        [N]   dtype   optional (NULL: 1)
 *   mean, rstd   [M]   fp32    required (as saved by ln_fwd)
 *   dx           [M,N] dtype   required
 *   dgamma       [N]   dparam_dtype  optional
 *   dbeta        [N]   dparam_dtype  optional
 *   dbias        [N]   dparam_dtype  optional: gradient of the bias of a
 *                              forward that fused (x + bias) + residual (the
 *                              column sums of dx); x and residual both
 *                              receive dx itself
 *   dparam_dtype NORM_F32 or NORM_BF16: dgamma / dbeta / dbias are summed in
 *                fp32 and rounded (to nearest, ties to even) to this type
 *   workspace    device memory of at least norm_bwd_workspace_size bytes,
 *                16-byte aligned (may be NULL when that size is 0)
 *   flags        NORM_ZERO_CENTERED_GAMMA and / or NORM_DPARAM_MEAN
 */
norm_status_t ln_bwd(const void *dy, const void *x, const void *gamma, const float *mean,
                     const float *rstd, int64_t M, int64_t N, int32_t dtype, void *dx,
                     void *dgamma, void *dbeta, void *dbias, int32_t dparam_dtype,
                     void *workspace, size_t workspace_bytes, uint32_t flags, void *stream);

/*
 * rms_bwd -- RMSNorm backward with the mix-order reduction.  Arguments as
 * ln_bwd, except: no mean; rstd [M] fp32 is optional -- NULL recomputes it
 * from x with `eps` inside the same pass (eps is ignored when rstd is given);
 * dbeta (optional) is the gradient of the optional shift beta.
 */
norm_status_t rms_bwd(const void *dy, const void *x, const void *gamma, const float *rstd,
                      float eps, int64_t M, int64_t N, int32_t dtype, void *dx, void *dgamma,
                      void *dbeta, void *dbias, int32_t dparam_dtype, void *workspace,
                      size_t workspace_bytes, uint32_t flags, void *stream);

/*
 * ln_bwd_noalloc -- ln_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and kernels, with the column partials in
 * the library's own static device scratch instead of a caller workspace.
 * Arguments as ln_bwd without workspace / workspace_bytes.
 *   - The scratch is NORM_STATIC_SCRATCH_BYTES per device, part of the
 *     library's code object; each device that runs the call holds it until
 *     the process ends.  A problem whose workspace (norm_bwd_workspace_size)
 *     exceeds it returns NORM_ERR_WORKSPACE and enqueues nothing.
 *   - The call allocates nothing; on its first call on a device it looks up
 *     that device's scratch address (hipGetSymbolAddress; NORM_ERR_DEVICE if
 *     that fails).  The scratch is the current device's: `stream` must be
 *     NULL or a stream of the current device (NORM_ERR_DEVICE otherwise).
 *   - Every call on a device shares that device's scratch: calls that may
 *     run at the same time on one device (different streams, or different
 *     threads' streams) race and give wrong results; order them on one
 *     stream.  The scratch needs no initialisation.
 */
#define NORM_STATIC_SCRATCH_BYTES (32u << 20)
norm_status_t ln_bwd_noalloc(const void *dy, const void *x, const void *gamma, const float *mean,
                             const float *rstd, int64_t M, int64_t N, int32_t dtype, void *dx,
                             void *dgamma, void *dbeta, void *dbias, int32_t dparam_dtype,
                             uint32_t flags, void *stream);

/* Static text for a status code. */
const char *norm_status_string(norm_status_t status);

/*
 * norm_describe -- the launches a call of operation `op` on an [M, N]
 * problem of `dtype` would make, as text in buf (at most len - 1 characters
 * and a terminating NUL): kernel template arguments, grid, row groups per
 * workgroup, and for the backward the column-sum launches.  Enqueues
 * nothing and touches no device; for profilers and benchmarks that label
 * what they timed.  It runs the same planning code as the calls and assumes
 * their pointers are 16-byte aligned.
 *   op    NORM_OP_LN_FWD, NORM_OP_RMS_FWD (ln_fwd / rms_fwd and their _fp8
 *         forms), NORM_OP_LN_BWD, NORM_OP_RMS_BWD, NORM_OP_SOFTMAX
 *   opts  NORM_DESCRIBE_AMAX (forward asked for amax), NORM_DESCRIBE_AMAX_WS
 *         (and passed an amax_ws), NORM_DESCRIBE_FP8 (the _fp8 forward),
 *         NORM_DESCRIBE_DBIAS (backward asked for dbias)
 * Errors: buf NULL or len 0 -> NORM_ERR_NULL; dtype / shape as the calls;
 * unknown op or opts -> NORM_ERR_ARG.
 */
#define NORM_OP_LN_FWD 0
#define NORM_OP_RMS_FWD 1
#define NORM_OP_LN_BWD 2
#define NORM_OP_RMS_BWD 3
#define NORM_OP_SOFTMAX 4
#define NORM_DESCRIBE_AMAX 1u
#define NORM_DESCRIBE_FP8 2u
#define NORM_DESCRIBE_DBIAS 4u
#define NORM_DESCRIBE_AMAX_WS 8u
norm_status_t norm_describe(int32_t op, int64_t M, int64_t N, int32_t dtype, uint32_t opts,
                            char *buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* NORMFUSE_H */
