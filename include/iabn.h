/*
 * iabn.h -- C ABI of the MI355X (gfx950) In-Place Activated BatchNorm library.
 *
 * The method: "In-Place Activated BatchNorm for Memory-Optimized Training of DNNs"
 * (Rota Bulo, Porzi, Kontschieder), as summarised on the paperlayer page of arXiv
 * 1712.02616v3.  Section 3 ("In-Place Activated Batch Normalization") fuses batch
 * normalisation with an invertible activation into one layer that keeps a single
 * buffer: the forward writes y over x, and the backward rebuilds everything it
 * needs from y by inverting the activation and the scale-and-shift.
 *
 * Conventions shared by every entry point
 *   - Tensors hold N*C*H*W elements of the storage dtype, contiguous, in layout
 *     NCHW (element (n,c,h,w) at ((n*C + c)*H + h)*W + w) or NHWC (at
 *     ((n*H + h)*W + w)*C + c).  Device pointers.  Element pointers must be
 *     aligned to their element size; 16-byte alignment (and H*W, resp. C, a
 *     multiple of 16/element-size) enables the 128-bit vector path, anything
 *     else takes the scalar path with identical results.
 *   - Per-channel vectors (gamma, beta, statistics, gradients) are fp32 device
 *     arrays of length C, for both storage dtypes.  Arithmetic is fp32, with the
 *     per-channel finishing steps in fp64.
 *   - m = N*H*W is the reduction length of one channel.
 *   - The caller owns every buffer, including the workspace.  The library never
 *     allocates or frees, and the compute entry points never synchronise: they
 *     are reentrant and keep no state besides one process-wide setting
 *     (iabn_set_grouped_kernels).  Only iabn_workspace_status synchronises.
 *     Calls are enqueued on `stream` and return once launched.  The status reports
 *     argument validation (done before any HIP call) and launch errors; faults
 *     inside kernels surface at the caller's next synchronisation.
 *   - Results are bitwise deterministic for a given shape, layout, dtype,
 *     pointer alignment and device CU count: no floating-point atomics, fixed
 *     reduction orders.
 *   - Calls that may run at the same time (on different streams) need separate
 *     workspaces; calls in stream order may share one.
 *   - NHWC maps, and NCHW maps whose channels are large or few, may run a
 *     kernel whose workgroups share a slice of channels or one channel and
 *     exchange partial sums through the workspace while all of them are
 *     resident (the grid never exceeds the CU count).  Should the device be held
 *     by other work so long that a partner does not arrive within about a
 *     second, the waiting workgroup gives up and its statistics, and every
 *     output computed from them, become NaN instead of the kernel hanging; it
 *     also records the timeout in the workspace, which iabn_workspace_status
 *     reports.  Callers that share the device with long-running work on other
 *     streams can switch these kernels off (iabn_set_grouped_kernels, or the
 *     environment variable IABN_GROUPED_KERNELS=0): every call then takes
 *     kernels whose workgroups never wait on one another.
 *   - Calls may be captured in a HIP graph (stream capture): they launch
 *     kernels only, with no allocation, memset, copy or synchronisation, and a
 *     replay gives the same bits as the eager call.
 *   - Preconditions that are not checked: gamma_c != 0 in the backward (the
 *     affine step must be invertible), finite inputs (NaN propagates), and no
 *     overlap between buffers other than the aliasing each call allows.
 */
#ifndef IABN_H
#define IABN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum iabn_status {
    IABN_OK = 0,
    IABN_ERR_INVALID_ARG = 1,   /* a size, enum, scalar or pointer is not acceptable  */
    IABN_ERR_UNSUPPORTED = 2,   /* valid request this build does not implement        */
    IABN_ERR_WORKSPACE = 3,     /* workspace missing or smaller than iabn_workspace_size */
    IABN_ERR_MISALIGNED = 4,    /* a pointer is not aligned to its element size       */
    IABN_ERR_HIP = 5            /* the HIP runtime reported an error at launch        */
} iabn_status;

typedef enum iabn_layout { IABN_NCHW = 0, IABN_NHWC = 1 } iabn_layout;

/* Storage dtype of x / y / dy / dx.  Arithmetic is fp32 (statistics finished in
 * fp64) for every storage dtype; stored results round to nearest even.  fp16
 * keeps IEEE binary16 subnormals and overflows to infinity. */
typedef enum iabn_dtype { IABN_F32 = 0, IABN_BF16 = 1, IABN_F16 = 2 } iabn_dtype;

/* Invertible activations (section 3, "INPLACE-ABN"; section 4, "Experimental
 * setup" uses leaky ReLU with slope 0.01).  act_param is the leaky slope
 * (must be > 0) or the ELU alpha (must be > 0); identity ignores it.
 *   leaky ReLU: y = z > 0 ? z : a*z        ELU: y = z > 0 ? z : alpha*(exp(z)-1) */
typedef enum iabn_act {
    IABN_ACT_IDENTITY = 0,
    IABN_ACT_LEAKY_RELU = 1,
    IABN_ACT_ELU = 2
} iabn_act;

/* Human-readable name of a status code (static storage). */
const char *iabn_status_string(iabn_status status);

/* Library ABI version: major*10000 + minor*100 + patch. */
int iabn_version(void);

/* Process-wide switch of the kernels whose workgroups wait on one another
 * (the exchanging kernels described above).  enabled = 1 allows them (the
 * default unless the environment variable IABN_GROUPED_KERNELS is "0" when the
 * library first plans a call), 0 forbids them: NHWC maps then take one
 * workgroup per slice of channels or the split kernels, NCHW maps one
 * workgroup per channel or the split kernels, with results equal within the
 * parity tolerances (the reduction order differs).  enabled < 0 changes
 * nothing.  Returns the setting in force before the call.  Calls planned
 * after it follow the new setting; iabn_workspace_size does not depend on it.
 * This is the only state the library keeps across calls besides per-device
 * caches of the CU count. */
int iabn_set_grouped_kernels(int enabled);

/* Reads the exchange status word that every workspace carries in its first
 * 256 bytes: *timed_out = 1 if an exchanging kernel that used this workspace
 * gave up waiting for a partner (its outputs then hold NaN) since the word was
 * last cleared, else 0.  clear != 0 resets the word after reading it.  Unlike
 * every other entry point this one synchronises `stream` (it copies the word
 * to the host); call it after the work to check, not inside graph capture.
 * A workspace whose contents were never written by the library reads as 0
 * (the recorded value is one fixed 64-bit pattern).
 * Errors: IABN_ERR_INVALID_ARG (timed_out NULL), IABN_ERR_WORKSPACE (NULL or
 * under 256 bytes), IABN_ERR_MISALIGNED, IABN_ERR_HIP (copy failed). */
iabn_status iabn_workspace_status(void *workspace, size_t workspace_bytes, int clear,
                                  int *timed_out, hipStream_t stream);

/* Bytes of device workspace that iabn_forward_train, iabn_forward_stats,
 * iabn_backward, iabn_backward_reduce and iabn_backward_eval need for this
 * shape (0 for an empty problem).  Depends on the arguments and on the current
 * device's CU count (which bounds the exchanging kernels' grid).
 * One buffer serves forward and backward of the same shape.  Returns 0 for
 * invalid arguments too. */
size_t iabn_workspace_size(int64_t N, int64_t C, int64_t H, int64_t W,
                           iabn_layout layout, iabn_dtype dtype);

/* Training forward, in place (section 3, "Batch Normalization Review" and
 * "INPLACE-ABN"; the single stored buffer of section 1):
 *   mu_c, var_c = empirical mean and biased variance of channel c over its m
 *   elements; invstd_c = 1/sqrt(var_c + eps);
 *   y = act(gamma_c * (x - mu_c) * invstd_c + beta_c), written over x.
 *   x_inout      in: x, out: y (same buffer, storage dtype, `layout`)
 *   gamma, beta  in: fp32 [C]
 *   running_mean, running_var  in/out fp32 [C], both or neither may be NULL:
 *                new = (1 - momentum)*old + momentum*batch, where the batch
 *                variance is the unbiased var_c*m/(m-1)
 *   save_mean, save_invstd     out fp32 [C]: mu_c and invstd_c
 *   eps >= 0, 0 <= momentum <= 1; training needs m >= 2.  C == 0 is a no-op.
 *   workspace    device, >= iabn_workspace_size bytes, 16-byte aligned; its
 *                contents on entry do not matter.
 * Equivalent to iabn_forward_stats followed by iabn_forward_apply. */
iabn_status iabn_forward_train(void *x_inout,
                               int64_t N, int64_t C, int64_t H, int64_t W,
                               iabn_layout layout, iabn_dtype dtype,
                               const float *gamma, const float *beta,
                               float *running_mean, float *running_var,
                               float *save_mean, float *save_invstd,
                               iabn_act act, float act_param, float eps, float momentum,
                               void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* First stage of iabn_forward_train: reads x, computes the statistics, writes
 * save_mean / save_invstd, updates the running statistics, and leaves the
 * per-channel affine constants in the workspace for iabn_forward_apply.  x is
 * not modified.  Arguments as for iabn_forward_train. */
iabn_status iabn_forward_stats(const void *x,
                               int64_t N, int64_t C, int64_t H, int64_t W,
                               iabn_layout layout, iabn_dtype dtype,
                               const float *gamma, const float *beta,
                               float *running_mean, float *running_var,
                               float *save_mean, float *save_invstd,
                               float eps, float momentum,
                               void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Second stage of iabn_forward_train: y = act(...) written over x, from the
 * constants iabn_forward_stats left in the same workspace, on the same stream,
 * for the same x, shape, layout and dtype. */
iabn_status iabn_forward_apply(void *x_inout,
                               int64_t N, int64_t C, int64_t H, int64_t W,
                               iabn_layout layout, iabn_dtype dtype,
                               iabn_act act, float act_param,
                               void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Inference forward, in place, with the running statistics: section 3, "Batch
 * Normalization Review" normalises with the minibatch statistics in training;
 * at inference the pages state no rule, and the usual one is taken, the
 * running estimates that iabn_forward_train keeps (momentum update, unbiased
 * variance) standing in for the batch statistics:
 *   y = act(gamma_c * (x - running_mean_c) / sqrt(running_var_c + eps) + beta_c)
 * written over x.  All per-channel inputs are fp32 [C] and required.  Needs no
 * workspace.  An empty tensor (any extent 0) is a no-op. */
iabn_status iabn_forward_eval(void *x_inout,
                              int64_t N, int64_t C, int64_t H, int64_t W,
                              iabn_layout layout, iabn_dtype dtype,
                              const float *gamma, const float *beta,
                              const float *running_mean, const float *running_var,
                              iabn_act act, float act_param, float eps,
                              hipStream_t stream);

/* Training backward from the stored output alone (section 3, "INPLACE-ABN" I
 * and II; Appendix, "Derivation of Gradient"):
 *   z = act^-1(y), dz = act'(z)*dy (both from y), xhat = (z - beta_c)/gamma_c,
 *   dbeta_c = sum dz, dgamma_c = sum dz*xhat,
 *   dx = gamma_c*invstd_c*(dz - dbeta_c/m - xhat*dgamma_c/m).
 *   y, dy        in, storage dtype, `layout`; y is never modified
 *   dx           out, storage dtype; may be exactly dy (in place), must not
 *                overlap y, and must not partly overlap dy
 *   gamma, beta  in fp32 [C], the values the forward used (gamma_c != 0)
 *   save_invstd  in fp32 [C], from the forward
 *   dgamma, dbeta out fp32 [C]
 *   Needs m >= 2.  C == 0 is a no-op.  Workspace as for the forward.
 * The ELU inverse clamps y/alpha to at least -1 + 2^-24, which only rounding of
 * the stored y can reach.  Equivalent to iabn_backward_reduce followed by
 * iabn_backward_apply. */
iabn_status iabn_backward(const void *y, const void *dy, void *dx,
                          int64_t N, int64_t C, int64_t H, int64_t W,
                          iabn_layout layout, iabn_dtype dtype,
                          const float *gamma, const float *beta, const float *save_invstd,
                          float *dgamma, float *dbeta,
                          iabn_act act, float act_param,
                          void *workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* First stage of iabn_backward: the per-channel sums, dgamma and dbeta, and the
 * per-channel coefficients of dx left in the workspace. */
iabn_status iabn_backward_reduce(const void *y, const void *dy,
                                 int64_t N, int64_t C, int64_t H, int64_t W,
                                 iabn_layout layout, iabn_dtype dtype,
                                 const float *gamma, const float *beta, const float *save_invstd,
                                 float *dgamma, float *dbeta,
                                 iabn_act act, float act_param,
                                 void *workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Second stage of iabn_backward: dx from y, dy and the coefficients that
 * iabn_backward_reduce left in the same workspace (same stream, shapes, act). */
iabn_status iabn_backward_apply(const void *y, const void *dy, void *dx,
                                int64_t N, int64_t C, int64_t H, int64_t W,
                                iabn_layout layout, iabn_dtype dtype,
                                iabn_act act, float act_param,
                                void *workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* Backward through iabn_forward_eval: the running statistics are frozen
 * constants of the layer, as when a pre-trained network is fine-tuned with its
 * normalisation statistics fixed (the "Eval mode" in the "Problem" section of
 * "Efficient ConvBN Blocks for Transfer Learning and Beyond").  The chain rule of
 * the inference forward, taken from the stored output alone:
 *   z = act^-1(y), dz = act'(z)*dy (both from y),
 *   dx = gamma_c * dz / sqrt(running_var_c + eps),
 *   dbeta_c = sum dz, dgamma_c = sum dz*(z - beta_c)/gamma_c.
 *   y, dy, dx    as for iabn_backward (dx may be exactly dy)
 *   gamma, beta, running_var, eps   in: the values iabn_forward_eval used
 *                (gamma_c != 0, eps >= 0)
 *   dgamma, dbeta out fp32 [C], both or neither may be NULL; when NULL the sums
 *                are skipped and only dx is written
 *   Needs m >= 1.  C == 0 is a no-op.  Workspace as for the forward.
 * HBM traffic: 3S for dx (read y, dy; write dx), 2S more for the sums. */
iabn_status iabn_backward_eval(const void *y, const void *dy, void *dx,
                               int64_t N, int64_t C, int64_t H, int64_t W,
                               iabn_layout layout, iabn_dtype dtype,
                               const float *gamma, const float *beta,
                               const float *running_var, float eps,
                               float *dgamma, float *dbeta,
                               iabn_act act, float act_param,
                               void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Optimized checkpointing (section 3, "Proposed Checkpointing"): the scheme the
 * pages weigh InPlace-ABN II against.  A BN + activation block keeps the
 * normalised xhat instead of its input x; the layer output y is rebuilt from
 * xhat (scale-and-shift, then the activation) when the following layer's
 * backward needs it, and the BN backward reads xhat itself rather than
 * recomputing it from x.  These run the split kernels (statistics pass, then an
 * elementwise pass; backward sums, then dx), on every layout, dtype and
 * activation, with the workspace of iabn_workspace_size.
 */

/* Training forward of the checkpointing block:
 *   mu_c, var_c, invstd_c, running statistics, save_mean, save_invstd exactly as
 *   iabn_forward_train;
 *   xhat = (x - mu_c)*invstd_c, written over x (the kept buffer);
 *   y = act(gamma_c*xhat' + beta_c) into y, where xhat' is xhat as stored, so
 *   that y equals what iabn_recompute_from_xhat gives from the kept buffer.
 *   y must not overlap x.  Errors as for iabn_forward_train.
 * HBM traffic: read x twice, write xhat and y (4S). */
iabn_status iabn_forward_train_ckpt(void *x_inout, void *y,
                                    int64_t N, int64_t C, int64_t H, int64_t W,
                                    iabn_layout layout, iabn_dtype dtype,
                                    const float *gamma, const float *beta,
                                    float *running_mean, float *running_var,
                                    float *save_mean, float *save_invstd,
                                    iabn_act act, float act_param, float eps, float momentum,
                                    void *workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* The layer output rebuilt from the kept buffer: y = act(gamma_c*xhat + beta_c).
 * y may be exactly xhat (in place) but must not partly overlap it.  Needs no
 * workspace; an empty tensor is a no-op.  HBM traffic 2S. */
iabn_status iabn_recompute_from_xhat(const void *xhat, void *y,
                                     int64_t N, int64_t C, int64_t H, int64_t W,
                                     iabn_layout layout, iabn_dtype dtype,
                                     const float *gamma, const float *beta,
                                     iabn_act act, float act_param, hipStream_t stream);

/* Training backward of the checkpointing block, from the kept xhat:
 *   z = gamma_c*xhat + beta_c, formed with one fused multiply-add so that the
 *   activation's branch follows the sign of the exact value; dz = act'(z)*dy;
 *   dbeta_c = sum dz, dgamma_c = sum dz*xhat,
 *   dx = gamma_c*invstd_c*(dz - dbeta_c/m - xhat*dgamma_c/m).
 *   Arguments, aliasing (dx may be exactly dy) and errors as for iabn_backward,
 *   with xhat in place of y.  HBM traffic 5S (sums, then dx). */
iabn_status iabn_backward_ckpt(const void *xhat, const void *dy, void *dx,
                               int64_t N, int64_t C, int64_t H, int64_t W,
                               iabn_layout layout, iabn_dtype dtype,
                               const float *gamma, const float *beta, const float *save_invstd,
                               float *dgamma, float *dbeta,
                               iabn_act act, float act_param,
                               void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the training
 * forward exactly as iabn_forward_train, with the same arguments, results and
 * errors, but no workspace argument.  Its workspace is a static device array of
 * IABN_NOALLOC_SCRATCH_BYTES bytes inside the library, one per device, held from
 * the library's load until the process ends; the call allocates nothing.
 *   - Shapes whose iabn_workspace_size exceeds the array are rejected with
 *     IABN_ERR_WORKSPACE before any HIP call (use iabn_forward_train).
 *   - Every call on a device shares that device's array: calls that may overlap
 *     on one device (different streams, or several host threads) race and give
 *     wrong results.  Calls in stream order are safe; the array keeps the last
 *     call's contents, which no call needs cleared.
 *   - A timeout of the exchanging kernels is recorded in the array, where
 *     iabn_workspace_status cannot reach it; callers that share the device with
 *     long-running work switch those kernels off (iabn_set_grouped_kernels).
 *   - The first call on a device looks up the array's device address (a HIP
 *     runtime query, no allocation); capture a graph after one eager call. */
#define IABN_NOALLOC_SCRATCH_BYTES (8u << 20)
iabn_status iabn_forward_train_noalloc(void *x_inout,
                                       int64_t N, int64_t C, int64_t H, int64_t W,
                                       iabn_layout layout, iabn_dtype dtype,
                                       const float *gamma, const float *beta,
                                       float *running_mean, float *running_var,
                                       float *save_mean, float *save_invstd,
                                       iabn_act act, float act_param, float eps, float momentum,
                                       hipStream_t stream);

/* Describes, as a short text, the kernels that iabn_forward_train and
 * iabn_backward launch for this problem when every tensor pointer is 16-byte
 * aligned (aligned16 != 0) or not, e.g.
 *   "forward=channel_resident(512x49) backward=channel_resident(512x49,dy_streamed)".
 * For logging, benchmarks and tests; it launches nothing.  Writes at most
 * `len` bytes including the terminating NUL into `buf` and returns the length
 * of the full description (like snprintf), or -1 for invalid arguments. */
int iabn_describe_plan(int64_t N, int64_t C, int64_t H, int64_t W,
                       iabn_layout layout, iabn_dtype dtype, iabn_act act,
                       int aligned16, char *buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* IABN_H */
