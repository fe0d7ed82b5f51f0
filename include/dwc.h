/*
 * dwc.h -- C ABI of libdwc, depthwise convolution (DWC) for AMD MI355X
 * (gfx950).
 *
 * The operations are those of "Flash-DWC: Making Depthwise Convolution
 * Compute-Efficient on GPUs" (ACM TACO):
 *   - forward convolution (FC), §2.1: every output pixel of channel c is the
 *     FH x FW inner product of its input patch with channel c's own filter
 *     (IC = OC = C), cross-correlation order (no filter flip);
 *   - backward data convolution (BDC), §5.1: the input gradient dX, i.e. the
 *     adjoint of the forward map in X (for stride 1: the forward map of dY
 *     with the filter turned by 180 degrees);
 *   - backward filter convolution (BFC), §5.1: the filter gradient
 *     dW[fh,fw,c] = sum over n,oh,ow of Xpad[n, oh*sh-ph+fh, ow*sw-pw+fw, c]
 *     * dY[n,oh,ow,c].
 * Padding is implicit zeros (§4.4) and symmetric; the output size is
 * OH = floor((H + 2*pad_h - FH) / stride_h) + 1 (likewise OW).
 *
 * Layouts (§2.3, unified channel-last layout), all dense and row-major:
 *   X, dX : N  x H  x W  x C
 *   Y, dY : N  x OH x OW x C
 *   W, dW : FH x FW x C
 *
 * Precision: operands X, W, dY are fp32, bf16, fp16 or fp8 (in_dtype, one
 * dtype for all operands of a call); every sum is accumulated in fp32 and
 * every output (Y, dX, dW) is fp32.  §4.1 argues that fp32 accumulation is
 * required for half-precision operands; §7 (low-bit data types) keeps the
 * same split for 8-bit operands: stored and multiplied in 8 bits, summed in
 * higher precision.  fp8 operands are the raw codes (one byte each) with no
 * scale factor; a per-tensor scale of a quantised tensor multiplies the
 * fp32 output.  Products of fp8 values are exact in fp32; the fp8 matrix
 * cores sum each group of products with an error of up to about 2^-12 of
 * the sum of their magnitudes (measured on MI355X), wider than fp32
 * rounding, while the vector kernels round every fp32 addition.
 *
 * Ownership and threading: every pointer is a device pointer owned by the
 * caller, who allocates all tensors and the workspace.  The library keeps no
 * state between calls except a per-process cache of device properties.
 * Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL is
 * the null stream); the library never synchronises.  Every call is
 * re-entrant.
 *
 * Errors: a bad argument is reported synchronously, before anything is
 * launched, and leaves every output untouched.  DWC_ERR_HIP means a launch
 * failed; faults inside a kernel surface at the caller's next
 * synchronisation.  dwc_last_error() returns a message for the calling
 * thread's last failed call.
 */
#ifndef DWC_H
#define DWC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DWC_VERSION 100 /* 1.0.0 */

typedef enum {
    DWC_F32 = 0,
    DWC_BF16 = 1,
    DWC_F16 = 2,
    DWC_FP8_E4M3 = 3, /* OCP fp8: 4 exponent bits (bias 7), 3 mantissa bits,
                         no infinities, S.1111.111 = NaN, max 448           */
    DWC_FP8_E5M2 = 4  /* OCP fp8: 5 exponent bits (bias 15), 2 mantissa
                         bits, IEEE-style infinities and NaNs, max 57344    */
} dwc_dtype;

typedef enum {
    DWC_ALGO_AUTO = 0,    /* library's choice                               */
    DWC_ALGO_VECTOR = 1,  /* register-window vector kernels (one channel per
                             lane, fp32 FMAs)                               */
    DWC_ALGO_DIRECT = 1,  /* the same value under its earlier name          */
    DWC_ALGO_MFMA = 2,    /* matrix-core kernels (stride 1, 16-byte aligned
                             tensors): the GEMV-to-GEMM packing of §4.2 on
                             CDNA4 MFMA.  bf16/fp16 operands: C a multiple
                             of 8, FW <= 32, output width <= 64 for the
                             forward and data gradient (the batch as the
                             second matrix dimension for widths up to 32
                             and tall filters; the 4x4x4 form with 4
                             images as the matrix rows for FW <= 17 on
                             narrow outputs), input width <= 64 and
                             FH <= 32 for the filter gradient; fp8: the
                             same with C a multiple of 16 for the forward
                             and data gradient (also the K=128 fp8 MFMA,
                             four filter or output rows per instruction,
                             §7); fp32: C a multiple of 16, FW <= 31 and
                             FH <= 64 for the forward and data gradient,
                             FH and FW <= 32 for the filter gradient
                             (4x4 outer products per channel, 16 channels
                             per instruction; output rows or images by
                             output columns, filter columns by rows).  AUTO takes them for the
                             problems where they beat the vector kernels
                             (16-bit and fp8: filters from 9x9 on, and
                             those outside the sweeps' square 3x3-7x7 set
                             with more than 5 rows or columns; fp32: from
                             10x10 on, by output width and batch).  Operands must be finite:
                             the packing multiplies staged elements by
                             structural zeros as well, so an inf or NaN
                             operand turns outputs that share an
                             instruction with it (forward, data gradient)
                             or its channel's filter gradient into NaN,
                             where the definition gives +-inf or a finite
                             value.  The vector and generic kernels follow
                             IEEE arithmetic on non-finite operands      */
    DWC_ALGO_GENERIC = 3, /* one output per lane; any filter size or stride */
    DWC_ALGO_HYBRID = 4   /* filter gradient of fp16 operands only (stride
                             1, square filter 3, 5, 7 or 9): the vector
                             sweep kernels with the hybrid accumulation of
                             §5.1 -- sub-units of at most 63 products per
                             tap summed in fp16 with packed FMAs, merged in
                             fp32.  Opt-in: faster, error ~1e-3 relative,
                             and an fp16 sub-unit sum above 65504 overflows */
} dwc_algo;

typedef enum {
    DWC_ACT_NONE = 0,   /* t                                   */
    DWC_ACT_RELU = 1,   /* max(t, 0)                           */
    DWC_ACT_RELU6 = 2,  /* min(max(t, 0), 6)                   */
    DWC_ACT_SILU = 3    /* t * sigmoid(t) = t / (1 + exp(-t))  */
} dwc_act;

typedef enum {
    DWC_OK = 0,
    DWC_ERR_BAD_PARAM = 1,   /* sizes, strides, pads or dtypes invalid         */
    DWC_ERR_UNSUPPORTED = 2, /* valid request the library does not implement   */
    DWC_ERR_MISALIGNED = 3,  /* pointer not aligned to its element size         */
    DWC_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required      */
    DWC_ERR_ALIAS = 5,       /* an output overlaps an input                     */
    DWC_ERR_HIP = 6          /* a HIP runtime call or kernel launch failed      */
} dwc_status;

/* One convolution problem.  n, h, w, c describe X (input of the forward
 * map).  All fields are plain integers so the struct has a fixed layout. */
typedef struct {
    int64_t n, h, w, c;         /* X: N x H x W x C, n >= 0, h, w, c >= 1   */
    int32_t fh, fw;             /* filter FH x FW, >= 1                     */
    int32_t stride_h, stride_w; /* >= 1                                     */
    int32_t pad_h, pad_w;       /* zero padding on both sides, >= 0         */
    int32_t in_dtype;           /* dwc_dtype of X, W, dY                    */
    int32_t out_dtype;          /* dwc_dtype of Y, dX, dW: must be DWC_F32  */
    int32_t algo;               /* dwc_algo                                 */
    int32_t wgrad_split;        /* filter gradient: number of slices of the
                                   N*OH accumulation axis (whole images for
                                   the half-precision packed kernels, at most
                                   N slices; runs of input rows for the fp32
                                   matrix-core kernel, at most N*H slices);
                                   0 = automatic                            */
} dwc_problem;

/* Version number (DWC_VERSION of the built library). */
int dwc_version(void);

/* Short text for a status code. */
const char* dwc_status_string(int status);

/* Message describing the calling thread's last failed call ("" if none). */
const char* dwc_last_error(void);

/* OH and OW of a problem (the formula above).  Host only, no GPU needed.
 * Returns DWC_ERR_BAD_PARAM if the filter does not fit the padded input. */
int dwc_output_dims(const dwc_problem* p, int64_t* oh, int64_t* ow);

/* Operation codes for dwc_check and dwc_plan_describe. */
#define DWC_OP_FWD 0
#define DWC_OP_BWD_DATA 1
#define DWC_OP_BWD_FILTER 2

/* Validate a problem for one operation without touching the GPU.  Returns
 * the status the compute call would return for argument errors. */
int dwc_check(const dwc_problem* p, int op);

/* Write a one-line description of the kernels and grid the library would
 * launch for `op` into buf (NUL-terminated, truncated to len).  Host only. */
int dwc_plan_describe(const dwc_problem* p, int op, char* buf, size_t len);

/* Forward convolution (FC, §2.1 / Fig. 1): y = DWC(x, w).
 *   x : N x H x W x C of in_dtype          (read)
 *   w : FH x FW x C of in_dtype            (read)
 *   y : N x OH x OW x C fp32               (overwritten)
 * Pointers must be aligned to their element size and y must not overlap x
 * or w.  n == 0 is a no-op. */
int dwc_fwd(const dwc_problem* p, const void* x, const void* w, void* y,
            void* stream);

/* Forward convolution with a fused prologue (Flash-DWC §5.2, "kernel
 * fusion": the batch normalisation and activation that usually precede a
 * DWC, applied to X as the forward reads it, so X' never goes to memory):
 *   X'[n,h,w,c] = act(x[n,h,w,c] * scale[c] + shift[c])    (fp32)
 *   y = DWC(X', w), with the zero padding around X' (padding stays 0).
 * Inference-form batch normalisation gives scale = gamma / sqrt(var + eps)
 * and shift = beta - mean * scale.
 *   x, w, y : as dwc_fwd
 *   scale, shift : C fp32 values each, device memory, 4-byte aligned (read;
 *                  may be NULL when n == 0)
 *   act : a dwc_act
 * Runs the register-window vector kernels (the pages fuse on their CUDA-core
 * kernels, for small filters): filter widths up to 9, stride 1 or 2,
 * any dtype; algo AUTO or DIRECT.  Otherwise DWC_ERR_UNSUPPORTED.  y must
 * not overlap x, w, scale or shift. */
int dwc_fwd_fused(const dwc_problem* p, const void* x, const float* scale,
                  const float* shift, int act, const void* w, void* y,
                  void* stream);

/* Backward data convolution (BDC, §5.1): dx = adjoint of the forward map
 * applied to dy.
 *   dy : N x OH x OW x C of in_dtype       (read)
 *   w  : FH x FW x C of in_dtype           (read)
 *   dx : N x H x W x C fp32                (overwritten; pixels no window
 *                                           reads get 0)
 * Any stride is accepted.  Stride 1 runs the rotated-filter forward kernels
 * the section describes.  Equal strides S >= 2 split dx into S*S output
 * phases, each a stride-1 correlation of dy with the sub-filter of taps
 * (fh, fw) = (f0h + S k, f0w + S l) (DWC_ALGO_DIRECT; sub-filters up to
 * 16 x 16).  Other strides run a gather kernel (DWC_ALGO_GENERIC). */
int dwc_bwd_data(const dwc_problem* p, const void* dy, const void* w,
                 void* dx, void* stream);

/* Bytes of workspace dwc_bwd_filter needs for this problem (may be 0). */
int dwc_bwd_filter_workspace_size(const dwc_problem* p, size_t* bytes);

/* Backward filter convolution (BFC, §5.1): dw = sum over the batch.
 *   x  : N x H x W x C of in_dtype         (read)
 *   dy : N x OH x OW x C of in_dtype       (read)
 *   dw : FH x FW x C fp32                  (overwritten, never accumulated)
 *   workspace : device memory of at least
 *               dwc_bwd_filter_workspace_size() bytes, 256-byte aligned,
 *               owned by the caller; its contents are scratch.
 * The N*OH accumulation axis is split into slices whose partial sums are
 * added in a fixed order (the split of §5.1, reduced deterministically
 * instead of with atomics), so results are bitwise reproducible for a given
 * problem, algo and wgrad_split.  The matrix-core kernels (DWC_ALGO_MFMA,
 * or AUTO where it applies) always write their slices' partial sums to the
 * workspace (one slice too) and need tensors 16-byte aligned; the fp32 one
 * slices runs of consecutive (image, input row) pairs, times the 56-column
 * groups of the output width.  n == 0 writes dw = 0. */
int dwc_bwd_filter(const dwc_problem* p, const void* x, const void* dy,
                   void* dw, void* workspace, size_t workspace_bytes,
                   void* stream);

/* Filter gradient that allocates nothing, for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same operation,
 * arguments and results as dwc_bwd_filter without the workspace: the slice
 * partials go to a fixed scratch array of DWC_NOALLOC_SCRATCH_BYTES inside
 * the library, one copy per device, held from the first call on that device
 * until the process ends.
 *   - The automatic split (wgrad_split == 0) is used when its partials fit
 *     the scratch, with the kernels and summation order of dwc_bwd_filter
 *     (bitwise the same result); otherwise the largest split that fits, then
 *     (AUTO) the vector kernels, whose single slice needs no scratch.  A
 *     split the caller sets is used as is.
 *   - A problem whose partials cannot fit returns DWC_ERR_WORKSPACE before
 *     anything is launched.
 *   - Nothing in the scratch needs to start at zero (every partial is
 *     written before it is read), and a call leaves its partials there.
 *   - Calls share their device's scratch: two calls that overlap in time on
 *     one device (different streams, or different threads) race on it and
 *     give wrong results.  Calls on one stream are ordered and safe. */
#define DWC_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int dwc_bwd_filter_noalloc(const dwc_problem* p, const void* x, const void* dy,
                           void* dw, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DWC_H */
