/*
 * hdq.h -- C ABI of libhdq, the MI355X (gfx950) library for the hot path of
 * 6Bit-Diffusion's dynamic mixed-precision quantization (DMPQ) of video
 * diffusion transformer linear layers.
 *
 * What the method computes, per linear layer and per denoising step
 * (sources: "6Bit-Diffusion" summary of arXiv:2603.18742 on vetunion.cn,
 * sections one, three and four; the gist.science explainer "6Bit-Diffusion:
 * Inference-Time Mixed-Precision Quantization for Video Diffusion Models",
 * sections 2 and 4):
 *   1. choose the activation precision from the relative difference of the
 *      module's input and output at the previous step (large: INT8, small:
 *      NVFP4), INT8 when there is no previous step, and full precision when
 *      the input's outlier ratio max|x| / mean|x| is too large;
 *   2. rotate the activations with a block Hadamard transform and quantize
 *      them in the same pass;
 *   3. run the quantized linear layer against weights prepared the same way.
 * hdq_select_precision is step 1, hdq_quantize is step 2 (and the offline
 * weight preparation), hdq_linear is steps 2 + 3.
 *
 * Conventions, for every entry point:
 *  - All tensors are row-major with the reduction dimension K contiguous:
 *    activations X [M, K], weights W [N, K], outputs Y [M, N] = X W^T.
 *  - bf16 tensors are raw 16-bit patterns (the upper half of an IEEE float).
 *  - Every pointer marked "device" is device memory the caller owns and keeps
 *    alive until the enqueued work has finished.  The library allocates no
 *    memory, never synchronises, and enqueues all work on `stream` (a
 *    hipStream_t passed as void*; NULL is the default stream).
 *  - Arguments are validated before anything is enqueued; on error nothing
 *    is enqueued and a negative HDQ_ERR_* code is returned.  A kernel fault
 *    surfaces at the caller's next synchronisation.
 *  - Calls are thread-safe; calls that share output or workspace buffers on
 *    overlapping streams race, as any stream work would.
 *  - Rotation: every aligned block of `had_block` consecutive elements along
 *    K is multiplied by H_b / sqrt(b), H_b the Sylvester Hadamard matrix, in
 *    float32 by the fast Walsh-Hadamard butterfly (strides 1, 2, 4, ... in
 *    that order) and one multiply by fl32(1/sqrt(b)).  Weights and
 *    activations are rotated alike, so (XQ)(WQ)^T = XW^T.  had_block 1
 *    rotates nothing.
 *  - Quantized codes use round-half-to-even.  Non-finite inputs are outside
 *    the quantizers' contract; hdq_select_precision routes them to BF16.
 */
#ifndef HDQ_H
#define HDQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define HDQ_OK 0
#define HDQ_ERR_INVALID (-1)     /* NULL pointer, bad enum or bad struct field  */
#define HDQ_ERR_SHAPE (-2)       /* size <= 0, K not a multiple of had_block or */
                                 /* of the format's block, had_block not a      */
                                 /* power of two in [1, 128], shapes disagree   */
#define HDQ_ERR_UNSUPPORTED (-3) /* precision/format/output-dtype combination   */
#define HDQ_ERR_HIP (-4)         /* a kernel launch failed                      */
#define HDQ_ERR_WORKSPACE (-5)   /* ws NULL or ws_bytes below what is required  */

/* ---- quantized formats (hdq_qtensor.fmt) ---- */
/* INT8, one fp32 scale per row: s = max|y| / 127, q = rne(y * (127 / max|y|)).
 * codes: int8 [rows, cols]; row_scale: fp32 [rows].  (The "INT8" activation
 * format of the summary's section one, per token.) */
#define HDQ_FMT_INT8_ROW 0
/* INT4, one fp32 scale per row (per output channel of a weight): same as
 * INT8 with 7 for 127.  codes: uint8 [rows, cols/2], element 2j in the low
 * nibble of byte j, two's complement; row_scale: fp32 [rows].  (The 4-bit
 * weights of the summary's W4A6 configuration, section four.) */
#define HDQ_FMT_INT4_ROW 1
/* NVFP4: FP4 E2M1 codes with one E4M3 scale per aligned 16 elements and one
 * fp32 tensor scale s_t = amax / 2688 (amax of the rotated tensor):
 * value = e2m1(code) * e4m3(blk_scale) * s_t.  codes: uint8 [rows, cols/2]
 * (even element in the low nibble); blk_scale: uint8 [rows, cols/16];
 * tensor_scale: fp32 [1].  (The "NVFP4" format of section one; the pages do
 * not define it, the encodings are those of the OCP MX v1.0 formats.) */
#define HDQ_FMT_NVFP4 2
/* NVFP4 bytes restricted so that every aligned pair of 16-blocks shares one
 * power-of-two scale (s_t = amax / 1536, scale = smallest power of two that
 * fits the pair): a valid NVFP4 tensor that is also MXFP4-shaped, so the
 * GEMM runs on gfx950's block-scaled FP4 matrix instructions. */
#define HDQ_FMT_NVFP4_MX 3
/* NVFP4 bytes restricted so that every aligned 16-block's scale is a power
 * of two (its own: s_t = amax / 1536, scale = smallest power of two that
 * fits the block): valid NVFP4, computed exactly on the block-scaled FP4
 * matrix instructions in two passes per 32 elements (one per 16-block half),
 * so at up to half the MX recipe's rate. */
#define HDQ_FMT_NVFP4_P2 4

/* ---- precisions (decisions) ---- */
#define HDQ_PREC_NVFP4 0
#define HDQ_PREC_INT8 1
#define HDQ_PREC_BF16 2 /* full precision: unrotated bf16 x bf16 GEMM */

/* ---- output dtypes of hdq_linear ---- */
#define HDQ_DTYPE_F32 0
#define HDQ_DTYPE_BF16 1
#define HDQ_DTYPE_I32 2 /* INT8 path only: the raw int32 accumulators */

/* ---- workspace queries (hdq_workspace_bytes op) ---- */
#define HDQ_OP_SELECT 0
#define HDQ_OP_QUANTIZE 1
#define HDQ_OP_LINEAR 2
#define HDQ_OP_SELECT_Q8 3
#define HDQ_OP_DQ_QUANTIZE 4
#define HDQ_OP_DQ_LINEAR 5

/* A quantized tensor.  The caller allocates every buffer (device memory)
 * and fills the pointers; hdq_quantize fills fmt, had_block, rows, cols. */
typedef struct hdq_qtensor {
    int32_t fmt;          /* HDQ_FMT_*                                       */
    int32_t had_block;    /* Hadamard block the rows were rotated with       */
    int64_t rows;         /* logical shape of the unquantized tensor         */
    int64_t cols;
    void *codes;          /* device, layout per format (see above)           */
    float *row_scale;     /* device, INT8/INT4 only (may be NULL otherwise)  */
    uint8_t *blk_scale;   /* device, NVFP4 formats only                      */
    float *tensor_scale;  /* device fp32[1], NVFP4 formats only              */
    void *dec;            /* NULL, or (NVFP4 formats) device bf16 [rows,
                           * cols]: each element's E2M1 value times its E4M3
                           * block scale, without the tensor scale -- exact in
                           * bf16.  hdq_quantize fills it when given; with
                           * plain NVFP4 on both operands of a GEMM the exact
                           * NVFP4 product reads its operands from it.
                           * Ignored for the INT formats.                    */
} hdq_qtensor;

/* A linear layer's weights in every form a precision may need.  Members a
 * call does not use may be NULL / zeroed. */
typedef struct hdq_weights {
    int64_t N;            /* output features                                 */
    int64_t K;            /* input features                                  */
    const void *w_bf16;   /* device bf16 [N, K], unrotated: HDQ_PREC_BF16    */
    hdq_qtensor w_int4;   /* HDQ_FMT_INT4_ROW [N, K]: HDQ_PREC_INT8          */
    hdq_qtensor w_fp4;    /* HDQ_FMT_NVFP4 or _MX [N, K]: HDQ_PREC_NVFP4     */
} hdq_weights;

/*
 * hdq_select_precision -- step 1 (summary section one: the previous step's
 * input/output difference picks INT8 or NVFP4; section three: the outlier
 * ratio max/mean forces full precision, and INT8 is used when there is no
 * previous-step difference; explainer sections 2 and 4).
 *
 *   prev_in, prev_out : device bf16 [prev_numel] each, the module's input and
 *                       output at the previous step; both NULL = no history.
 *   cur_in            : device bf16 [rows, cols], the current input.
 *   had_block         : 0, or the Hadamard block (power of two in [2, 128],
 *                       dividing cols) used to also report the rotated amax.
 *   delta_thresh, ratio_thresh : thresholds (e.g. 0.1 and 50).
 *   decision_dev      : device int32[1] <- HDQ_PREC_*.
 *   stats_dev         : device fp32[5] <- {delta, ratio, max|x|, mean|x|,
 *                       rotated amax (0 when had_block == 0)}.
 *   ws, ws_bytes      : device scratch, >= hdq_workspace_bytes(HDQ_OP_SELECT,
 *                       rows, cols, prev_numel, 0) bytes.
 * delta = sum|prev_out - prev_in| / sum|prev_in| (0 if both sums are 0, +inf
 * if only the denominator is, NaN without history); ratio = max|x| / mean|x|
 * over cur_in (0 for all zeros, NaN if cur_in holds a NaN or an infinity).
 * Decision: ratio not <= ratio_thresh -> BF16; else no history -> INT8; else
 * delta not < delta_thresh -> INT8; else NVFP4.  Sums are float32 partials
 * reduced in double in a fixed order, so results are deterministic.
 */
int hdq_select_precision(const void *prev_in, const void *prev_out, int64_t prev_numel,
                         const void *cur_in, int64_t rows, int64_t cols, int32_t had_block,
                         float delta_thresh, float ratio_thresh, int32_t *decision_dev,
                         float *stats_dev, void *ws, size_t ws_bytes, void *stream);

/*
 * hdq_delta_sums and hdq_select_precision_sums -- step 1 in two parts (same
 * sources as hdq_select_precision).  The difference statistic depends only
 * on the previous step's tensors, so it can be computed off the critical
 * path (e.g. on a second stream while earlier layers' GEMMs run), leaving
 * only the current input for the selection proper.
 *
 * hdq_delta_sums:
 *   prev_in, prev_out : device bf16 [numel] each (the module's previous-step
 *                       input and output).
 *   sums_dev          : device double[2] <- {sum|prev_out - prev_in|,
 *                       sum|prev_in|}.
 *   ws, ws_bytes      : device scratch, >= hdq_workspace_bytes(HDQ_OP_SELECT,
 *                       1, numel, numel, 0) bytes.
 * hdq_select_precision_sums:
 *   delta_sums_dev    : device double[2 * delta_parts]: delta_parts pairs
 *                       {sum|prev_out - prev_in|, sum|prev_in|} over parts
 *                       of the tensors, summed in order (delta_parts = 1:
 *                       the double[2] of hdq_delta_sums; more: the chunk
 *                       partials of hdq_linear_dispatch_delta).  Complete
 *                       before this call's kernels run (same stream or an
 *                       event), or NULL for no history.
 *   delta_parts       : >= 1 when delta_sums_dev is given (HDQ_ERR_SHAPE
 *                       otherwise); ignored for NULL.
 *   the other arguments are those of hdq_select_precision.
 * The two calls together write what hdq_select_precision writes for the
 * same tensors, bit for bit when numel == rows * cols (the statistics'
 * per-workgroup partials and their fixed-order reduction are the same); for
 * other sizes, equal up to the rounding of the double sums.
 */
int hdq_delta_sums(const void *prev_in, const void *prev_out, int64_t numel, double *sums_dev,
                   void *ws, size_t ws_bytes, void *stream);
int hdq_select_precision_sums(const double *delta_sums_dev, int64_t delta_parts, const void *cur_in,
                              int64_t rows, int64_t cols, int32_t had_block, float delta_thresh,
                              float ratio_thresh, int32_t *decision_dev, float *stats_dev,
                              void *ws, size_t ws_bytes, void *stream);

/*
 * hdq_select_quantize_int8 -- hdq_select_precision_sums fused with the INT8
 * per-token quantization of the same input (steps 1 and 2 for the INT8
 * path): x is read once, the INT8 codes are written whatever the decision
 * turns out to be (a caller then runs the INT8 GEMM gated on the decision).
 *   delta_sums_dev, delta_parts, cur_in, rows, cols, thresholds,
 *   decision_dev, stats_dev:
 *                 as for hdq_select_precision_sums; had_block must be > 0.
 *   xq8         : caller-allocated INT8_ROW buffers (codes int8 [rows, cols],
 *                 row_scale fp32 [rows]); fmt, had_block, rows, cols are
 *                 written.
 *   ws, ws_bytes: >= hdq_workspace_bytes(HDQ_OP_SELECT_Q8, rows, cols, 0, 0)
 *                 bytes (one partial per row).
 * The codes equal hdq_quantize's INT8_ROW codes bit for bit; the decision,
 * delta, max|x| and rotated amax equal hdq_select_precision_sums'; mean |x|
 * and the ratio agree up to the order of the double sum of |x| (per row
 * here, per chunk range there).  Rows over 16384 columns run the two passes
 * one after the other.
 */
int hdq_select_quantize_int8(const double *delta_sums_dev, int64_t delta_parts, const void *cur_in,
                             int64_t rows, int64_t cols, int32_t had_block, float delta_thresh,
                             float ratio_thresh, int32_t *decision_dev, float *stats_dev,
                             hdq_qtensor *xq8, void *ws, size_t ws_bytes, void *stream);

/*
 * hdq_select_quantize_int8_noalloc -- hdq_select_quantize_int8 with no
 * workspace argument, for callers that cannot allocate device memory: code
 * recorded under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments and results as hdq_select_quantize_int8
 * (bit for bit), without ws / ws_bytes.
 *   Scratch: the per-row statistics partials live in a static device array
 *   of HDQ_NOALLOC_SCRATCH_BYTES bytes, one per GPU the library runs on,
 *   held until the process ends.  Its address is looked up once per device
 *   (hipGetSymbolAddress, with that device current) on the first call there;
 *   the call allocates nothing.
 *   Limit: hdq_workspace_bytes(HDQ_OP_SELECT_Q8, rows, cols, 0, 0) (48 bytes
 *   per row, at least 48 KiB) must not exceed HDQ_NOALLOC_SCRATCH_BYTES, i.e.
 *   rows <= 43690; larger inputs return HDQ_ERR_TOO_LARGE before anything is
 *   enqueued.
 *   Sharing: every call on one GPU uses that GPU's one array and overwrites
 *   it (nothing in it needs to start at zero).  Calls that overlap on one GPU
 *   (other streams or threads, with the earlier call's kernels not yet done)
 *   race on it: order them on one stream or with events.
 */
#define HDQ_NOALLOC_SCRATCH_BYTES (2u << 20)
#define HDQ_ERR_TOO_LARGE (-6)   /* input beyond an allocation-free call's fixed scratch */
int hdq_select_quantize_int8_noalloc(const double *delta_sums_dev, int64_t delta_parts,
                                     const void *cur_in, int64_t rows, int64_t cols,
                                     int32_t had_block, float delta_thresh, float ratio_thresh,
                                     int32_t *decision_dev, float *stats_dev, hdq_qtensor *xq8,
                                     void *stream);

/*
 * hdq_quantize -- step 2: block-Hadamard rotation fused with quantization
 * (summary sections one and four).  Also prepares weights offline.
 *
 *   x           : device bf16 [rows, cols].
 *   had_block   : power of two in [2, 128] dividing cols.
 *   fmt         : HDQ_FMT_*; cols must be a multiple of 2 (INT4), 16 (NVFP4)
 *                 or 32 (NVFP4_MX).
 *   tensor_amax : NVFP4 formats: device fp32[1] holding the amax of the
 *                 rotated tensor (e.g. stats_dev + 4 from
 *                 hdq_select_precision), or NULL to compute it in a pre-pass
 *                 (then ws must hold hdq_workspace_bytes(HDQ_OP_QUANTIZE,
 *                 rows, cols, 0, fmt) bytes).  Ignored for INT formats.
 *   decision_dev: NULL, or device int32[1]: the kernels then do their work
 *                 only when it holds the precision that consumes `fmt`
 *                 (HDQ_PREC_INT8 for INT8_ROW, HDQ_PREC_NVFP4 for the NVFP4
 *                 formats; not allowed with INT4_ROW), so one enqueued call
 *                 serves a device-side decision without a host round trip.
 *   out         : host struct with caller-allocated device buffers sized for
 *                 the format; fmt, had_block, rows, cols are written.  For
 *                 the NVFP4 formats a non-NULL out->dec also receives the
 *                 codes' exact bf16 values (gated like the codes).
 * Rows whose max |rotated value| is below 2^-100 get zero codes and a zero
 * scale; an NVFP4 tensor whose amax is below 2^-100 gets s_t = 0 and zero
 * codes and scale bytes.
 */
int hdq_quantize(const void *x, int64_t rows, int64_t cols, int32_t had_block, int32_t fmt,
                 const float *tensor_amax, const int32_t *decision_dev, hdq_qtensor *out,
                 void *ws, size_t ws_bytes, void *stream);

/*
 * hdq_linear -- steps 2 + 3: Y[M, N] = quantized X[M, K] times the weights'
 * matching form (summary section one: NVFP4 or INT8 activations against
 * 4-bit weights; section three: full-precision fallback).
 *
 *   precision   : HDQ_PREC_* to run, or -1 to read it from decision_dev on
 *                 the device (every candidate kernel is enqueued and the ones
 *                 not selected exit at once; no host synchronisation).
 *   decision_dev: NULL, or device int32[1].  With precision -1 it selects
 *                 the path; with a fixed precision P the work is done only
 *                 when it holds P (so a caller can enqueue each path's
 *                 pieces, e.g. one quantization shared by several GEMMs).
 *   x           : device bf16 [M, K] (the unrotated activations).
 *   xq          : NULL, or already-quantized activations to use instead of
 *                 quantizing x (fixed precision INT8 or NVFP4 only; its format
 *                 must match the weights': INT8_ROW for INT8, the w_fp4
 *                 format for NVFP4).
 *   x_amax      : NVFP4 only: device fp32[1] rotated amax of x, or NULL to
 *                 compute it in a pre-pass.
 *   w           : weights; w->K == K and had_block of both quantized forms
 *                 must be equal; the needed forms must be present.
 *   y, y_dtype  : device output [M, N]: HDQ_DTYPE_F32 or _BF16 (all
 *                 precisions), _I32 (INT8 only: raw accumulators).
 *   ws, ws_bytes: device scratch >= hdq_workspace_bytes(HDQ_OP_LINEAR, M, K,
 *                 N, w_fp4.fmt) (0 when xq is given for INT8).
 * INT8:  acc = sum_k qx*qw (exact int32); y = fl32(fl32(acc * sx[m]) * sw[n]).
 * NVFP4: y = s_tx * s_tw * sum over 16-blocks of E_x E_w sum_k e2m1 e2m1,
 *        float32 accumulation.  Plain NVFP4 (HDQ_FMT_NVFP4) runs on bf16
 *        MFMAs: when xq->dec (and w->w_fp4.dec) are given the GEMM reads
 *        those exact bf16 values, otherwise it decodes the codes as it
 *        stages them -- the same products in the same order, so the same
 *        output bits.  Both copies given is the fastest form.
 * BF16:  y = x w^T with the unrotated bf16 operands, float32 accumulation.
 */
int hdq_linear(int32_t precision, const int32_t *decision_dev, const void *x,
               const hdq_qtensor *xq, const float *x_amax, int64_t M, int64_t K,
               const hdq_weights *w, void *y, int32_t y_dtype, void *ws, size_t ws_bytes,
               void *stream);

/*
 * hdq_linear_dispatch -- step 3 for a device-side decision in one launch:
 * the GEMM of the precision decision_dev names (summary section one: INT8
 * or NVFP4 activations against 4-bit weights; section three: full
 * precision), with every path's operands already prepared -- xq8 (INT8_ROW
 * from hdq_quantize or hdq_select_quantize_int8), xq4 (the weights' FP4
 * format), x (bf16, unrotated) and all three weight forms.  Results equal
 * hdq_linear(P, decision_dev, x or xq, ...) of the decided P, bit for bit.
 * One kernel reads the decision and runs that GEMM (K a multiple of 256 and
 * 2 * K * max(M, N) < 2^31); other shapes enqueue the three gated GEMMs.
 * Plain NVFP4 with xq4->dec (and w->w_fp4.dec) given reads the decoded
 * operands, as hdq_linear does.
 * y_dtype F32 or BF16.  No workspace.
 */
int hdq_linear_dispatch(const int32_t *decision_dev, const void *x, const hdq_qtensor *xq8,
                        const hdq_qtensor *xq4, int64_t M, int64_t K, const hdq_weights *w,
                        void *y, int32_t y_dtype, void *stream);

/*
 * hdq_linear_dispatch_delta -- hdq_linear_dispatch that also computes part
 * of step 1's difference statistic (summary section one: the previous
 * step's input/output difference) for later layer calls, inside the same
 * launch.  The difference depends only on earlier tensors, so it can run
 * beside this call's compute-bound GEMM: on workgroups appended after the
 * GEMM's persistent ones, which hold the CUs the GEMM leaves free and,
 * once its workgroups retire, every CU, claiming chunks from a queue until
 * none is left.  The launch ends when both are done, so the difference
 * never shares the GPU with the memory-bound passes of the next call.
 *
 * The tensors of one module are split into chunks of HDQ_DELTA_CHUNK
 * elements; chunk c's {sum|prev_out - prev_in|, sum|prev_in|} (float over
 * each 8 elements, double beyond, in a fixed order: the same whichever
 * workgroup runs it) go to partials[2c], partials[2c + 1].  A module's
 * chunks may be spread over several calls; once all of them have run,
 * partials is the delta_sums_dev input of hdq_select_quantize_int8 or
 * hdq_select_precision_sums with delta_parts = ceil(numel / HDQ_DELTA_CHUNK).
 *
 *   decision_dev ... stream: as for hdq_linear_dispatch, except that only
 *              the one-launch kernel's shapes are taken (K a multiple of 256,
 *              2 * K * max(M, N) < 2^31; HDQ_ERR_SHAPE otherwise).
 *   slices   : nslices (0..HDQ_DELTA_MAX_SLICES) chunk ranges:
 *     prev_in, prev_out : device bf16 [numel] each, 16-byte aligned.
 *     numel             : elements per tensor, a positive multiple of 8.
 *     chunk_begin/end   : the chunks [chunk_begin, chunk_end) to run here,
 *                         within [0, ceil(numel / HDQ_DELTA_CHUNK)].
 *     partials          : device double [2 * ceil(numel / HDQ_DELTA_CHUNK)].
 *   queue_dev: device uint32[2], zero before the first call; every call
 *              with work leaves it zero again.  Calls that may overlap
 *              (other streams) need their own queue.
 * With nslices = 0 (or empty ranges) this is hdq_linear_dispatch's GEMM
 * alone.  The GEMM output equals hdq_linear_dispatch's bit for bit.
 */
#define HDQ_DELTA_CHUNK 65536
#define HDQ_DELTA_MAX_SLICES 4
typedef struct hdq_delta_slice {
  const void *prev_in;
  const void *prev_out;
  int64_t numel;
  int64_t chunk_begin;
  int64_t chunk_end;
  double *partials;
} hdq_delta_slice;

int hdq_linear_dispatch_delta(const int32_t *decision_dev, const void *x, const hdq_qtensor *xq8,
                              const hdq_qtensor *xq4, int64_t M, int64_t K, const hdq_weights *w,
                              void *y, int32_t y_dtype, const hdq_delta_slice *slices,
                              int32_t nslices, uint32_t *queue_dev, void *stream);

/*
 * hdq_tdc_decide -- the temporal delta cache's skip rule (summary on
 * vetunion.cn, section two; gist.science explainer, section three), for n
 * modules at once, once per diffusion step.  A module whose output changed
 * little between its last two computed steps reuses its cached output at
 * the next step; an accumulator adds the predicted change of every skipped
 * step and forces a computation once it would pass its budget.
 *   sums_dev : device double [n][2]; for a module computed at this step
 *              with an earlier output, {sum|new - earlier|, sum|earlier|}
 *              (hdq_delta_sums(earlier, new, ...) writes exactly this);
 *              ignored otherwise.  With parts_offsets_dev: pairs of partial
 *              sums, module i's being pairs [off[i], off[i + 1]), summed in a
 *              fixed order (e.g. the chunk partials hdq_linear_dispatch_delta
 *              writes for the two outputs while later modules' GEMMs run).
 *   parts_offsets_dev: NULL, or device int64 [n + 1], nondecreasing.
 *   state_dev: device int32 [n]: 0 skipped at this step, 1 computed with no
 *              earlier output, 2 computed with one (sums valid).
 *   c_dev    : device float [n], in/out: relative change between the last
 *              two computed outputs (NaN: none yet); rewritten when state
 *              is 1 (NaN) or 2 (diff / base in double, then float; base 0
 *              gives 0 if diff is 0, else +inf).
 *   acc_dev  : device float [n], in/out: reset to 0 when state != 0.
 *   skip_dev : device int32 [n] <- 1 when the next step reuses the cache:
 *              c < tau_skip and fl32(acc + c) <= tau_acc (NaN is false);
 *              acc then becomes fl32(acc + c).
 * Errors: HDQ_ERR_INVALID for a null pointer, HDQ_ERR_SHAPE for n <= 0 or
 * n >= 2^31.  The state arrays are the caller's; one call per step.
 */
int hdq_tdc_decide(const double *sums_dev, const int64_t *parts_offsets_dev, const int32_t *state_dev,
                   float *c_dev, float *acc_dev, int32_t *skip_dev, int64_t n, float tau_skip,
                   float tau_acc, void *stream);

/* ---- DeltaQuant cube-delta quantization (a second workload) ---------------
 * DeltaQuant (paper-radar CVPR 2026 listing, abstract): video activations are
 * grouped in local 3D spatiotemporal cubes; each cube's mean token (the core)
 * is kept in FP8 and only each token's difference from it is quantized to 4
 * bits.  Here: the tokens of a frames x height x width grid are the rows of
 * x, frame outermost ((f * height + h) * width + w); cubes are cube_f x
 * cube_h x cube_w blocks, ragged at the far edges, numbered the same way over
 * the cube grid.  The core is the float32 sum of its tokens in that order
 * divided by their count; it is stored as E4M3 with one fp32 scale per cube,
 * max|core| / 448 (0 below 2^-100), each code the nearest E4M3 of |c| / s
 * (ties to even) with the sign in bit 7 and a zero magnitude stored as +0.  A
 * token's difference fl32(x - fl32(E * s)) is quantized to NVFP4 (fmt) with
 * no rotation (had_block 1) and the tensor scale of the largest |difference|.
 */
typedef struct hdq_dq_grid {
  int64_t frames, height, width;
  int32_t cube_f, cube_h, cube_w;
} hdq_dq_grid;

/* Cubes of the grid, -1 for a bad grid (a size <= 0, over 2^31 - 1 tokens, or
 * more than 256 tokens per cube). */
int64_t hdq_dq_cubes(const hdq_dq_grid *g);

/*
 * hdq_dq_quantize -- the activation side.
 *   x          : device bf16 [tokens, K], K a multiple of 32, at most 32768.
 *   fmt        : HDQ_FMT_NVFP4, _NVFP4_MX or _NVFP4_P2 for the differences.
 *   core_codes : device uint8 [cubes, K] (signed E4M3); core_scale: fp32 [cubes].
 *   core_bf16  : NULL, or device bf16 [cubes, K]: the signed E4M3 code values
 *                (exact), the bf16 core GEMM's operand (plain NVFP4, or K not
 *                a multiple of 128).
 *   delta      : fmt, had_block 1, rows = tokens, cols = K, with codes,
 *                blk_scale and tensor_scale set (written).
 *   ws, ws_bytes: device scratch >= hdq_workspace_bytes(HDQ_OP_DQ_QUANTIZE, ...)
 *                (256 bytes).
 * Non-finite values (not covered by the method's description): when any
 * difference is not finite -- which a NaN or infinite element of x, or a
 * cube sum or a difference beyond the float32 range, always causes -- the
 * tensor scale *delta->tensor_scale is written as NaN, a flag on the device;
 * the codes and scales are then unspecified (a linear layer on them yields
 * NaN outputs).  Finite inputs never raise it.
 */
int hdq_dq_quantize(const void *x, int64_t K, const hdq_dq_grid *g, int32_t fmt, uint8_t *core_codes,
                    float *core_scale, void *core_bf16, hdq_qtensor *delta, void *ws, size_t ws_bytes,
                    void *stream);

/* NVFP4 weights (any of the three formats, [N, K]) to device bf16 [N, K]
 * holding E2M1 x block scale per element (exact), the tensor scale left out:
 * the core GEMM's weight operand, made once per layer. */
int hdq_dq_decode_weights(const hdq_qtensor *w_fp4, void *w_dec, void *stream);

/* Scratch bytes hdq_dq_linear needs for this grid, reduction size K, N
 * outputs and difference format fmt: the core GEMM's fp32 [cubes, N], plus an
 * fp32 [tokens, N] only when the difference GEMM cannot add the core term in
 * its own epilogue (plain NVFP4, K not a multiple of 256, N not a multiple of
 * 4 or operands past 32-bit offsets).  0 on bad arguments. */
size_t hdq_dq_linear_workspace_bytes(const hdq_dq_grid *g, int64_t K, int64_t N, int32_t fmt);

/*
 * hdq_dq_linear -- y = (differences) x W^T + (the token's cube core) x W^T.
 *   delta       : from hdq_dq_quantize; w_fp4: the layer's NVFP4 weights in
 *                 the same format with had_block 1 (hdq_quantize with
 *                 had_block 1 rotates nothing), N a multiple of 4.
 *   core_codes, core_scale: from hdq_dq_quantize.
 *   core_bf16, w_dec: the bf16 core values (hdq_dq_quantize) and decoded
 *                 weights (hdq_dq_decode_weights); needed only when the
 *                 weights' block scales are not powers of two or K is not a
 *                 multiple of 128 (plain NVFP4), may be NULL otherwise.
 *   y, y_dtype  : device [tokens, N], HDQ_DTYPE_F32 or _BF16.
 *   ws, ws_bytes: >= hdq_dq_linear_workspace_bytes(g, K, N, delta->fmt)
 *                 (hdq_workspace_bytes(HDQ_OP_DQ_LINEAR, tokens, cubes, N, 0)
 *                 is an upper bound for every route).
 * The core GEMM yc = sum_k core * w (exact products, float32 accumulation)
 * runs on the FP8 x FP4 scaled matrix instructions straight from the core's
 * E4M3 codes and the weights' E2M1 codes with their power-of-two block
 * scales (MX and per-16 power-of-two formats, K % 128 == 0), else on the
 * bf16 ones from core_bf16 and w_dec; the difference GEMM is the NVFP4 GEMM
 * of the format, which adds the core term in its epilogue (MX and per-16
 * formats, K % 256 == 0) or writes fp32 into ws for a combine pass; either
 * way y = fl(yd + fl32(fl32(yc * s_core) * s_w)).  Errors: HDQ_ERR_INVALID
 * for a NULL pointer the route needs.
 */
int hdq_dq_linear(const hdq_dq_grid *g, const uint8_t *core_codes, const void *core_bf16, const float *core_scale,
                  const hdq_qtensor *delta, const hdq_qtensor *w_fp4, const void *w_dec, void *y, int32_t y_dtype,
                  void *ws, size_t ws_bytes, void *stream);

/* Scratch bytes an entry point needs.  op = HDQ_OP_SELECT: (M = rows,
 * K = cols, N = prev_numel); HDQ_OP_SELECT_Q8: (M = rows, K = cols);
 * HDQ_OP_QUANTIZE: (M = rows, K = cols, fmt);
 * HDQ_OP_LINEAR: (M, K, N, fmt = the weights' FP4 format, or -1 when only
 * INT8/BF16 will run); HDQ_OP_DQ_QUANTIZE: 256; HDQ_OP_DQ_LINEAR: (M = tokens,
 * K = cubes, N).  Returns 0 on bad arguments. */
size_t hdq_workspace_bytes(int32_t op, int64_t M, int64_t K, int64_t N, int32_t fmt);

/* Static text for a status code. */
const char *hdq_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int hdq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HDQ_H */
