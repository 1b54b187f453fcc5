/*
 * mdcn.h -- C ABI of the MI355X (gfx950) modulated deformable 2-D convolution
 * forward pass (DCNv2).
 *
 * The operator is the one described on the page "TensorRT 插件解析：
 * modulatedDeformConvPlugin 可变形卷积插件的原理、参数与使用指南" (trdm.cn),
 * cited here as [plugin guide §N]:
 *
 *   out[n][co][ho][wo] = bias[co]
 *     + sum over c' < C/group, i < kh, j < kw of
 *         weight[co][c'][i][j] * mask[n][q*K + k][ho][wo]
 *         * bilinear0(x[n][c], ho*stride_h - pad_h + i*dil_h + offset[n][q*2K + 2k][ho][wo],
 *                               wo*stride_w - pad_w + j*dil_w + offset[n][q*2K + 2k + 1][ho][wo])
 *   with K = kh*kw, k = i*kw + j, group index gi = co / (Co/group),
 *   c = gi*(C/group) + c', offset group q = c / (C/deformable_group),
 *   and bilinear0 the bilinear interpolation that reads 0 off the image.
 *   [plugin guide §二 (tensors), §三 (attributes), §五 steps 1-3 (algorithm)]
 *
 * Conventions shared by every call:
 *  - Tensors are dense, contiguous NCHW ("kLINEAR") and all share one dtype;
 *    the output has that dtype too [plugin guide §四].  BF16 is accepted in
 *    addition to the page's FP32 and FP16.  Interpolation and accumulation are
 *    done in fp32 whatever the storage dtype; the output is rounded to nearest
 *    even once, at the end.
 *  - Shapes are passed per call (dynamic shapes) as a dims[16] array of int64:
 *      dims[0..3]   x      [N, C, H, W]
 *      dims[4..7]   offset [N, 2*deformable_group*kh*kw, Ho, Wo]
 *      dims[8..11]  mask   [N, deformable_group*kh*kw, Ho, Wo]
 *      dims[12..15] weight [Co, C/group, kh, kw]
 *    The output is [N, Co, Ho, Wo]: batch from x, channels from weight,
 *    spatial size from offset [plugin guide §二, getOutputShapes].
 *  - Pointers to tensors are device pointers.  The caller owns every buffer
 *    (inputs, output, workspace); the library never allocates device memory
 *    in mdcn_forward and keeps no pointer after the call returns
 *    [TensorRT developer guide ch. 9 on plugin ownership].  Inputs are read
 *    only; the output and the workspace must not overlap any input or each
 *    other.  The workspace content is undefined after the call.
 *  - All device work is enqueued on the caller's stream (a hipStream_t passed
 *    as void*; NULL is the null stream); the call returns before the work
 *    completes and performs no device-wide synchronisation.
 *  - Every function returns a status code and never lets a C++ exception
 *    cross this boundary [page "如何编写高效的TensorRT插件来支持新型算子？",
 *    on clone() returning null instead of throwing].  Launch failures are
 *    caught with hipGetLastError after each launch (same page, on checking
 *    cudaGetLastError at the end of enqueue).
 *  - An op handle is immutable after creation: concurrent forwards with one
 *    handle on different streams, each with its own workspace, are safe.
 */
#ifndef MDCN_H
#define MDCN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MDCN_ABI_VERSION 2

typedef enum mdcn_status {
    MDCN_OK = 0,
    MDCN_E_NULL = 1,        /* a required pointer is NULL                            */
    MDCN_E_ATTR = 2,        /* stride/dilation <= 0, padding < 0, group or dg <= 0   */
    MDCN_E_SHAPE = 3,       /* the dims break a binding listed at mdcn_forward       */
    MDCN_E_DTYPE = 4,       /* dtype is not one of mdcn_dtype                        */
    MDCN_E_WORKSPACE = 5,   /* workspace NULL or smaller than mdcn_workspace_min_bytes */
    MDCN_E_LAUNCH = 6,      /* a kernel launch or HIP runtime call failed            */
    MDCN_E_DEVICE = 7,      /* the current device is not a gfx950 GPU                */
    MDCN_E_ALIAS = 8,       /* output or workspace overlaps another buffer           */
    MDCN_E_PATH = 9,        /* the requested path cannot run this problem            */
    MDCN_E_INTERNAL = 10,   /* unexpected host-side failure                          */
    MDCN_E_SYNC = 11        /* a workgroup's bounded wait for another's partial sums
                               gave up; that tile's outputs are NaN (see
                               mdcn_forward_check)                                    */
} mdcn_status;

typedef enum mdcn_dtype {
    MDCN_F32 = 0,
    MDCN_F16 = 1,
    MDCN_BF16 = 2
} mdcn_dtype;

/* How the forward is computed.  All paths compute the same function. */
typedef enum mdcn_path {
    MDCN_PATH_AUTO = 0,        /* choose per problem                                     */
    MDCN_PATH_GATHER_GEMM = 1, /* deformable im2col into the workspace, then a grouped
                                  MFMA GEMM with the bias fused in its epilogue
                                  [plugin guide §五 steps 1-3]                             */
    MDCN_PATH_DEPTHWISE = 2,   /* a direct gather-and-multiply-add kernel; requires
                                  C/group == 1 [plugin guide §三: group == #outputs is the
                                  depthwise case].  Where a plane of the input fits in LDS
                                  the sampling geometry (16 bytes per offset group, tap and
                                  output pixel) is first written to the workspace by a
                                  small kernel; otherwise no workspace is used            */
    MDCN_PATH_FUSED = 3,       /* the gather fused into the MFMA GEMM: the GEMM's B tiles
                                  are made in LDS from the bilinear samples, with no column
                                  buffer [plugin guide §五 steps 1-3 without the columns];
                                  requires C/group to be a multiple of 64 (fp16/bf16) or 32
                                  (fp32), C/deformable_group of 8 or 4, and a per-tile
                                  geometry table (32 bytes per offset group, tap and output
                                  column; 64 or 128 columns) that fits in LDS beside the
                                  operand stages                                          */
    MDCN_PATH_WINDOW = 4,      /* the gather fused into the MFMA GEMM with each output
                                  tile's input window staged in LDS: a tile is 256 output
                                  channels x 256 output pixels (16x16, 8x32, 32x8, or 256
                                  consecutive pixels of a narrow image); per chunk of 16
                                  input channels the input rectangle its samples can reach
                                  (anchors plus an offset margin) is copied to LDS once and
                                  the 9 taps read their bilinear corners from it; a sample
                                  with a corner on the image outside the rectangle is read
                                  from global memory.  One workgroup per CU walks a range
                                  of (tile, chunk) units; tiles split between two
                                  workgroups are summed through the workspace.  Requires
                                  fp16/bf16, a 3x3 kernel, C/group a multiple of 16 and
                                  each group inside one deformable group; the automatic
                                  choice when its tiles are at least 7/8 full
                                  [plugin guide §五 steps 1-3]                             */
    MDCN_PATH_DIRECT = 5,      /* the whole forward in one launch, one thread per output
                                  element reading x, offsets, masks and weights where they
                                  are; for problems of at most 2^20 multiply-adds (the
                                  automatic choice there), any problem when forced; no
                                  workspace [plugin guide §五 steps 1-3]                   */
    MDCN_PATH_GATHER_GEMM_FP8 = 6, /* REDUCED PRECISION, never chosen automatically: gather +
                                  GEMM with both contraction operands in OCP FP8 E4M3 and
                                  fp32 sums on the gfx950 FP8 matrix cores.  Each column
                                  value (the modulated bilinear sample) is saturated to
                                  +-448 and rounded to nearest even E4M3 (values below
                                  2^-9 vanish: inputs are used unscaled); each output
                                  channel's weight row is scaled by 2^e, e the largest
                                  integer with max|row| * 2^e <= 448, rounded the same way,
                                  and its sums are multiplied by 2^-e before the bias is
                                  added.  Any dtype and problem the gather + GEMM path
                                  takes; output in the input dtype.  Results differ from the
                                  other paths by the E4M3 rounding (about 2^-4 relative per
                                  operand) [plugin guide §五 steps 1-3 with 8-bit operands;
                                  the FP8 format is not on the pages]                       */
    MDCN_PATH_WINDOW_FP8 = 7   /* REDUCED PRECISION, never chosen automatically: the
                                  windowed kernel (MDCN_PATH_WINDOW, same tiles, window
                                  and eligibility) with the E4M3 rounding of
                                  MDCN_PATH_GATHER_GEMM_FP8: each modulated bilinear
                                  sample is computed in fp32 from the LDS window,
                                  saturated to +-448 and rounded to E4M3; the weight rows
                                  are scaled by 2^e and rounded likewise; the products are
                                  summed in fp32 on the FP8 matrix cores (four taps of 16
                                  channels per 64-deep instruction, the ninth tap of a
                                  16-channel chunk on the 16-deep one) and each output is
                                  2^-e * sum + bias, rounded once to the input dtype.  No
                                  column buffer.  Results agree with
                                  MDCN_PATH_GATHER_GEMM_FP8 up to the order of the fp32
                                  sums [plugin guide §五 steps 1-3 with 8-bit operands; the
                                  FP8 format is not on the pages]                          */
} mdcn_path;

typedef struct mdcn_op mdcn_op;

/* Create an op.  All five attributes are required [plugin guide §三]:
 * stride[2] (> 0), padding[2] (>= 0), dilation[2] (> 0), group (> 0),
 * deformable_group (> 0); index 0 is the height axis, 1 the width axis.
 * Values are stored as int64.  On success *out receives a handle the caller
 * must release with mdcn_destroy.  Errors: MDCN_E_NULL, MDCN_E_ATTR. */
mdcn_status mdcn_create(const int32_t stride[2], const int32_t padding[2],
                        const int32_t dilation[2], int32_t group, int32_t deformable_group,
                        mdcn_op **out);

/* As mdcn_create, with a fixed computation path instead of MDCN_PATH_AUTO. */
mdcn_status mdcn_create_with_path(const int32_t stride[2], const int32_t padding[2],
                                  const int32_t dilation[2], int32_t group,
                                  int32_t deformable_group, mdcn_path path, mdcn_op **out);

/* Release an op; NULL is ignored. */
void mdcn_destroy(mdcn_op *op);

/* Output dims [N, Co, Ho, Wo] = [x.d0, weight.d0, offset.d2, offset.d3]
 * [plugin guide §二].  Validates dims as mdcn_forward does.  Host only. */
mdcn_status mdcn_output_shape(const mdcn_op *op, const int64_t dims[16], int64_t out_dims[4]);

/* Workspace, in bytes, for a forward of this problem: *bytes is the size the
 * default plan uses (all images in as few chunks as a 256 MiB column buffer
 * allows), *min_bytes (may be NULL) the least mdcn_forward accepts (one image
 * at a time).  0 when the chosen path needs none.  The page sizes its
 * workspace as one image's im2col columns rounded up to 16 bytes
 * [plugin guide §五, workspace]; the sizing here is this library's own.
 * Host only.  Errors as mdcn_output_shape, plus MDCN_E_DTYPE, MDCN_E_PATH. */
mdcn_status mdcn_workspace_bytes(const mdcn_op *op, mdcn_dtype dtype, const int64_t dims[16],
                                 size_t *bytes, size_t *min_bytes);

/* The forward pass, enqueued on `stream`.
 *   x, offset, mask, weight: device pointers, shapes per dims (see above).
 *   bias: device pointer to bias_len values, or NULL for no bias (the
 *         page's 4-input form) [plugin guide §二: bias used iff present].
 *   out:  device pointer to N*Co*Ho*Wo values.
 *   workspace / workspace_bytes: device scratch of at least min_bytes from
 *         mdcn_workspace_bytes (may be NULL when that is 0).  More workspace
 *         lets more images go through at once.
 * Dims bindings checked (MDCN_E_SHAPE) [plugin guide §四 plus what keeps every
 * read in bounds]: every dim >= 0; C, H, W, Co, kh, kw > 0;
 * offset.d0 == mask.d0 == x.d0; mask.d2 == offset.d2, mask.d3 == offset.d3;
 * offset.d1 >= 2 and == 2*dg*kh*kw; mask.d1 == dg*kh*kw;
 * weight.d1*group == x.d1; weight.d0 % group == 0; x.d1 % dg == 0;
 * bias_len == weight.d0 when bias is given; per-image sizes below 2^31
 * elements and spatial extents below 2^24.
 * N == 0 or Ho*Wo == 0 is a valid empty call that does nothing.
 * Errors: every code above.  On error nothing has been enqueued, except for
 * MDCN_E_LAUNCH, where earlier launches of this call may have been. */
mdcn_status mdcn_forward(const mdcn_op *op, mdcn_dtype dtype, const int64_t dims[16],
                         const void *x, const void *offset, const void *mask,
                         const void *weight, const void *bias, int64_t bias_len, void *out,
                         void *workspace, size_t workspace_bytes, void *stream);

/* Completion check of the last mdcn_forward that used `workspace`: waits for
 * `stream` (host synchronisation), then reports MDCN_E_SYNC if a bounded
 * wait inside that forward gave up, MDCN_OK otherwise.  op, dtype, dims and
 * workspace_bytes must be those of that forward.  Only the windowed path
 * waits (a workgroup that finishes an output tile started by another one
 * polls a flag in the workspace, at most a fixed number of times, so that a
 * broken invariant can never hang the GPU); a forward whose wait gave up
 * writes NaN for the affected tile and sets a status word in the workspace,
 * cleared at the start of every forward.  The other paths always report
 * MDCN_OK.  The pages ask a plugin to check for errors after enqueueing work
 * [efficient-plugin page]; this is that check for the one error the kernels
 * themselves can detect.  Errors: MDCN_E_NULL, the shape/attribute codes of
 * mdcn_forward, MDCN_E_LAUNCH (a HIP call failed), MDCN_E_SYNC. */
mdcn_status mdcn_forward_check(const mdcn_op *op, mdcn_dtype dtype, const int64_t dims[16],
                               const void *workspace, size_t workspace_bytes, void *stream);

/* ---- forward without allocation ------------------------------------------ */

/* Bytes of the device array mdcn_forward_noalloc uses as its workspace (per
 * GPU, held from the library's first use on that GPU until the process
 * ends). */
#define MDCN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * forward pass of mdcn_forward, with the same arguments except the
 * workspace, which is a fixed array of MDCN_NOALLOC_SCRATCH_BYTES in this
 * library's device memory instead of a caller's buffer.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine) and
 * enqueues only kernel launches on `stream`.  Images go through in as few
 * launches as the array allows; a problem whose least workspace
 * (mdcn_workspace_bytes' min_bytes) exceeds it is rejected with
 * MDCN_E_WORKSPACE before anything is enqueued.  Every call on one GPU uses
 * that GPU's single array and leaves its contents behind (each forward
 * clears what must start at zero): calls that overlap in time on one GPU
 * (other streams, other threads) race and corrupt each other's results; the
 * caller must order them.  mdcn_forward_check does not apply (its workspace
 * is internal); a bounded wait that gave up still shows as NaN outputs.
 * Errors as mdcn_forward. */
mdcn_status mdcn_forward_noalloc(const mdcn_op *op, mdcn_dtype dtype, const int64_t dims[16],
                                 const void *x, const void *offset, const void *mask,
                                 const void *weight, const void *bias, int64_t bias_len,
                                 void *out, void *stream);

/* ---- backward ------------------------------------------------------------ */

/* Gradients of a scalar loss L through the forward, given grad_out = dL/dout
 * ([N][Co][Ho][Wo]): grad_x, grad_offset, grad_mask, grad_weight (the shapes
 * of x, offset, mask, weight) and, if grad_bias is not NULL, grad_bias
 * (bias_len == Co values).  The pages define only the forward
 * [plugin guide §五 steps 1-3]; these are the derivatives of that
 * definition, with the bilinear sample differentiated on the cell floor()
 * selects (corners off the image count as 0, so at an integer coordinate
 * this is the derivative from above) and zero derivatives for a sample
 * outside the open window (-1, H) x (-1, W) or with a non-finite coordinate.
 * Inputs and gradients in the dtype (fp32, fp16 or bf16), arithmetic and
 * accumulation in fp32, one rounding of each gradient.  Accumulations into
 * grad_x and grad_weight use atomic adds, so their last bits may differ from
 * run to run.  Buffers: device pointers, the outputs and the workspace (at least
 * mdcn_backward_workspace_bytes) must overlap no input and no other output
 * (MDCN_E_ALIAS).  Every output is written (zeros for an empty batch or
 * output grid).  Errors as mdcn_forward. */
mdcn_status mdcn_backward_workspace_bytes(const mdcn_op *op, mdcn_dtype dtype,
                                          const int64_t dims[16], size_t *bytes);
mdcn_status mdcn_backward(const mdcn_op *op, mdcn_dtype dtype, const int64_t dims[16],
                          const void *x, const void *offset, const void *mask,
                          const void *weight, const void *grad_out, void *grad_x,
                          void *grad_offset, void *grad_mask, void *grad_weight, void *grad_bias,
                          int64_t bias_len, void *workspace, size_t workspace_bytes,
                          void *stream);

/* ---- tracing: per-kernel device time, for profiling --------------------- */

typedef struct mdcn_trace mdcn_trace;

/* A trace records a pair of HIP events around every kernel that
 * mdcn_forward_traced launches, up to `capacity` launches (later launches
 * run untraced).  Creating it creates the events; no device memory is
 * allocated.  Errors: MDCN_E_NULL, MDCN_E_SHAPE (capacity <= 0), MDCN_E_LAUNCH. */
mdcn_status mdcn_trace_create(int32_t capacity, mdcn_trace **out);
void mdcn_trace_destroy(mdcn_trace *trace);
/* Forget recorded launches (the events are reused). */
mdcn_status mdcn_trace_reset(mdcn_trace *trace);

/* mdcn_forward, recording events around each kernel launch on `stream`. */
mdcn_status mdcn_forward_traced(const mdcn_op *op, mdcn_dtype dtype, const int64_t dims[16],
                                const void *x, const void *offset, const void *mask,
                                const void *weight, const void *bias, int64_t bias_len,
                                void *out, void *workspace, size_t workspace_bytes,
                                void *stream, mdcn_trace *trace);

/* mdcn_backward, recording events around each kernel launch on `stream`. */
mdcn_status mdcn_backward_traced(const mdcn_op *op, mdcn_dtype dtype, const int64_t dims[16],
                                 const void *x, const void *offset, const void *mask,
                                 const void *weight, const void *grad_out, void *grad_x,
                                 void *grad_offset, void *grad_mask, void *grad_weight,
                                 void *grad_bias, int64_t bias_len, void *workspace,
                                 size_t workspace_bytes, void *stream, mdcn_trace *trace);

/* Number of launches recorded so far. */
mdcn_status mdcn_trace_count(const mdcn_trace *trace, int32_t *count);

/* Kernel id and device milliseconds of recorded launch i; waits for that
 * launch's end event.  Errors: MDCN_E_NULL, MDCN_E_SHAPE (i out of range),
 * MDCN_E_LAUNCH. */
mdcn_status mdcn_trace_read(mdcn_trace *trace, int32_t i, int32_t *kernel_id, float *ms);

/* Name of a kernel id: "prep_nhwc" / "prep_blocks" (the weight repacked and
 * the first chunk of x to channels-last / 8-channel blocks, in one launch),
 * "to_nhwc" / "to_channel_blocks" (x of a later chunk), "deform_gather",
 * "gemm_bias", "fused_gather_gemm", "window_gather_gemm",
 * "depthwise_geometry", "depthwise_direct", "direct"; for the FP8 path
 * "prep_nhwc_fp8" (the weight rounded to E4M3 and the first chunk of x to
 * channels-last), "deform_gather_fp8", "gemm_fp8_bias"; for the windowed
 * FP8 path "prep_blocks_fp8" (the weight rounded to E4M3 in the windowed
 * kernel's chunk layout and the first chunk of x to 8-channel blocks) and
 * "window_gather_gemm_fp8"; for the backward
 * "bwd_zero", "bwd_bias", "bwd_weight_gemm", "bwd_col_gemm", "bwd_sample",
 * "bwd_to_nchw", "bwd_weight_out" (with "pack_weight", "to_nhwc" and
 * "deform_gather"); "pack_weight" (outside the backward) and
 * "pack_weight_steps" (standalone weight repacking) are not launched by the
 * forward.  "?" if unknown. */
const char *mdcn_kernel_name(int32_t kernel_id);

/* ---- misc ---------------------------------------------------------------- */

/* Static message for a status code. */
const char *mdcn_status_string(mdcn_status status);

/* MDCN_ABI_VERSION of the built library. */
int32_t mdcn_abi_version(void);

/* A one-line description of the plan mdcn_forward would use (path, chunk,
 * tile shapes, workspace split), written NUL-terminated into buf[len].
 * Host only.  Errors as mdcn_workspace_bytes, plus MDCN_E_NULL. */
mdcn_status mdcn_describe_plan(const mdcn_op *op, mdcn_dtype dtype, const int64_t dims[16],
                               size_t workspace_bytes, char *buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* MDCN_H */
