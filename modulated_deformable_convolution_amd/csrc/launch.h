// launch.h -- host launchers of the HIP kernels.  Each launcher checks
// hipGetLastError after its launch and returns it.
#pragma once

#include <hip/hip_runtime_api.h>

#include "plan.h"

namespace mdcn {

// Kernel ids reported by the tracing API.
enum KernelId : int32_t {
    K_PACK_WEIGHT = 0,
    K_TO_NHWC = 1,
    K_GATHER = 2,
    K_GEMM = 3,
    K_DEPTHWISE = 4,
    K_FUSED = 5,
    K_DW_GEOMETRY = 6,
    K_WINDOW = 7,
    K_PACK_WEIGHT_STEPS = 8,
    K_TO_BLOCKS = 9,
    K_PREP_NHWC = 10,
    K_PREP_BLOCKS = 11,
    K_DIRECT = 12,
    K_PREP_NHWC_FP8 = 13,
    K_GATHER_FP8 = 14,
    K_GEMM_FP8 = 15,
    K_BWD_ZERO = 16,
    K_BWD_BIAS = 17,
    K_BWD_WEIGHT_GEMM = 18,
    K_BWD_COL_GEMM = 19,
    K_BWD_SAMPLE = 20,
    K_BWD_WEIGHT_OUT = 21,
    K_BWD_TO_NCHW = 22,
    K_FUSED_ONE = 23,
    K_PREP_BLOCKS_FP8 = 24,
    K_WINDOW_FP8 = 25,
    K_COUNT = 26
};

// Compute units of the current device (cached per device; 1 if unknown).
int device_cu_count();

// weight [Co][Cg][kh][kw] -> packed [G][Mg][Kp], contraction index
// kk = k*Cg + c' (tap-major), zero for kk >= Kg.
hipError_t launch_pack_weight(const Problem &p, const Plan &plan, const void *weight,
                              void *wpack, hipStream_t stream);

// weight [Co][Cg][kh][kw] -> the window path's step-major planes:
// [G][S][2][Mg][8], S = (Cg/16)*K steps (chunk of 16 channels, tap), half h
// of the chunk's channels; requires Cg % 16 == 0.
// Also zeroes nflags flags at `flags` (the windowed kernel's; may be null).
hipError_t launch_pack_weight_steps(const Problem &p, const void *weight, void *wpack,
                                    uint32_t *flags, int nflags, hipStream_t stream);

// x [cnt][C][H][W] -> xb [cnt][C/8][H][W][8] (8-channel blocks; C % 8 == 0).
hipError_t launch_to_channel_blocks(const Problem &p, int64_t cnt, const void *x, void *xb,
                                    hipStream_t stream);

// The first chunk's set-up in one launch: x of cnt images to channels-last
// (window path: to 8-channel blocks) and the weight repacked for the plan's
// path (window path: step-major, with nflags flags cleared; FP8 path: each
// output channel's row scaled by 2^e and rounded to E4M3, wpack [Co][Kp]
// bytes tap-major, e the largest integer with max|w[co]| * 2^e <= 448, and
// wscale[co] = 2^-e).
hipError_t launch_prep(const Problem &p, const Plan &plan, int64_t cnt, const void *x, void *xt,
                       const void *weight, void *wpack, uint32_t *flags, int nflags,
                       float *wscale, hipStream_t stream);

// The whole forward of all N images, one thread per output element.
hipError_t launch_direct(const Problem &p, const void *x, const void *offset, const void *mask,
                         const void *weight, const void *bias, void *out, hipStream_t stream);

// x [cnt][C][H][W] -> xt [cnt][H][W][C] (channels innermost).
hipError_t launch_to_nhwc(const Problem &p, int64_t cnt, const void *x, void *xt,
                          hipStream_t stream);

// Deformable im2col of cnt images: col [G][cnt*P][Kp], row (n, pixel),
// column kk = k*Cg + c', value bilinear0(x[n][g*Cg + c'], sample) * mask
// (FP8 path: as an E4M3 byte, saturated to +-448).
hipError_t launch_gather(const Problem &p, const Plan &plan, int64_t cnt, const void *xt,
                         const void *offset, const void *mask, void *col, hipStream_t stream);

// The same columns in fp32 whatever the input dtype (the backward's).
hipError_t launch_gather_f32(const Problem &p, const Plan &plan, int64_t cnt, const void *xt,
                             const void *offset, const void *mask, float *col,
                             hipStream_t stream);
// The same fp32 columns of one image, transposed: colT[g][kk][pix] (rows kk
// in [Kg, Kp) zero).
hipError_t launch_gather_f32_t(const Problem &p, const Plan &plan, const void *xt,
                               const void *offset, const void *mask, float *colT,
                               hipStream_t stream);

// out[n][g*Mg + m][pix] = sum_kk wpack[g][m][kk] * col[g][n*P + pix][kk] (+ bias);
// The same fp32 GEMM (no bias) with explicit operand geometry: each row of A
// and of B holds kb bytes of K (a multiple of 128), consecutive rows sa / sb
// bytes apart, group g's blocks at A + g*ga and B + g*gb; out as above with
// cnt = 1 (rows g*Mg + m, p.P columns; the columns are B's p.P rows).
struct GemmStrides {
    uint32_t kb, sa, sb;
    uint64_t ga, gb;
};
hipError_t launch_gemm_strided(const Problem &p, const Plan &plan, const void *a, const void *b,
                               void *out, const GemmStrides &st, hipStream_t stream);
// The two fp32 GEMMs of the backward (launch_gemm_strided above, and this
// one: launch_gemm's fp32 GEMM with cnt = 1 and no bias) run on the bf16
// matrix cores with every operand split into three bf16 parts (six product
// terms; about 2^-22 relative error per product, fp32 sums).
hipError_t launch_gemm_f32_split(const Problem &p, const Plan &plan, const void *a,
                                 const void *b, void *out, hipStream_t stream);

// FP8 path: E4M3 operands and the sums times wscale[g*Mg + m] before the bias
// (wscale null otherwise).
hipError_t launch_gemm(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                       const void *col, const void *bias, const float *wscale, void *out,
                       hipStream_t stream);

// The fused forward of a whole chunk in one launch: the kernel below, whose
// workgroups first move x (cnt images, NCHW) to the NHWC copy `xt` and repack
// `weight` into `wpack` themselves, then meet at a bounded grid barrier.
// Opt-in (MDCN_FUSED_ONE=1; slower than the two launches on gfx950, see
// fused.hip).  hipErrorNotSupported (nothing enqueued) when it is not asked
// for or the problem or the stream does not allow it: more workgroups than
// CUs, a tile without the variant, or a capturing stream.
hipError_t launch_fused_one(const Problem &p, const Plan &plan, int64_t cnt, const void *x,
                            const void *weight, void *wpack, void *xt, const void *offset,
                            const void *mask, const void *bias, void *out, hipStream_t stream);

// Fused deformable gather + grouped GEMM + bias of cnt images:
// out[n][g*Mg + m][pix] from the packed weight, NHWC x, offset and mask.
hipError_t launch_fused(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                        const void *xt, const void *offset, const void *mask, const void *bias,
                        void *out, hipStream_t stream);

// The same, with each output tile's input window staged in LDS (fp16/bf16,
// 3x3 kernels; plan.win_tile, win_margin, win_lead), from the step-major
// weight (launch_pack_weight_steps) and x in 8-channel blocks
// (launch_to_channel_blocks).
// Scratch of the windowed kernel: `slots` partial-sum slots of 256 KiB (one
// per workgroup; a tile split between two workgroups passes its first
// chunks' sums through the first one's slot), one flag per slot and a status
// word after them (flags[slots]), all zeroed before the forward
// (launch_pack_weight_steps); `epoch` (> 0) is the value a launch publishes
// its flags with, distinct for every launch of one forward.  A hand-over
// wait that gives up sets the status word to kWindowGaveUp.
struct WindowScratch {
    float *partial;
    uint32_t *flags;
    int slots;
    int epoch;
};
// plan.path == Path::WindowFp8: the E4M3 variant, from the E4M3 chunk blocks
// and the row scales `wscale` (launch_prep with that plan); otherwise wscale
// is unused.
hipError_t launch_window(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                         const float *wscale, const void *xt, const void *offset,
                         const void *mask, const void *bias, void *out, const WindowScratch &ws,
                         hipStream_t stream);

// Depthwise sampling geometry of cnt images: for each (image, offset group,
// tap, pixel) a 16-byte record geo[((img*DG + q)*K + k)*P + pix] = {staged
// plane entry of the sample's top-left corner (0 for a sample with no corner
// on the image), ly, lx*m, (1-lx)*m}.
hipError_t launch_dw_geometry(const Problem &p, int64_t cnt, const void *offset,
                              const void *mask, void *geo, hipStream_t stream);

// Direct depthwise (C/group == 1) forward of cnt images (geo from
// launch_dw_geometry; null when the plan uses the plain kernel).
hipError_t launch_depthwise(const Problem &p, int64_t cnt, const void *x, const void *geo,
                            const void *offset, const void *mask, const void *weight,
                            const void *bias, void *out, hipStream_t stream);

// ---- backward (fp32 arithmetic; inputs and gradients in the dtype) ------
// Workspace of the backward, for one image at a time (offsets from the
// 256-byte aligned start): the packed weight [G][Mg][Kp] (tap-major, dtype),
// x of the image in NHWC (dtype), its grad_x accumulator in NHWC and the
// same in NCHW (fp32), its columns [G][P][Kp] (tap-major, as the forward's
// gather writes them, fp32), the column gradient in the same layout, and the
// weight-gradient accumulator [Co][Kp] (fp32).
// With mfma_col, also grad_out of the image transposed to [P][Co] and the
// packed weight transposed to [Kp][Co] (fp32), for the MFMA GEMM.
struct BackwardLayout {
    int64_t Kp;
    size_t wpack_off, xt_off, gxt_off, gxn_off, col_off, gcol_off, wacc_off, bytes;
    size_t goT_off, wT_off;
    bool mfma_col;
    int64_t wsplit;    // > 0: the weight gradient on the MFMA GEMM in wsplit pixel chunks
    bool binned;       // grad_x gathered from per-cell buckets (else atomic adds)
    size_t bins_off;   // the buckets' area; inside it:
    size_t cnt_off, start_off, bsum_off, entries_off;
};
// acc[t] += sum over s < S of part[s*n + t].
hipError_t launch_bwd_reduce_parts(const float *part, float *acc, int64_t n, int S,
                                   hipStream_t stream);
BackwardLayout backward_layout(const Problem &p);
hipError_t launch_bwd_fill_zero(float *ptr, int64_t n, hipStream_t stream);
// n zeros of the problem's dtype.
hipError_t launch_bwd_fill_zero_dtype(const Problem &p, void *ptr, int64_t n, hipStream_t stream);
// grad_bias[co] = sum over images and pixels of g[n][co][p].
hipError_t launch_bwd_bias(const Problem &p, const void *g, void *gb, hipStream_t stream);
// acc[g][m][kk] += sum_p g_n[g*Mg + m][p] * col[g][p][kk] (atomic adds).
hipError_t launch_bwd_weight_gemm(const Problem &p, const BackwardLayout &l, const void *g_n,
                                  const float *col, float *acc, hipStream_t stream);
// gcol[g][p][kk] = sum_m g_n[g*Mg + m][p] * wpack[g][m][kk] (kk tap-major).
hipError_t launch_bwd_col_gemm(const Problem &p, const BackwardLayout &l, const void *wpack,
                               const void *g_n, float *gcol, hipStream_t stream);
// grad_mask, grad_offset of image n (stored) and its grad_x in NHWC from
// gcol and the NHWC x.  l.binned: grad_x summed per input cell from buckets
// built at `bins` (the layout's bins area, whose counts must be zero; they
// are zero again afterwards), every element of gxt_n written; otherwise
// atomic adds into gxt_n, which the caller zeroes.
hipError_t launch_bwd_sample(const Problem &p, const BackwardLayout &l, const void *xt_n,
                             const void *off_n, const void *msk_n, const float *gcol,
                             float *gxt_n, void *goff_n, void *gmask_n, char *bins,
                             hipStream_t stream);
// dst[t] = src[t] rounded to the dtype (n values).
hipError_t launch_bwd_convert(const Problem &p, const float *src, void *dst, int64_t n,
                              hipStream_t stream);
// grad_weight[g*Mg + m][c'][k] = acc[g][m][k*Cg + c'].
hipError_t launch_bwd_weight_out(const Problem &p, const BackwardLayout &l, const float *acc,
                                 void *gw, hipStream_t stream);

}  // namespace mdcn
