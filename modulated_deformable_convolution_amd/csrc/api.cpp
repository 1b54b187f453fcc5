// api.cpp -- the extern "C" boundary declared in include/mdcn.h: validation,
// planning, launches on the caller's stream, tracing.  No C++ exception
// crosses the boundary.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <vector>

#include "entry.h"
#include "launch.h"
#include "mdcn.h"
#include "plan.h"

struct mdcn_op {
    mdcn::Attrs attrs;
};

struct mdcn_trace {
    int32_t capacity = 0;
    int32_t count = 0;
    std::vector<hipEvent_t> start, stop;
    std::vector<int32_t> kernel;
};

namespace {

using mdcn::Path;
using mdcn::Plan;
using mdcn::Problem;

mdcn_status device_ok()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        return MDCN_E_DEVICE;
    static std::mutex mu;
    static std::map<int, bool> known;
    std::lock_guard<std::mutex> lock(mu);
    auto it = known.find(dev);
    if (it == known.end()) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return MDCN_E_DEVICE;
        const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        it = known.emplace(dev, ok).first;
    }
    return it->second ? MDCN_OK : MDCN_E_DEVICE;
}

struct Range {
    const char *lo, *hi;
};

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

Range range_of(const void *p, size_t bytes)
{
    const char *c = static_cast<const char *>(p);
    return Range{c, c + bytes};
}

// Records an event pair around each launch while the trace has room.
struct Recorder {
    hipStream_t stream;
    mdcn_trace *trace;

    template <class F>
    hipError_t run(int32_t kernel, F &&launch)
    {
        int32_t slot = -1;
        if (trace && trace->count < trace->capacity) {
            slot = trace->count++;
            trace->kernel[slot] = kernel;
            hipError_t e = hipEventRecord(trace->start[slot], stream);
            if (e != hipSuccess)
                return e;
        }
        hipError_t e = launch();
        if (e == hipErrorNotSupported && slot >= 0 && slot == trace->count - 1)
            trace->count--;                  // nothing was enqueued: no record
        if (e != hipSuccess)
            return e;
        if (slot >= 0)
            e = hipEventRecord(trace->stop[slot], stream);
        return e;
    }
};

mdcn_status forward_impl(const mdcn_op *op, mdcn_dtype dtype, const int64_t dims[16],
                         const void *x, const void *offset, const void *mask,
                         const void *weight, const void *bias, int64_t bias_len, void *out,
                         void *workspace, size_t workspace_bytes, void *stream_ptr,
                         mdcn_trace *trace)
{
    if (!op || !dims)
        return MDCN_E_NULL;
    Problem p;
    mdcn_status st = mdcn::derive_problem(op->attrs, dtype, dims, &p);
    if (st != MDCN_OK)
        return st;
    if (bias && bias_len != p.Co)       // bias_0 == weight_0 [plugin guide §四]
        return MDCN_E_SHAPE;
    Plan plan;
    st = mdcn::make_plan(op->attrs, p, workspace_bytes, true, &plan);
    if (st != MDCN_OK)
        return st;
    if (p.N == 0 || p.P == 0)
        return MDCN_OK;                 // nothing to compute
    if (!x || !offset || !mask || !weight || !out)
        return MDCN_E_NULL;
    if (plan.ws_bytes > 0) {
        if (!workspace)
            return MDCN_E_WORKSPACE;
        st = mdcn::make_plan(op->attrs, p, workspace_bytes, false, &plan);
        if (st != MDCN_OK)
            return st;
    }

    const size_t e = p.elem;
    const Range inputs[] = {
        range_of(x, size_t(p.N * p.C * p.H * p.W) * e),
        range_of(offset, size_t(p.N * 2 * p.DG * p.K * p.P) * e),
        range_of(mask, size_t(p.N * p.DG * p.K * p.P) * e),
        range_of(weight, size_t(p.Co * p.Cg * p.K) * e),
        range_of(bias, bias ? size_t(p.Co) * e : 0),
    };
    const Range out_r = range_of(out, size_t(p.N * p.Co * p.P) * e);
    // the workspace layout starts at the caller's pointer aligned up to kAlign
    char *ws = nullptr;
    if (plan.ws_bytes > 0) {
        const uintptr_t raw = reinterpret_cast<uintptr_t>(workspace);
        ws = reinterpret_cast<char *>((raw + mdcn::kAlign - 1) / mdcn::kAlign * mdcn::kAlign);
    }
    const Range ws_r = range_of(ws, plan.ws_bytes);
    for (const Range &in : inputs) {
        if (overlap(out_r, in) || overlap(ws_r, in))
            return MDCN_E_ALIAS;
    }
    if (overlap(out_r, ws_r))
        return MDCN_E_ALIAS;

    st = device_ok();
    if (st != MDCN_OK)
        return st;

    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    Recorder rec{stream, trace};
    hipError_t err = hipSuccess;

    const size_t x_img = size_t(p.C * p.H * p.W) * e;
    const size_t off_img = size_t(2 * p.DG * p.K * p.P) * e;
    const size_t msk_img = size_t(p.DG * p.K * p.P) * e;
    const size_t out_img = size_t(p.Co * p.P) * e;
    if (plan.path == Path::Direct) {
        err = rec.run(mdcn::K_DIRECT, [&] {
            return mdcn::launch_direct(p, x, offset, mask, weight, bias, out, stream);
        });
        return err == hipSuccess ? MDCN_OK : MDCN_E_LAUNCH;
    }
    if (plan.path == Path::Depthwise) {
        for (int64_t n0 = 0; n0 < p.N; n0 += plan.chunk) {
            const int64_t cnt = std::min<int64_t>(plan.chunk, p.N - n0);
            const char *xc = static_cast<const char *>(x) + size_t(n0) * x_img;
            const char *oc = static_cast<const char *>(offset) + size_t(n0) * off_img;
            const char *mc = static_cast<const char *>(mask) + size_t(n0) * msk_img;
            char *outc = static_cast<char *>(out) + size_t(n0) * out_img;
            if (plan.ws_bytes > 0) {
                err = rec.run(mdcn::K_DW_GEOMETRY, [&] {
                    return mdcn::launch_dw_geometry(p, cnt, oc, mc, ws, stream);
                });
                if (err != hipSuccess)
                    return MDCN_E_LAUNCH;
            }
            err = rec.run(mdcn::K_DEPTHWISE, [&] {
                return mdcn::launch_depthwise(p, cnt, xc, plan.ws_bytes > 0 ? ws : nullptr, oc,
                                              mc, weight, bias, outc, stream);
            });
            if (err != hipSuccess)
                return MDCN_E_LAUNCH;
        }
        return MDCN_OK;
    }

    void *wpack = ws + plan.wpack_off;
    void *xt = ws + plan.xt_off;
    void *col = ws + plan.col_off;
    uint32_t *win_flags = reinterpret_cast<uint32_t *>(ws + plan.flag_off);
    const bool fp8 = plan.path == Path::GatherGemmFp8;
    const bool windowed = plan.path == Path::Window || plan.path == Path::WindowFp8;
    float *wscale = (fp8 || plan.path == Path::WindowFp8)
                        ? reinterpret_cast<float *>(ws + plan.wpack_off + plan.wscale_off)
                        : nullptr;
    // The weight is repacked (and the window path's flags cleared) in the
    // same launch as the first chunk's x layout change.
    if (plan.path == Path::Fused && plan.chunk >= p.N) {
        // the whole batch in one launch when the grid fits the device
        err = rec.run(mdcn::K_FUSED_ONE, [&] {
            return mdcn::launch_fused_one(p, plan, p.N, x, weight, wpack, xt, offset, mask, bias,
                                          out, stream);
        });
        if (err == hipSuccess)
            return MDCN_OK;
        if (err != hipErrorNotSupported)
            return MDCN_E_LAUNCH;
    }
    for (int64_t n0 = 0; n0 < p.N; n0 += plan.chunk) {
        const int64_t cnt = std::min<int64_t>(plan.chunk, p.N - n0);
        const char *xc = static_cast<const char *>(x) + size_t(n0) * x_img;
        const char *oc = static_cast<const char *>(offset) + size_t(n0) * off_img;
        const char *mc = static_cast<const char *>(mask) + size_t(n0) * msk_img;
        char *outc = static_cast<char *>(out) + size_t(n0) * out_img;
        if (n0 == 0)
            err = rec.run(plan.path == Path::Window          ? mdcn::K_PREP_BLOCKS
                          : plan.path == Path::WindowFp8     ? mdcn::K_PREP_BLOCKS_FP8
                          : plan.path == Path::GatherGemmFp8 ? mdcn::K_PREP_NHWC_FP8
                                                             : mdcn::K_PREP_NHWC,
                          [&] {
                              return mdcn::launch_prep(p, plan, cnt, xc, xt, weight, wpack,
                                                       win_flags,
                                                       windowed ? int(plan.win_slots) + 1 : 0,
                                                       wscale, stream);
                          });
        else if (windowed)
            err = rec.run(mdcn::K_TO_BLOCKS,
                          [&] { return mdcn::launch_to_channel_blocks(p, cnt, xc, xt, stream); });
        else
            err = rec.run(mdcn::K_TO_NHWC,
                          [&] { return mdcn::launch_to_nhwc(p, cnt, xc, xt, stream); });
        if (err != hipSuccess)
            return MDCN_E_LAUNCH;
        if (plan.path == Path::Fused) {
            err = rec.run(mdcn::K_FUSED, [&] {
                return mdcn::launch_fused(p, plan, cnt, wpack, xt, oc, mc, bias, outc, stream);
            });
            if (err != hipSuccess)
                return MDCN_E_LAUNCH;
            continue;
        }
        if (windowed) {
            // every launch of this forward publishes partial sums with its own
            // flag value (the flags were zeroed with the weight packing)
            const mdcn::WindowScratch scratch{reinterpret_cast<float *>(ws + plan.part_off),
                                              win_flags, int(plan.win_slots),
                                              int(n0 / plan.chunk) + 1};
            err = rec.run(plan.path == Path::WindowFp8 ? mdcn::K_WINDOW_FP8 : mdcn::K_WINDOW,
                          [&] {
                              return mdcn::launch_window(p, plan, cnt, wpack, wscale, xt, oc, mc,
                                                         bias, outc, scratch, stream);
                          });
            if (err != hipSuccess)
                return MDCN_E_LAUNCH;
            continue;
        }
        err = rec.run(fp8 ? mdcn::K_GATHER_FP8 : mdcn::K_GATHER, [&] {
            return mdcn::launch_gather(p, plan, cnt, xt, oc, mc, col, stream);
        });
        if (err != hipSuccess)
            return MDCN_E_LAUNCH;
        err = rec.run(fp8 ? mdcn::K_GEMM_FP8 : mdcn::K_GEMM, [&] {
            return mdcn::launch_gemm(p, plan, cnt, wpack, col, bias, wscale, outc, stream);
        });
        if (err != hipSuccess)
            return MDCN_E_LAUNCH;
    }
    return MDCN_OK;
}

mdcn_status backward_impl(const mdcn_op *op, mdcn_dtype dtype, const int64_t dims[16],
                          const void *x, const void *offset, const void *mask,
                          const void *weight, const void *grad_out, void *grad_x,
                          void *grad_offset, void *grad_mask, void *grad_weight, void *grad_bias,
                          int64_t bias_len, void *workspace, size_t workspace_bytes,
                          void *stream_ptr, mdcn_trace *trace)
{
    if (!op || !dims)
        return MDCN_E_NULL;
    Problem p;
    mdcn_status st = mdcn::derive_problem(op->attrs, dtype, dims, &p);
    if (st != MDCN_OK)
        return st;
    if (grad_bias && bias_len != p.Co)
        return MDCN_E_SHAPE;
    if (!x || !offset || !mask || !weight || !grad_out || !grad_x || !grad_offset ||
        !grad_mask || !grad_weight)
        return MDCN_E_NULL;
    const mdcn::BackwardLayout l = mdcn::backward_layout(p);
    if (!workspace || workspace_bytes < l.bytes + mdcn::kAlign)
        return MDCN_E_WORKSPACE;
    const size_t x_n = size_t(p.C * p.H * p.W), off_n = size_t(2 * p.DG * p.K * p.P);
    const size_t msk_n = size_t(p.DG * p.K * p.P), out_n = size_t(p.Co * p.P);
    const size_t w_n = size_t(p.Co * p.Cg * p.K);
    const size_t e = p.elem;
    const Range inputs[] = {
        range_of(x, size_t(p.N) * x_n * e), range_of(offset, size_t(p.N) * off_n * e),
        range_of(mask, size_t(p.N) * msk_n * e), range_of(weight, w_n * e),
        range_of(grad_out, size_t(p.N) * out_n * e)};
    const uintptr_t raw = reinterpret_cast<uintptr_t>(workspace);
    char *ws = reinterpret_cast<char *>((raw + mdcn::kAlign - 1) / mdcn::kAlign * mdcn::kAlign);
    const Range outputs[] = {
        range_of(grad_x, size_t(p.N) * x_n * e), range_of(grad_offset, size_t(p.N) * off_n * e),
        range_of(grad_mask, size_t(p.N) * msk_n * e), range_of(grad_weight, w_n * e),
        range_of(grad_bias, grad_bias ? size_t(p.Co) * e : 0), range_of(ws, l.bytes)};
    for (size_t i = 0; i < sizeof(outputs) / sizeof(outputs[0]); ++i) {
        for (const Range &in : inputs)
            if (overlap(outputs[i], in))
                return MDCN_E_ALIAS;
        for (size_t j = i + 1; j < sizeof(outputs) / sizeof(outputs[0]); ++j)
            if (overlap(outputs[i], outputs[j]))
                return MDCN_E_ALIAS;
    }
    st = device_ok();
    if (st != MDCN_OK)
        return st;

    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    Recorder rec{stream, trace};
    char *gx = static_cast<char *>(grad_x);
    float *wacc = reinterpret_cast<float *>(ws + l.wacc_off);
    char *wpack = ws + l.wpack_off;
    char *xt = ws + l.xt_off;
    float *gxt = reinterpret_cast<float *>(ws + l.gxt_off);
    float *gxn = reinterpret_cast<float *>(ws + l.gxn_off);
    float *col = reinterpret_cast<float *>(ws + l.col_off);
    float *gcol = reinterpret_cast<float *>(ws + l.gcol_off);
    const bool empty = p.N == 0 || p.P == 0;
    // the weight accumulator takes atomic adds; an empty batch or output grid
    // leaves every gradient zero
    char *bins = ws + l.bins_off;
    hipError_t err = rec.run(mdcn::K_BWD_ZERO, [&] {
        hipError_t e = mdcn::launch_bwd_fill_zero(wacc, p.Co * l.Kp, stream);
        if (e == hipSuccess && empty)
            e = mdcn::launch_bwd_fill_zero_dtype(p, gx, int64_t(p.N) * int64_t(x_n), stream);
        // the bucket counts (each image's fill pass leaves them zero again)
        if (e == hipSuccess && l.binned && !empty)
            e = mdcn::launch_bwd_fill_zero(reinterpret_cast<float *>(bins + l.cnt_off),
                                           p.DG * p.H * p.W, stream);
        return e;
    });
    if (err != hipSuccess)
        return MDCN_E_LAUNCH;
    if (grad_bias) {
        err = (p.N == 0 || p.P == 0)
                  ? mdcn::launch_bwd_fill_zero_dtype(p, grad_bias, p.Co, stream)
                  : rec.run(mdcn::K_BWD_BIAS, [&] {
                        return mdcn::launch_bwd_bias(p, grad_out, grad_bias, stream);
                    });
        if (err != hipSuccess)
            return MDCN_E_LAUNCH;
    }
    Plan gp{};
    gp.path = Path::GatherGemm;     // the forward's im2col and weight packing, fp32
    gp.Kp = l.Kp;
    if (!empty) {
        err = rec.run(mdcn::K_PACK_WEIGHT, [&] {
            return mdcn::launch_pack_weight(p, gp, weight, wpack, stream);
        });
        if (err != hipSuccess)
            return MDCN_E_LAUNCH;
    }
    // grad_x of one image in NHWC -> NCHW: the NHWC transpose with the roles
    // of channels and positions exchanged ([H*W][C] read as C' = H*W channels
    // of C positions)
    Problem pt = p;
    pt.C = p.H * p.W;
    pt.H = p.C;
    pt.W = 1;
    pt.dtype = MDCN_F32;               // the accumulator is fp32 whatever the dtype
    pt.elem = 4;
    // the column gradient on the MFMA GEMM: C(p, kk) = sum_m goT[p][m] * wT[kk][m],
    // i.e. the GEMM kernel with rows = pixels, columns = kk, contraction = Co
    float *goT = reinterpret_cast<float *>(ws + l.goT_off);
    float *wT = reinterpret_cast<float *>(ws + l.wT_off);
    Problem pq = p;                    // the GEMM's view
    pq.G = 1; pq.Mg = p.P; pq.Co = p.P; pq.P = l.Kp;
    Plan qp{};
    qp.path = Path::GatherGemm;
    qp.Kp = p.Co;
    qp.gemm_tile = mdcn::gemm_tile_for(pq, 1);
    Problem pgo = p;                   // grad_out [Co][P] -> [P][Co]: the NHWC transpose
    pgo.C = p.Co; pgo.H = p.Ho; pgo.W = p.Wo;
    Problem pwt = p;                   // packed weight [Co][Kp] -> [Kp][Co]
    pwt.C = p.Co; pwt.H = l.Kp; pwt.W = 1;
    if (l.mfma_col && !empty) {
        err = rec.run(mdcn::K_BWD_TO_NCHW, [&] {
            return mdcn::launch_to_nhwc(pwt, 1, wpack, wT, stream);
        });
        if (err != hipSuccess)
            return MDCN_E_LAUNCH;
    }
    for (int64_t n = 0; n < p.N && !empty; ++n) {
        const char *xn = static_cast<const char *>(x) + size_t(n) * x_n * e;
        const char *on = static_cast<const char *>(offset) + size_t(n) * off_n * e;
        const char *mn = static_cast<const char *>(mask) + size_t(n) * msk_n * e;
        const char *gn = static_cast<const char *>(grad_out) + size_t(n) * out_n * e;
        err = rec.run(mdcn::K_TO_NHWC, [&] { return mdcn::launch_to_nhwc(p, 1, xn, xt, stream); });
        // the columns: [P][Kp], or (weight gradient in pixel chunks) straight
        // into the column-gradient buffer transposed, [Kp][P]
        if (err == hipSuccess)
            err = rec.run(mdcn::K_GATHER, [&] {
                return l.wsplit == 0
                           ? mdcn::launch_gather_f32(p, gp, 1, xt, on, mn, col, stream)
                           : mdcn::launch_gather_f32_t(p, gp, xt, on, mn, gcol, stream);
            });
        if (err == hipSuccess)
            err = rec.run(mdcn::K_BWD_WEIGHT_GEMM, [&] {
                if (l.wsplit == 0)
                    return mdcn::launch_bwd_weight_gemm(p, l, gn, col, wacc, stream);
                // per pixel chunk s of the transposed columns [Kp][P] (in the
                // column-gradient buffer): part[s][m][kk] = sum over the
                // chunk's pixels of g[m][p] * colT[kk][p], then summed into wacc
                const int64_t S = l.wsplit, pc = p.P / S;
                hipError_t r = hipSuccess;
                Problem pw = p;
                pw.G = S; pw.Mg = p.Co; pw.Co = S * p.Co; pw.P = l.Kp;
                Plan wp{};
                wp.path = Path::GatherGemm;
                wp.Kp = pc;
                wp.gemm_tile = mdcn::gemm_tile_for(pw, 1);
                const mdcn::GemmStrides st{uint32_t(pc * 4), uint32_t(p.P * 4), uint32_t(p.P * 4),
                                           uint64_t(pc) * 4, uint64_t(pc) * 4};
                r = mdcn::launch_gemm_strided(pw, wp, gn, gcol, col, st, stream);
                return r != hipSuccess ? r
                                       : mdcn::launch_bwd_reduce_parts(col, wacc, p.Co * l.Kp,
                                                                       int(S), stream);
            });
        if (err == hipSuccess)
            err = rec.run(mdcn::K_BWD_COL_GEMM, [&] {
                if (!l.mfma_col)
                    return mdcn::launch_bwd_col_gemm(p, l, wpack, gn, gcol, stream);
                hipError_t r = mdcn::launch_to_nhwc(pgo, 1, gn, goT, stream);
                return r != hipSuccess
                           ? r
                           : mdcn::launch_gemm_f32_split(pq, qp, goT, wT, gcol, stream);
            });
        if (err == hipSuccess && !l.binned)
            err = rec.run(mdcn::K_BWD_ZERO, [&] {
                return mdcn::launch_bwd_fill_zero(gxt, int64_t(x_n), stream);
            });
        if (err == hipSuccess)
            err = rec.run(mdcn::K_BWD_SAMPLE, [&] {
                return mdcn::launch_bwd_sample(
                    p, l, xt, on, mn, gcol, gxt,
                    static_cast<char *>(grad_offset) + size_t(n) * off_n * e,
                    static_cast<char *>(grad_mask) + size_t(n) * msk_n * e, bins, stream);
            });
        if (err == hipSuccess)
            err = rec.run(mdcn::K_BWD_TO_NCHW, [&] {
                // fp32: straight into grad_x; fp16/bf16: through fp32 NCHW, then rounded
                if (p.dtype == MDCN_F32)
                    return mdcn::launch_to_nhwc(pt, 1, gxt, gx + size_t(n) * x_n * e, stream);
                hipError_t r = mdcn::launch_to_nhwc(pt, 1, gxt, gxn, stream);
                return r != hipSuccess ? r
                                       : mdcn::launch_bwd_convert(p, gxn, gx + size_t(n) * x_n * e,
                                                                  int64_t(x_n), stream);
            });
        if (err != hipSuccess)
            return MDCN_E_LAUNCH;
    }
    err = rec.run(mdcn::K_BWD_WEIGHT_OUT, [&] {
        return mdcn::launch_bwd_weight_out(p, l, wacc, grad_weight, stream);
    });
    return err == hipSuccess ? MDCN_OK : MDCN_E_LAUNCH;
}

mdcn_status create_impl(const int32_t stride[2], const int32_t padding[2],
                        const int32_t dilation[2], int32_t group, int32_t dgroup,
                        mdcn_path path, mdcn_op **out)
{
    if (!out)
        return MDCN_E_NULL;
    *out = nullptr;
    mdcn_status st = mdcn::check_attrs(stride, padding, dilation, group, dgroup);
    if (st != MDCN_OK)
        return st;
    if (path != MDCN_PATH_AUTO && path != MDCN_PATH_GATHER_GEMM &&
        path != MDCN_PATH_DEPTHWISE && path != MDCN_PATH_FUSED && path != MDCN_PATH_WINDOW &&
        path != MDCN_PATH_DIRECT && path != MDCN_PATH_GATHER_GEMM_FP8 &&
        path != MDCN_PATH_WINDOW_FP8)
        return MDCN_E_PATH;
    mdcn_op *op = new (std::nothrow) mdcn_op;
    if (!op)
        return MDCN_E_INTERNAL;
    op->attrs = mdcn::Attrs{stride[0], stride[1], padding[0], padding[1], dilation[0],
                            dilation[1], group, dgroup, path};
    *out = op;
    return MDCN_OK;
}

}  // namespace

namespace mdcn {

mdcn_status forward_with_workspace(const mdcn_op *op, mdcn_dtype dtype, const int64_t dims[16],
                                   const void *x, const void *offset, const void *mask,
                                   const void *weight, const void *bias, int64_t bias_len,
                                   void *out, void *workspace, size_t workspace_bytes,
                                   void *stream)
{
    return forward_impl(op, dtype, dims, x, offset, mask, weight, bias, bias_len, out, workspace,
                        workspace_bytes, stream, nullptr);
}

}  // namespace mdcn


extern "C" {

mdcn_status mdcn_create(const int32_t stride[2], const int32_t padding[2],
                        const int32_t dilation[2], int32_t group, int32_t deformable_group,
                        mdcn_op **out)
{
    try {
        return create_impl(stride, padding, dilation, group, deformable_group, MDCN_PATH_AUTO, out);
    } catch (...) {
        return MDCN_E_INTERNAL;
    }
}

mdcn_status mdcn_create_with_path(const int32_t stride[2], const int32_t padding[2],
                                  const int32_t dilation[2], int32_t group,
                                  int32_t deformable_group, mdcn_path path, mdcn_op **out)
{
    try {
        return create_impl(stride, padding, dilation, group, deformable_group, path, out);
    } catch (...) {
        return MDCN_E_INTERNAL;
    }
}

void mdcn_destroy(mdcn_op *op) { delete op; }

mdcn_status mdcn_output_shape(const mdcn_op *op, const int64_t dims[16], int64_t out_dims[4])
{
    try {
        if (!op || !dims || !out_dims)
            return MDCN_E_NULL;
        Problem p;
        mdcn_status st = mdcn::derive_problem(op->attrs, MDCN_F32, dims, &p);
        if (st != MDCN_OK)
            return st;
        out_dims[0] = p.N;
        out_dims[1] = p.Co;
        out_dims[2] = p.Ho;
        out_dims[3] = p.Wo;
        return MDCN_OK;
    } catch (...) {
        return MDCN_E_INTERNAL;
    }
}

mdcn_status mdcn_workspace_bytes(const mdcn_op *op, mdcn_dtype dtype, const int64_t dims[16],
                                 size_t *bytes, size_t *min_bytes)
{
    try {
        if (!op || !dims || !bytes)
            return MDCN_E_NULL;
        Problem p;
        mdcn_status st = mdcn::derive_problem(op->attrs, dtype, dims, &p);
        if (st != MDCN_OK)
            return st;
        Plan plan;
        st = mdcn::make_plan(op->attrs, p, 0, true, &plan);
        if (st != MDCN_OK)
            return st;
        const bool none = plan.ws_bytes == 0 || p.N == 0 || p.P == 0;
        *bytes = none ? 0 : mdcn::workspace_request(plan);
        if (min_bytes)
            *min_bytes = none ? 0 : mdcn::min_workspace(p, plan);
        return MDCN_OK;
    } catch (...) {
        return MDCN_E_INTERNAL;
    }
}

mdcn_status mdcn_forward_check(const mdcn_op *op, mdcn_dtype dtype, const int64_t dims[16],
                               const void *workspace, size_t workspace_bytes, void *stream_ptr)
{
    try {
        if (!op || !dims)
            return MDCN_E_NULL;
        Problem p;
        mdcn_status st = mdcn::derive_problem(op->attrs, dtype, dims, &p);
        if (st != MDCN_OK)
            return st;
        Plan plan;
        st = mdcn::make_plan(op->attrs, p, workspace_bytes, true, &plan);
        if (st != MDCN_OK)
            return st;
        hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
        if ((plan.path != Path::Window && plan.path != Path::WindowFp8) || p.N == 0 ||
            p.P == 0 || plan.ws_bytes == 0)
            return hipStreamSynchronize(stream) == hipSuccess ? MDCN_OK : MDCN_E_LAUNCH;
        if (!workspace)
            return MDCN_E_NULL;
        st = mdcn::make_plan(op->attrs, p, workspace_bytes, false, &plan);
        if (st != MDCN_OK)
            return st;
        const uintptr_t raw = reinterpret_cast<uintptr_t>(workspace);
        const char *ws =
            reinterpret_cast<const char *>((raw + mdcn::kAlign - 1) / mdcn::kAlign * mdcn::kAlign);
        const uint32_t *status =
            reinterpret_cast<const uint32_t *>(ws + plan.flag_off) + plan.win_slots;
        uint32_t word = 0;
        if (hipMemcpyAsync(&word, status, sizeof(word), hipMemcpyDeviceToHost, stream) !=
                hipSuccess ||
            hipStreamSynchronize(stream) != hipSuccess)
            return MDCN_E_LAUNCH;
        return word == mdcn::kWindowGaveUp ? MDCN_E_SYNC : MDCN_OK;
    } catch (...) {
        return MDCN_E_INTERNAL;
    }
}

mdcn_status mdcn_forward(const mdcn_op *op, mdcn_dtype dtype, const int64_t dims[16],
                         const void *x, const void *offset, const void *mask,
                         const void *weight, const void *bias, int64_t bias_len, void *out,
                         void *workspace, size_t workspace_bytes, void *stream)
{
    try {
        return forward_impl(op, dtype, dims, x, offset, mask, weight, bias, bias_len, out,
                            workspace, workspace_bytes, stream, nullptr);
    } catch (...) {
        return MDCN_E_INTERNAL;
    }
}

mdcn_status mdcn_forward_traced(const mdcn_op *op, mdcn_dtype dtype, const int64_t dims[16],
                                const void *x, const void *offset, const void *mask,
                                const void *weight, const void *bias, int64_t bias_len,
                                void *out, void *workspace, size_t workspace_bytes,
                                void *stream, mdcn_trace *trace)
{
    try {
        if (!trace)
            return MDCN_E_NULL;
        return forward_impl(op, dtype, dims, x, offset, mask, weight, bias, bias_len, out,
                            workspace, workspace_bytes, stream, trace);
    } catch (...) {
        return MDCN_E_INTERNAL;
    }
}

mdcn_status mdcn_backward_workspace_bytes(const mdcn_op *op, mdcn_dtype dtype,
                                          const int64_t dims[16], size_t *bytes)
{
    try {
        if (!op || !dims || !bytes)
            return MDCN_E_NULL;
        Problem p;
        mdcn_status st = mdcn::derive_problem(op->attrs, dtype, dims, &p);
        if (st != MDCN_OK)
            return st;
        *bytes = mdcn::backward_layout(p).bytes + mdcn::kAlign;
        return MDCN_OK;
    } catch (...) {
        return MDCN_E_INTERNAL;
    }
}

mdcn_status mdcn_backward(const mdcn_op *op, mdcn_dtype dtype, const int64_t dims[16],
                          const void *x, const void *offset, const void *mask,
                          const void *weight, const void *grad_out, void *grad_x,
                          void *grad_offset, void *grad_mask, void *grad_weight, void *grad_bias,
                          int64_t bias_len, void *workspace, size_t workspace_bytes, void *stream)
{
    try {
        return backward_impl(op, dtype, dims, x, offset, mask, weight, grad_out, grad_x,
                             grad_offset, grad_mask, grad_weight, grad_bias, bias_len, workspace,
                             workspace_bytes, stream, nullptr);
    } catch (...) {
        return MDCN_E_INTERNAL;
    }
}

mdcn_status mdcn_backward_traced(const mdcn_op *op, mdcn_dtype dtype, const int64_t dims[16],
                                 const void *x, const void *offset, const void *mask,
                                 const void *weight, const void *grad_out, void *grad_x,
                                 void *grad_offset, void *grad_mask, void *grad_weight,
                                 void *grad_bias, int64_t bias_len, void *workspace,
                                 size_t workspace_bytes, void *stream, mdcn_trace *trace)
{
    try {
        if (!trace)
            return MDCN_E_NULL;
        return backward_impl(op, dtype, dims, x, offset, mask, weight, grad_out, grad_x,
                             grad_offset, grad_mask, grad_weight, grad_bias, bias_len, workspace,
                             workspace_bytes, stream, trace);
    } catch (...) {
        return MDCN_E_INTERNAL;
    }
}

mdcn_status mdcn_trace_create(int32_t capacity, mdcn_trace **out)
{
    try {
        if (!out)
            return MDCN_E_NULL;
        *out = nullptr;
        if (capacity <= 0)
            return MDCN_E_SHAPE;
        mdcn_trace *t = new (std::nothrow) mdcn_trace;
        if (!t)
            return MDCN_E_INTERNAL;
        t->capacity = capacity;
        t->start.assign(size_t(capacity), nullptr);
        t->stop.assign(size_t(capacity), nullptr);
        t->kernel.assign(size_t(capacity), -1);
        for (int32_t i = 0; i < capacity; ++i) {
            if (hipEventCreate(&t->start[i]) != hipSuccess ||
                hipEventCreate(&t->stop[i]) != hipSuccess) {
                mdcn_trace_destroy(t);
                return MDCN_E_LAUNCH;
            }
        }
        *out = t;
        return MDCN_OK;
    } catch (...) {
        return MDCN_E_INTERNAL;
    }
}

void mdcn_trace_destroy(mdcn_trace *trace)
{
    if (!trace)
        return;
    for (hipEvent_t ev : trace->start)
        if (ev)
            (void)hipEventDestroy(ev);
    for (hipEvent_t ev : trace->stop)
        if (ev)
            (void)hipEventDestroy(ev);
    delete trace;
}

mdcn_status mdcn_trace_reset(mdcn_trace *trace)
{
    if (!trace)
        return MDCN_E_NULL;
    trace->count = 0;
    return MDCN_OK;
}

mdcn_status mdcn_trace_count(const mdcn_trace *trace, int32_t *count)
{
    if (!trace || !count)
        return MDCN_E_NULL;
    *count = trace->count;
    return MDCN_OK;
}

mdcn_status mdcn_trace_read(mdcn_trace *trace, int32_t i, int32_t *kernel_id, float *ms)
{
    if (!trace || !kernel_id || !ms)
        return MDCN_E_NULL;
    if (i < 0 || i >= trace->count)
        return MDCN_E_SHAPE;
    if (hipEventSynchronize(trace->stop[i]) != hipSuccess)
        return MDCN_E_LAUNCH;
    float t = 0.0f;
    if (hipEventElapsedTime(&t, trace->start[i], trace->stop[i]) != hipSuccess)
        return MDCN_E_LAUNCH;
    *kernel_id = trace->kernel[i];
    *ms = t;
    return MDCN_OK;
}

const char *mdcn_kernel_name(int32_t kernel_id)
{
    switch (kernel_id) {
    case mdcn::K_PACK_WEIGHT: return "pack_weight";
    case mdcn::K_TO_NHWC: return "to_nhwc";
    case mdcn::K_GATHER: return "deform_gather";
    case mdcn::K_GEMM: return "gemm_bias";
    case mdcn::K_DEPTHWISE: return "depthwise_direct";
    case mdcn::K_FUSED: return "fused_gather_gemm";
    case mdcn::K_DW_GEOMETRY: return "depthwise_geometry";
    case mdcn::K_WINDOW: return "window_gather_gemm";
    case mdcn::K_PACK_WEIGHT_STEPS: return "pack_weight_steps";
    case mdcn::K_TO_BLOCKS: return "to_channel_blocks";
    case mdcn::K_PREP_NHWC: return "prep_nhwc";
    case mdcn::K_PREP_BLOCKS: return "prep_blocks";
    case mdcn::K_DIRECT: return "direct";
    case mdcn::K_PREP_NHWC_FP8: return "prep_nhwc_fp8";
    case mdcn::K_GATHER_FP8: return "deform_gather_fp8";
    case mdcn::K_GEMM_FP8: return "gemm_fp8_bias";
    case mdcn::K_BWD_ZERO: return "bwd_zero";
    case mdcn::K_BWD_BIAS: return "bwd_bias";
    case mdcn::K_BWD_WEIGHT_GEMM: return "bwd_weight_gemm";
    case mdcn::K_BWD_COL_GEMM: return "bwd_col_gemm";
    case mdcn::K_BWD_SAMPLE: return "bwd_sample";
    case mdcn::K_BWD_WEIGHT_OUT: return "bwd_weight_out";
    case mdcn::K_BWD_TO_NCHW: return "bwd_to_nchw";
    case mdcn::K_FUSED_ONE: return "fused_one_launch";
    case mdcn::K_PREP_BLOCKS_FP8: return "prep_blocks_fp8";
    case mdcn::K_WINDOW_FP8: return "window_gather_gemm_fp8";
    }
    return "?";
}

const char *mdcn_status_string(mdcn_status status)
{
    switch (status) {
    case MDCN_OK: return "ok";
    case MDCN_E_NULL: return "a required pointer is NULL";
    case MDCN_E_ATTR: return "invalid attribute (stride/dilation must be > 0, padding >= 0, "
                             "group and deformable_group > 0)";
    case MDCN_E_SHAPE: return "tensor dims violate the operator's shape bindings or limits";
    case MDCN_E_DTYPE: return "unsupported dtype";
    case MDCN_E_WORKSPACE: return "workspace missing or too small";
    case MDCN_E_LAUNCH: return "HIP launch or runtime call failed";
    case MDCN_E_DEVICE: return "the current device is not a gfx950 GPU";
    case MDCN_E_ALIAS: return "output or workspace overlaps another buffer";
    case MDCN_E_PATH: return "the requested computation path cannot run this problem";
    case MDCN_E_INTERNAL: return "internal error";
    case MDCN_E_SYNC: return "a bounded wait for partial sums gave up; the affected outputs are NaN";
    }
    return "unknown status";
}

int32_t mdcn_abi_version(void) { return MDCN_ABI_VERSION; }

mdcn_status mdcn_describe_plan(const mdcn_op *op, mdcn_dtype dtype, const int64_t dims[16],
                               size_t workspace_bytes, char *buf, size_t len)
{
    try {
        if (!op || !dims || !buf || len == 0)
            return MDCN_E_NULL;
        Problem p;
        mdcn_status st = mdcn::derive_problem(op->attrs, dtype, dims, &p);
        if (st != MDCN_OK)
            return st;
        Plan plan;
        st = mdcn::make_plan(op->attrs, p, workspace_bytes, workspace_bytes == 0, &plan);
        if (st != MDCN_OK)
            return st;
        if (plan.path == Path::Direct)
            std::snprintf(buf, len, "path=direct N=%lld Co=%lld P=%lld Cg=%lld K=%lld ws=0",
                          (long long)p.N, (long long)p.Co, (long long)p.P, (long long)p.Cg,
                          (long long)p.K);
        else if (plan.path == Path::Depthwise)
            std::snprintf(buf, len,
                          "path=depthwise_direct N=%lld C=%lld Co=%lld P=%lld chunk=%lld entry=%d "
                          "ws=%zu (geometry/img=%zu)",
                          (long long)p.N, (long long)p.C, (long long)p.Co, (long long)p.P,
                          (long long)plan.chunk, mdcn::dw_default_entry(p), plan.ws_bytes,
                          plan.geo_bytes_per_image);
        else if (plan.path == Path::Fused)
            std::snprintf(buf, len,
                          "path=fused chunk=%lld Kg=%lld Kp=%lld G=%lld Mg=%lld P=%lld tile=%d "
                          "ws=%zu (wpack=%zu xt/img=%zu)",
                          (long long)plan.chunk, (long long)p.Kg, (long long)plan.Kp,
                          (long long)p.G, (long long)p.Mg, (long long)p.P,
                          int(plan.fused_tile), plan.ws_bytes, plan.wpack_bytes,
                          plan.xt_bytes_per_image);
        else if (plan.path == Path::Window || plan.path == Path::WindowFp8)
            std::snprintf(buf, len,
                          "path=%s chunk=%lld Kg=%lld Kp=%lld G=%lld Mg=%lld P=%lld tile=%d "
                          "margin=%lld slots=%lld ws=%zu (wpack=%zu xt/img=%zu)",
                          plan.path == Path::WindowFp8 ? "window_fp8" : "window",
                          (long long)plan.chunk, (long long)p.Kg, (long long)plan.Kp,
                          (long long)p.G, (long long)p.Mg, (long long)p.P, int(plan.win_tile),
                          (long long)plan.win_margin, (long long)plan.win_slots, plan.ws_bytes,
                          plan.wpack_bytes, plan.xt_bytes_per_image);
        else
            std::snprintf(buf, len,
                          "path=%s chunk=%lld Kg=%lld Kp=%lld G=%lld Mg=%lld P=%lld "
                          "ws=%zu (wpack=%zu xt/img=%zu col/img=%zu)",
                          plan.path == Path::GatherGemmFp8 ? "gather_gemm_fp8" : "gather_gemm",
                          (long long)plan.chunk, (long long)p.Kg, (long long)plan.Kp,
                          (long long)p.G, (long long)p.Mg, (long long)p.P, plan.ws_bytes,
                          plan.wpack_bytes, plan.xt_bytes_per_image, plan.col_bytes_per_image);
        return MDCN_OK;
    } catch (...) {
        return MDCN_E_INTERNAL;
    }
}

}  // extern "C"
