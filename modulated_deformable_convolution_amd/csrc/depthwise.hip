// depthwise.hip -- direct forward for C/group == 1 (each output channel reads
// one input channel) [plugin guide §三: group equal to the number of
// outputs gives the depthwise convolution].  With one input channel per
// group the contraction is only kh*kw long, far too short for matrix cores,
// so one kernel samples, modulates, weighs and sums in registers and writes
// the output directly, with no column buffer:
//   out[n][co][pix] = bias[co] + sum_k w[co][k] * mask * bilinear0(x[n][co / Mg], sample)
//
// The samples land anywhere on the plane (offsets are unbounded), so each
// output needs kh*kw*4 effectively random reads of its input plane.  The
// fastest memory for random reads is LDS: a workgroup stages CB whole input
// planes there, in a layout where one 16-byte read returns all four bilinear
// corners.  The plane is padded by one zero row/column on every side (the
// zero that bilinear interpolation reads off the image), and entry [r][c] of
// the staged plane holds the vertical pair (X[r][c], X[r+1][c]) of the padded
// plane X.  Corners (h0, w0) .. (h0+1, w0+1) are then pairs [h0+1][w0+1] and
// [h0+1][w0+2]: adjacent 8-byte entries, one ds_read2_b64.  Any sample with
// -1 <= h0 <= H-1 and -1 <= w0 <= W-1 reads inside the staged plane; any other
// sample is entirely off the image and contributes 0.
//
// Workgroups are ordered so that those of one image run on one XCD: the
// image's offsets and masks, read by every channel block, stay in that L2.
// When a plane does not fit in LDS, a plain kernel reading x from global
// memory is used instead.
#include "device_common.h"
#include "launch.h"

namespace mdcn {

namespace {

struct DwArgs {
    uint32_t total;          // Co * P (plain kernel)
    int N, C, H, W, HW, Co, Mg, Cdg, K, P, Wo, kw;
    int sh, sw, ph, pw, dh, dw;
    int offC, mskC;
    int has_bias;
    int cblocks;             // channel blocks per image (staged kernel)
};

constexpr int kStagedThreads = 512;
constexpr int kMaxMg = 4;                    // output channels per input channel per pass
constexpr size_t kLdsBytes = 160 * 1024;

template <typename T, int CB>
__global__ __launch_bounds__(kStagedThreads) void depthwise_staged_kernel(
    const T *__restrict__ x, const T *__restrict__ off, const T *__restrict__ msk,
    const T *__restrict__ w, const T *__restrict__ bias, T *__restrict__ out, DwArgs a)
{
    extern __shared__ __attribute__((aligned(16))) float2 planes[];
    const int PW = a.W + 2;                          // staged row length (pairs)
    const int PL = (a.H + 1) * PW;                   // staged plane length (pairs)

    const uint32_t lid = xcd_swizzle(blockIdx.x, gridDim.x);
    const int n = __builtin_amdgcn_readfirstlane(int(lid / uint32_t(a.cblocks)));
    const int c0 = __builtin_amdgcn_readfirstlane(int(lid % uint32_t(a.cblocks)) * CB);
    const int ncb = min(CB, a.C - c0);

    // Stage: pair [r][c] = (X[r][c], X[r+1][c]), X[r][c] = x[r-1][c-1] or 0.
    for (int cb = 0; cb < CB; ++cb) {
        const T *plane = x + (size_t(n) * a.C + min(c0 + cb, a.C - 1)) * a.HW;
        for (int e = int(threadIdx.x); e < PL; e += kStagedThreads) {
            const int r = e / PW, c = e - (e / PW) * PW;
            const int xr = r - 1, xc = c - 1;
            const bool cin = xc >= 0 && xc < a.W;
            const float v0 = (cin && xr >= 0) ? to_f32(plane[xr * a.W + xc]) : 0.0f;
            const float v1 = (cin && xr + 1 < a.H) ? to_f32(plane[(xr + 1) * a.W + xc]) : 0.0f;
            planes[cb * PL + e] = make_float2(v0, v1);
        }
    }
    __syncthreads();

    // Weights and bias of the workgroup's output channels (uniform).
    const int q = c0 / a.Cdg;                        // every staged channel is in block q
    for (int m0 = 0; m0 < a.Mg; m0 += kMaxMg) {
        const int nm = min(kMaxMg, a.Mg - m0);
        for (int pix = int(threadIdx.x); pix < a.P; pix += kStagedThreads) {
            const int ho = pix / a.Wo, wo = pix - (pix / a.Wo) * a.Wo;
            const T *offp = off + (size_t(n) * a.offC + size_t(q) * 2 * a.K) * a.P + pix;
            const T *mskp = msk + (size_t(n) * a.mskC + size_t(q) * a.K) * a.P + pix;
            float acc[CB][kMaxMg];
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int mm = 0; mm < kMaxMg; ++mm)
                    acc[cb][mm] = 0.0f;
            for (int k = 0; k < a.K; ++k) {
                const int i = k / a.kw, j = k - (k / a.kw) * a.kw;
                const float oh = to_f32(offp[size_t(2 * k) * a.P]);
                const float ow = to_f32(offp[size_t(2 * k + 1) * a.P]);
                const float m = to_f32(mskp[size_t(k) * a.P]);
                const float lim = 33554432.0f;       // 2^25: farther is off any image
                if (!(fabsf(oh) <= lim && fabsf(ow) <= lim))
                    continue;
                const float fh = floorf(oh), fw = floorf(ow);
                const int h0 = ho * a.sh - a.ph + i * a.dh + int(fh);
                const int w0 = wo * a.sw - a.pw + j * a.dw + int(fw);
                if (h0 < -1 || h0 >= a.H || w0 < -1 || w0 >= a.W)
                    continue;                         // all four corners off the image
                const float ly = oh - fh, lx = ow - fw;
                const float hy = 1.0f - ly, hx = 1.0f - lx;
                const float w00 = hy * hx, w10 = ly * hx, w01 = hy * lx, w11 = ly * lx;
                const int idx = (h0 + 1) * PW + (w0 + 1);
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    if (cb >= ncb)
                        break;
                    const float2 left = planes[cb * PL + idx];       // (X[h0][w0], X[h0+1][w0])
                    const float2 right = planes[cb * PL + idx + 1];  // (.., w0+1)
                    float v = w00 * left.x;
                    v = fmaf(w10, left.y, v);
                    v = fmaf(w01, right.x, v);
                    v = fmaf(w11, right.y, v);
                    v *= m;
                    const int co = (c0 + cb) * a.Mg + m0;
#pragma unroll
                    for (int mm = 0; mm < kMaxMg; ++mm)
                        if (mm < nm)
                            acc[cb][mm] = fmaf(to_f32(w[size_t(co + mm) * a.K + k]), v,
                                               acc[cb][mm]);
                }
            }
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                if (cb >= ncb)
                    break;
#pragma unroll
                for (int mm = 0; mm < kMaxMg; ++mm) {
                    if (mm >= nm)
                        break;
                    const int co = (c0 + cb) * a.Mg + m0 + mm;
                    const float b = a.has_bias ? to_f32(bias[co]) : 0.0f;
                    out[(size_t(n) * a.Co + co) * a.P + pix] = from_f32<T>(acc[cb][mm] + b);
                }
            }
        }
    }
}

// Plain kernel: one thread per (output channel, pixel), x read from global.
template <typename T>
__global__ __launch_bounds__(256) void depthwise_kernel(const T *__restrict__ x,
                                                        const T *__restrict__ off,
                                                        const T *__restrict__ msk,
                                                        const T *__restrict__ w,
                                                        const T *__restrict__ bias,
                                                        T *__restrict__ out, DwArgs a)
{
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    if (t >= a.total)
        return;
    const int pix = int(t % uint32_t(a.P));
    const int co = int(t / uint32_t(a.P));
    const int c = co / a.Mg;          // the one input channel of this output channel
    const int q = c / a.Cdg;          // its offset group
    const int ho = pix / a.Wo, wo = pix - (pix / a.Wo) * a.Wo;
    const float b = a.has_bias ? to_f32(bias[co]) : 0.0f;
    for (int n = blockIdx.y; n < a.N; n += gridDim.y) {
        const T *plane = x + (size_t(n) * a.C + c) * a.HW;
        const T *offn = off + (size_t(n) * a.offC + size_t(q) * 2 * a.K) * a.P + pix;
        const T *mskn = msk + (size_t(n) * a.mskC + size_t(q) * a.K) * a.P + pix;
        float acc = 0.0f;
        for (int k = 0; k < a.K; ++k) {
            const int i = k / a.kw, j = k - (k / a.kw) * a.kw;
            const float oh = to_f32(offn[size_t(2 * k) * a.P]);
            const float ow = to_f32(offn[size_t(2 * k + 1) * a.P]);
            const float m = to_f32(mskn[size_t(k) * a.P]);
            const Taps tp = make_taps(ho * a.sh - a.ph + i * a.dh, wo * a.sw - a.pw + j * a.dw,
                                      oh, ow, m, a.H, a.W);
            float v = 0.0f;
#pragma unroll
            for (int s = 0; s < 4; ++s)
                if (tp.valid[s])
                    v = fmaf(tp.wt[s], to_f32(plane[tp.idx[s]]), v);
            acc = fmaf(to_f32(w[size_t(co) * a.K + k]), v, acc);
        }
        out[(size_t(n) * a.Co + co) * a.P + pix] = from_f32<T>(acc + b);
    }
}

template <typename T>
hipError_t depthwise_t(const Problem &p, const void *x, const void *offset, const void *mask,
                       const void *weight, const void *bias, void *out, hipStream_t s)
{
    DwArgs a;
    a.total = uint32_t(p.Co * p.P);
    a.N = int(p.N); a.C = int(p.C); a.H = int(p.H); a.W = int(p.W); a.HW = int(p.H * p.W);
    a.Co = int(p.Co); a.Mg = int(p.Mg); a.Cdg = int(p.Cdg); a.K = int(p.K); a.P = int(p.P);
    a.Wo = int(p.Wo); a.kw = int(p.kw);
    a.sh = int(p.sh); a.sw = int(p.sw); a.ph = int(p.ph); a.pw = int(p.pw);
    a.dh = int(p.dh); a.dw = int(p.dw);
    a.offC = int(2 * p.DG * p.K); a.mskC = int(p.DG * p.K);
    a.has_bias = bias != nullptr;
    const size_t plane_bytes = size_t(p.H + 1) * size_t(p.W + 2) * sizeof(float2);
    // Two planes per workgroup when they fit and share an offset group.
    const int cb = (2 * plane_bytes <= kLdsBytes && p.Cdg % 2 == 0) ? 2 : 1;
    if (cb * plane_bytes <= kLdsBytes) {
        a.cblocks = int((p.C + cb - 1) / cb);
        const dim3 grid(unsigned(uint64_t(p.N) * a.cblocks));
        const size_t lds = cb * plane_bytes;
        const void *fn = cb == 2
                             ? reinterpret_cast<const void *>(&depthwise_staged_kernel<T, 2>)
                             : reinterpret_cast<const void *>(&depthwise_staged_kernel<T, 1>);
        if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) !=
            hipSuccess) {
            (void)hipGetLastError();       // clear it; use the plain kernel below
        } else if (cb == 2) {
            hipLaunchKernelGGL((depthwise_staged_kernel<T, 2>), grid, dim3(kStagedThreads), lds,
                               s, static_cast<const T *>(x), static_cast<const T *>(offset),
                               static_cast<const T *>(mask), static_cast<const T *>(weight),
                               static_cast<const T *>(bias), static_cast<T *>(out), a);
            return hipGetLastError();
        } else {
            hipLaunchKernelGGL((depthwise_staged_kernel<T, 1>), grid, dim3(kStagedThreads), lds,
                               s, static_cast<const T *>(x), static_cast<const T *>(offset),
                               static_cast<const T *>(mask), static_cast<const T *>(weight),
                               static_cast<const T *>(bias), static_cast<T *>(out), a);
            return hipGetLastError();
        }
    }
    const dim3 grid((a.total + 255u) / 256u, unsigned(std::min<int64_t>(p.N, 65535)));
    hipLaunchKernelGGL(depthwise_kernel<T>, grid, dim3(256), 0, s, static_cast<const T *>(x),
                       static_cast<const T *>(offset), static_cast<const T *>(mask),
                       static_cast<const T *>(weight), static_cast<const T *>(bias),
                       static_cast<T *>(out), a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_depthwise(const Problem &p, const void *x, const void *offset,
                            const void *mask, const void *weight, const void *bias, void *out,
                            hipStream_t stream)
{
    switch (p.dtype) {
    case MDCN_F32: return depthwise_t<float>(p, x, offset, mask, weight, bias, out, stream);
    case MDCN_F16: return depthwise_t<half_t>(p, x, offset, mask, weight, bias, out, stream);
    case MDCN_BF16: return depthwise_t<bf16_t>(p, x, offset, mask, weight, bias, out, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mdcn
