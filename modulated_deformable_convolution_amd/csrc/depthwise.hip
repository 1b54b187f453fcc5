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
// Taps are branch-free: a sample entirely off the image reads a safe address
// with factor 0.  With one output channel per input channel and 3x3 taps
// (the common case) the nine weights are loaded once per workgroup.
//
// Workgroups are ordered so that those of one image run on one XCD: the
// image's offsets and masks, read by every channel block, stay in that L2.
// When a plane does not fit in LDS, a plain kernel reading x from global
// memory is used instead.
#include <cstdlib>

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

template <typename T, int CB, int KT, int UP, bool MG1>
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

    const int q = c0 / a.Cdg;                        // every staged channel is in block q
    // Weights of the workgroup's output channels, when known to be few.
    float wreg[CB][KT > 0 ? KT : 1];
    if constexpr (MG1 && KT > 0) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int k = 0; k < KT; ++k)
                wreg[cb][k] = to_f32(w[size_t(min(c0 + cb, a.C - 1)) * KT + k]);
    }
    const int mg_pass = MG1 ? 1 : kMaxMg;
    for (int m0 = 0; m0 < a.Mg; m0 += mg_pass) {
        const int nm = MG1 ? 1 : min(kMaxMg, a.Mg - m0);
        // Each thread takes UP pixels at a time (kStagedThreads apart), so that
        // the offsets and masks of all of them are in flight together.
        for (int pbase = int(threadIdx.x); pbase < a.P; pbase += UP * kStagedThreads) {
            float acc[UP][CB][kMaxMg];
#pragma unroll
            for (int u = 0; u < UP; ++u)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int mm = 0; mm < kMaxMg; ++mm)
                        acc[u][cb][mm] = 0.0f;
            // Per pixel slot: the anchor (top-left tap position without offset),
            // one division per pixel.  A slot past the end works on pixel 0 and
            // stores nothing.
            int pix_u[UP], ah[UP], aw[UP];
#pragma unroll
            for (int u = 0; u < UP; ++u) {
                const int pix = pbase + u * kStagedThreads < a.P ? pbase + u * kStagedThreads : 0;
                const int ho = pix / a.Wo;
                pix_u[u] = pix;
                ah[u] = ho * a.sh - a.ph;
                aw[u] = (pix - ho * a.Wo) * a.sw - a.pw;
            }
            // One tap: sample the staged planes at anchor + tap offset + the
            // learned offset, and accumulate into slot u.  Branch-free: a sample
            // entirely off the image reads staged entry 0 with factor 0.
            auto tap = [&](int u, int k, int th, int tw, float oh, float ow, float m) {
                const float lim = 33554432.0f;       // 2^25: farther is off any image
                const bool fin = fabsf(oh) <= lim && fabsf(ow) <= lim;
                const float fh = fin ? floorf(oh) : 0.0f, fw = fin ? floorf(ow) : 0.0f;
                const int h0 = ah[u] + th + int(fh);
                const int w0 = aw[u] + tw + int(fw);
                const bool ok = fin && h0 >= -1 && h0 < a.H && w0 >= -1 && w0 < a.W;
                // fractions in [0, 1) (0 for a non-finite or huge offset, so
                // that every weight stays finite and the factor 0 gives 0)
                const float ly = fin ? oh - fh : 0.0f, lx = fin ? ow - fw : 0.0f;
                const float hy = 1.0f - ly, hx = 1.0f - lx;
                const float fac = ok ? m : 0.0f;
                const float w00 = hy * hx, w10 = ly * hx, w01 = hy * lx, w11 = ly * lx;
                const int idx = ok ? (h0 + 1) * PW + (w0 + 1) : 0;
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    const float2 left = planes[cb * PL + idx];       // (X[h0][w0], X[h0+1][w0])
                    const float2 right = planes[cb * PL + idx + 1];  // (.., w0+1)
                    float v = w00 * left.x;
                    v = fmaf(w10, left.y, v);
                    v = fmaf(w01, right.x, v);
                    v = fmaf(w11, right.y, v);
                    v *= fac;
                    if constexpr (MG1 && KT > 0) {
                        acc[u][cb][0] = fmaf(wreg[cb][k], v, acc[u][cb][0]);
                    } else {
                        const int co = min(c0 + cb, a.C - 1) * a.Mg + m0;
#pragma unroll
                        for (int mm = 0; mm < kMaxMg; ++mm)
                            if (mm < nm)
                                acc[u][cb][mm] = fmaf(to_f32(w[size_t(co + mm) * a.K + k]), v,
                                                      acc[u][cb][mm]);
                    }
                }
            };
            if constexpr (KT > 0) {
                // 3x3 taps: tap rows/columns are compile-time, all of the
                // pixels' offsets and masks are in flight at once
                float oh[UP][KT], ow[UP][KT], mk[UP][KT];
#pragma unroll
                for (int u = 0; u < UP; ++u) {
                    const T *offp = off + (size_t(n) * a.offC + size_t(q) * 2 * KT) * a.P + pix_u[u];
                    const T *mskp = msk + (size_t(n) * a.mskC + size_t(q) * KT) * a.P + pix_u[u];
#pragma unroll
                    for (int k = 0; k < KT; ++k) {
                        oh[u][k] = to_f32(offp[size_t(2 * k) * a.P]);
                        ow[u][k] = to_f32(offp[size_t(2 * k + 1) * a.P]);
                        mk[u][k] = to_f32(mskp[size_t(k) * a.P]);
                    }
                }
#pragma unroll
                for (int u = 0; u < UP; ++u)
#pragma unroll
                    for (int k = 0; k < KT; ++k)
                        tap(u, k, (k / 3) * a.dh, (k % 3) * a.dw, oh[u][k], ow[u][k], mk[u][k]);
            } else {
#pragma unroll
                for (int u = 0; u < UP; ++u) {
                    const T *offp = off + (size_t(n) * a.offC + size_t(q) * 2 * a.K) * a.P + pix_u[u];
                    const T *mskp = msk + (size_t(n) * a.mskC + size_t(q) * a.K) * a.P + pix_u[u];
                    int i = 0, j = 0;
                    for (int k = 0; k < a.K; ++k) {
                        tap(u, k, i * a.dh, j * a.dw, to_f32(offp[size_t(2 * k) * a.P]),
                            to_f32(offp[size_t(2 * k + 1) * a.P]), to_f32(mskp[size_t(k) * a.P]));
                        if (++j == a.kw) {
                            j = 0;
                            ++i;
                        }
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < UP; ++u) {
                const int pix = pbase + u * kStagedThreads;
                if (pix >= a.P)
                    break;
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
                        out[(size_t(n) * a.Co + co) * a.P + pix] = from_f32<T>(acc[u][cb][mm] + b);
                    }
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
using DwKernel = void (*)(const T *, const T *, const T *, const T *, const T *, T *, DwArgs);

// The staged kernel instance for (planes, compile-time taps, pixels per
// thread, exactly one output per input channel).
template <typename T>
DwKernel<T> staged_fn(int cb, int kt, int up, bool mg1)
{
#define MDCN_DW_PICK(CB_, KT_, UP_)                                                            \
    if (cb == CB_ && kt == KT_ && up == UP_)                                                   \
        return mg1 ? &depthwise_staged_kernel<T, CB_, KT_, UP_, true>                          \
                   : &depthwise_staged_kernel<T, CB_, KT_, UP_, false>;
    MDCN_DW_PICK(1, 9, 1) MDCN_DW_PICK(1, 9, 2) MDCN_DW_PICK(1, 9, 4)
    MDCN_DW_PICK(1, 0, 1) MDCN_DW_PICK(1, 0, 2) MDCN_DW_PICK(1, 0, 4)
    MDCN_DW_PICK(2, 9, 1) MDCN_DW_PICK(2, 9, 2) MDCN_DW_PICK(2, 9, 4)
    MDCN_DW_PICK(2, 0, 1) MDCN_DW_PICK(2, 0, 2) MDCN_DW_PICK(2, 0, 4)
#undef MDCN_DW_PICK
    return nullptr;
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
    // Two planes per workgroup when they fit and share an offset group (each
    // workgroup reads all of its image's offsets and masks, so sharing them
    // between planes halves that traffic), two pixels per thread in flight.
    // MDCN_DW_PLANES=1|2 and MDCN_DW_PIXELS=1|2|4 override (for tuning).
    int cb = (p.Cdg % 2 == 0 && 2 * plane_bytes <= kLdsBytes) ? 2 : 1, up = 2;
    if (const char *env = std::getenv("MDCN_DW_PLANES")) {
        const int v = std::atoi(env);
        if (v == 1)
            cb = 1;
        else if (v == 2 && p.Cdg % 2 == 0 && 2 * plane_bytes <= kLdsBytes)
            cb = 2;
    }
    if (const char *env = std::getenv("MDCN_DW_PIXELS")) {
        const int v = std::atoi(env);
        if (v == 1 || v == 2 || v == 4)
            up = v;
    }
    if (cb * plane_bytes <= kLdsBytes) {
        a.cblocks = int((p.C + cb - 1) / cb);
        const dim3 grid(unsigned(uint64_t(p.N) * a.cblocks));
        const size_t lds = cb * plane_bytes;
        const int kt = (p.kh == 3 && p.kw == 3) ? 9 : 0;   // compile-time 3x3 taps
        const DwKernel<T> fn = staged_fn<T>(cb, kt, up, p.Mg == 1);
        if (hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) != hipSuccess) {
            (void)hipGetLastError();       // clear it; use the plain kernel below
        } else {
            hipLaunchKernelGGL(fn, grid, dim3(kStagedThreads), lds, s, static_cast<const T *>(x),
                               static_cast<const T *>(offset), static_cast<const T *>(mask),
                               static_cast<const T *>(weight), static_cast<const T *>(bias),
                               static_cast<T *>(out), a);
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
