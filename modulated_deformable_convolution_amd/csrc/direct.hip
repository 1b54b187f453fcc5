// direct.hip -- the whole forward of a small problem in one launch: one
// thread per output element, x, offsets, masks and weights read where they
// are (NCHW), fp32 arithmetic, one rounding.
//   out[n][co][ho][wo] = bias[co]
//       + sum_{c', i, j} w[co][c'][i][j] * mask * bilinear0(x[n][g*Cg + c'], h, w)
// [plugin guide §五 steps 1-3, computed per output element].
//
// For a problem of a few million multiply-adds the layout and GEMM kernels
// of the other paths cost a launch each, more than the arithmetic; here the
// sampling geometry of a (tap, offset group) is made once per thread and
// serves every input channel of that offset group.
#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace mdcn {

namespace {

struct DirectArgs {
    int N, C, H, W, Co, Cg, Mg, Cdg, kh, kw, Ho, Wo;
    int sh, sw, ph, pw, dh, dw;
    int offC, mskC;            // offset / mask channels per image
    uint32_t total;            // N * Co * Ho * Wo
};

// KK = 9: 3x3 taps, fully unrolled, so that every load of a thread is in
// flight at once (the thread's work is a few dependent round trips to
// memory, not arithmetic); KK = 0: any kernel size.
template <typename T, int KK>
__global__ __launch_bounds__(256) void direct_kernel(const T *__restrict__ x,
                                                     const T *__restrict__ off,
                                                     const T *__restrict__ msk,
                                                     const T *__restrict__ w,
                                                     const T *__restrict__ bias,
                                                     T *__restrict__ out, DirectArgs a)
{
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    if (t >= a.total)
        return;
    const int P = a.Ho * a.Wo;
    const int pix = int(t % uint32_t(P));
    const int co = int((t / uint32_t(P)) % uint32_t(a.Co));
    const int n = int(t / (uint32_t(P) * uint32_t(a.Co)));
    const int ho = pix / a.Wo, wo = pix - ho * a.Wo;
    const int g = co / a.Mg;
    const int K = KK ? KK : a.kh * a.kw;
    const int kw = KK ? 3 : a.kw;
    const int HW = a.H * a.W;
    const int c_first = g * a.Cg, c_end = c_first + a.Cg;
    const T *xn = x + size_t(n) * a.C * HW;
    const T *wrow = w + size_t(co) * a.Cg * K;
    float acc = 0.0f;
    // the group's channels, offset group by offset group
    for (int c0 = c_first; c0 < c_end;) {
        const int q = c0 / a.Cdg;
        const int c1 = min(c_end, (q + 1) * a.Cdg);
        const size_t ob = (size_t(n) * a.offC + size_t(q) * 2 * K) * P + pix;
        const size_t mb = (size_t(n) * a.mskC + size_t(q) * K) * P + pix;
        if constexpr (KK > 0) {
            // every tap's sample first, then 4 channels at a time
            Taps tp[KK];
#pragma unroll
            for (int k = 0; k < KK; ++k) {
                const int i = k / 3, j = k % 3;
                tp[k] = make_taps(ho * a.sh - a.ph + i * a.dh, wo * a.sw - a.pw + j * a.dw,
                                  to_f32(off[ob + size_t(2 * k) * P]),
                                  to_f32(off[ob + size_t(2 * k + 1) * P]),
                                  to_f32(msk[mb + size_t(k) * P]), a.H, a.W);
            }
            for (int cb = c0; cb < c1; cb += 4) {
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    const int c = min(cb + cc, c1 - 1);
                    const float on = cb + cc < c1 ? 1.0f : 0.0f;
                    const T *plane = xn + size_t(c) * HW;
#pragma unroll
                    for (int k = 0; k < KK; ++k) {
                        float v = 0.0f;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            // a corner off the image reads 0 (its safe address
                            // holds a pixel whose value must not enter)
                            const float xv = to_f32(plane[tp[k].idx[e]]);
                            v = fmaf(tp[k].wt[e], tp[k].valid[e] ? xv : 0.0f, v);
                        }
                        acc = fmaf(on * to_f32(wrow[size_t(c - c_first) * KK + k]), v, acc);
                    }
                }
            }
        } else {
            for (int k = 0; k < K; ++k) {
                const int i = k / kw, j = k - (k / kw) * kw;
                const Taps tp = make_taps(ho * a.sh - a.ph + i * a.dh, wo * a.sw - a.pw + j * a.dw,
                                          to_f32(off[ob + size_t(2 * k) * P]),
                                          to_f32(off[ob + size_t(2 * k + 1) * P]),
                                          to_f32(msk[mb + size_t(k) * P]), a.H, a.W);
                for (int c = c0; c < c1; ++c) {
                    const T *plane = xn + size_t(c) * HW;
                    float v = 0.0f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float xv = to_f32(plane[tp.idx[e]]);
                        v = fmaf(tp.wt[e], tp.valid[e] ? xv : 0.0f, v);
                    }
                    acc = fmaf(to_f32(wrow[size_t(c - c_first) * K + k]), v, acc);
                }
            }
        }
        c0 = c1;
    }
    if (bias)
        acc += to_f32(bias[co]);
    out[t] = from_f32<T>(acc);
}

template <typename T>
hipError_t direct_t(const Problem &p, const void *x, const void *offset, const void *mask,
                    const void *weight, const void *bias, void *out, hipStream_t s)
{
    const uint64_t total = uint64_t(p.N) * uint64_t(p.Co) * uint64_t(p.P);
    if (total == 0)
        return hipSuccess;
    if (total > 0xffffffffull - 255u)
        return hipErrorInvalidValue;
    DirectArgs a;
    a.N = int(p.N); a.C = int(p.C); a.H = int(p.H); a.W = int(p.W); a.Co = int(p.Co);
    a.Cg = int(p.Cg); a.Mg = int(p.Mg); a.Cdg = int(p.Cdg); a.kh = int(p.kh); a.kw = int(p.kw);
    a.Ho = int(p.Ho); a.Wo = int(p.Wo);
    a.sh = int(p.sh); a.sw = int(p.sw); a.ph = int(p.ph); a.pw = int(p.pw);
    a.dh = int(p.dh); a.dw = int(p.dw);
    a.offC = int(2 * p.DG * p.K); a.mskC = int(p.DG * p.K);
    a.total = uint32_t(total);
    const dim3 grid(unsigned((total + 255) / 256));
    if (p.kh == 3 && p.kw == 3)
        hipLaunchKernelGGL((direct_kernel<T, 9>), grid, dim3(256), 0, s,
                           static_cast<const T *>(x), static_cast<const T *>(offset),
                           static_cast<const T *>(mask), static_cast<const T *>(weight),
                           static_cast<const T *>(bias), static_cast<T *>(out), a);
    else
        hipLaunchKernelGGL((direct_kernel<T, 0>), grid, dim3(256), 0, s,
                           static_cast<const T *>(x), static_cast<const T *>(offset),
                           static_cast<const T *>(mask), static_cast<const T *>(weight),
                           static_cast<const T *>(bias), static_cast<T *>(out), a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_direct(const Problem &p, const void *x, const void *offset, const void *mask,
                         const void *weight, const void *bias, void *out, hipStream_t stream)
{
    switch (p.dtype) {
    case MDCN_F32: return direct_t<float>(p, x, offset, mask, weight, bias, out, stream);
    case MDCN_F16: return direct_t<half_t>(p, x, offset, mask, weight, bias, out, stream);
    case MDCN_BF16: return direct_t<bf16_t>(p, x, offset, mask, weight, bias, out, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mdcn
