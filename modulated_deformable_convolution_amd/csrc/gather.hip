// gather.hip -- deformable im2col: for every (group, image, output pixel,
// tap, channel) the modulated bilinear sample of the input
// [plugin guide §五 step 1: anchor = out*stride - pad, sample = anchor +
// tap*dilation + learned offset, bilinear interpolation reading 0 off the
// image, times the mask, into the column buffer].
//
// Layout choice (this library's, not the page's): x is read channels-last
// (NHWC, prepared by to_nhwc) and the columns are written K-contiguous,
// col[g][n*P + pix][k*Cg + c'], so that
//  - the 16-byte vector of channels c'..c'+VEC-1 at one bilinear corner is a
//    single contiguous load, and consecutive lanes (consecutive channel
//    vectors, then taps) read and write consecutive memory;
//  - the geometry (4 corner indices and 4 weights with the mask folded in)
//    is computed in fp32 per (tap, pixel) and reused for all VEC channels;
//  - the GEMM reads both of its operands K-contiguous, which is the register
//    layout of the MFMA A and B fragments.
#include "device_common.h"
#include "launch.h"

namespace mdcn {

namespace {

struct GatherArgs {
    uint32_t total;            // work items: G * cnt * P * K * CV
    uint32_t CV;               // channel vectors per group: Cg / VEC
    uint32_t K, P, cnt;
    int Cg, Cdg, C, H, W, HW, Wo, kw;
    int sh, sw, ph, pw, dh, dw;
    int offC, mskC;            // channels of offset and mask: 2*DG*K, DG*K
    int Kg, Kp;
};

template <typename T, int VEC>
__global__ __launch_bounds__(256) void deform_gather_kernel(const T *__restrict__ xt,
                                                            const T *__restrict__ off,
                                                            const T *__restrict__ msk,
                                                            T *__restrict__ col, GatherArgs a)
{
    uint32_t t = blockIdx.x * 256u + threadIdx.x;
    if (t >= a.total)
        return;
    const uint32_t cv = t % a.CV;
    t /= a.CV;
    const uint32_t k = t % a.K;
    t /= a.K;
    const uint32_t pix = t % a.P;
    t /= a.P;
    const uint32_t nl = t % a.cnt;
    const uint32_t g = t / a.cnt;

    const int c = int(g) * a.Cg + int(cv) * VEC;   // first input channel of this vector
    const int q = c / a.Cdg;                       // its offset group
    const int ho = int(pix) / a.Wo, wo = int(pix) - (int(pix) / a.Wo) * a.Wo;
    const int i = int(k) / a.kw, j = int(k) - (int(k) / a.kw) * a.kw;

    const size_t ob = (size_t(nl) * a.offC + size_t(q) * 2 * a.K + 2 * k) * a.P + pix;
    const float oh = to_f32(off[ob]);
    const float ow = to_f32(off[ob + a.P]);
    const float m = to_f32(msk[(size_t(nl) * a.mskC + size_t(q) * a.K + k) * a.P + pix]);
    const Taps tp = make_taps(ho * a.sh - a.ph + i * a.dh, wo * a.sw - a.pw + j * a.dw, oh, ow,
                              m, a.H, a.W);

    const T *img = xt + size_t(nl) * a.HW * a.C + c;
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e)
        acc[e] = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        if (!tp.valid[s])
            continue;
        const T *src = img + size_t(tp.idx[s]) * a.C;
        if constexpr (VEC == 1) {
            acc[0] = fmaf(tp.wt[s], to_f32(src[0]), acc[0]);
        } else {
            const Vec16<T> v = load16(src);
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                acc[e] = fmaf(tp.wt[s], to_f32(v.e[e]), acc[e]);
        }
    }
    T *row = col + (size_t(g) * a.cnt + nl) * a.P * a.Kp + size_t(pix) * a.Kp;
    T *dst = row + k * a.Cg + cv * VEC;
    if constexpr (VEC == 1) {
        dst[0] = from_f32<T>(acc[0]);
    } else {
        Vec16<T> o;
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            o.e[e] = from_f32<T>(acc[e]);
        store16(dst, o);
    }
    // The last item of each row zeroes the row's padding [Kg, Kp).
    if (k == a.K - 1 && cv == a.CV - 1) {
        for (int kk = a.Kg; kk < a.Kp; ++kk)
            row[kk] = T(0);
    }
}

template <typename T>
hipError_t gather_t(const Problem &p, const Plan &plan, int64_t cnt, const void *xt,
                    const void *offset, const void *mask, void *col, hipStream_t s)
{
    constexpr int V = 16 / sizeof(T);
    const bool vec = (p.Cg % V == 0) && (p.Cdg % V == 0);
    GatherArgs a;
    a.CV = uint32_t(vec ? p.Cg / V : p.Cg);
    a.K = uint32_t(p.K);
    a.P = uint32_t(p.P);
    a.cnt = uint32_t(cnt);
    a.total = uint32_t(uint64_t(p.G) * uint64_t(cnt) * uint64_t(p.P) * uint64_t(p.K) * a.CV);
    a.Cg = int(p.Cg); a.Cdg = int(p.Cdg); a.C = int(p.C);
    a.H = int(p.H); a.W = int(p.W); a.HW = int(p.H * p.W);
    a.Wo = int(p.Wo); a.kw = int(p.kw);
    a.sh = int(p.sh); a.sw = int(p.sw); a.ph = int(p.ph); a.pw = int(p.pw);
    a.dh = int(p.dh); a.dw = int(p.dw);
    a.offC = int(2 * p.DG * p.K); a.mskC = int(p.DG * p.K);
    a.Kg = int(p.Kg); a.Kp = int(plan.Kp);
    const dim3 grid((a.total + 255u) / 256u);
    if (vec)
        hipLaunchKernelGGL((deform_gather_kernel<T, V>), grid, dim3(256), 0, s,
                           static_cast<const T *>(xt), static_cast<const T *>(offset),
                           static_cast<const T *>(mask), static_cast<T *>(col), a);
    else
        hipLaunchKernelGGL((deform_gather_kernel<T, 1>), grid, dim3(256), 0, s,
                           static_cast<const T *>(xt), static_cast<const T *>(offset),
                           static_cast<const T *>(mask), static_cast<T *>(col), a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gather(const Problem &p, const Plan &plan, int64_t cnt, const void *xt,
                         const void *offset, const void *mask, void *col, hipStream_t stream)
{
    switch (p.dtype) {
    case MDCN_F32: return gather_t<float>(p, plan, cnt, xt, offset, mask, col, stream);
    case MDCN_F16: return gather_t<half_t>(p, plan, cnt, xt, offset, mask, col, stream);
    case MDCN_BF16: return gather_t<bf16_t>(p, plan, cnt, xt, offset, mask, col, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mdcn
