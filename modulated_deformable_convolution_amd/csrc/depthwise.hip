// depthwise.hip -- direct forward for C/group == 1 (each output channel reads
// one input channel) [plugin guide §三: group equal to the number of
// outputs gives the depthwise convolution].  With one input channel per
// group the contraction is only kh*kw long, far too short for matrix cores,
// so one kernel samples, modulates, weighs and sums in registers and writes
// the output directly, with no column buffer:
//   out[n][co][pix] = bias[co] + sum_k w[co][k] * mask * bilinear0(x[n][co / Mg], sample)
#include "device_common.h"
#include "launch.h"

namespace mdcn {

namespace {

struct DwArgs {
    uint32_t total;          // Co * P
    int N, C, H, W, HW, Co, Mg, Cdg, K, P, Wo, kw;
    int sh, sw, ph, pw, dh, dw;
    int offC, mskC;
    int has_bias;
};

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
