// quant.hip -- the FP8 path's weight: each output channel's row scaled by a
// power of two and rounded to OCP E4M3, in the tap-major order of the
// columns (kk = k*Cg + c', zero for kk >= Kg).
//
// Row co gets the exponent e, the largest integer with
// max|w[co]| * 2^e <= 448 (0 for a row with no nonzero finite maximum;
// clamped to [-126, 126]); wq[co][kk] = E4M3(w * 2^e) and
// wscale[co] = 2^-e, which the GEMM epilogue applies to the row's sums.
// Scaling by a power of two is exact, so the only rounding is E4M3's own.
#include "device_common.h"
#include "launch.h"

namespace mdcn {

namespace {

template <typename T>
__global__ __launch_bounds__(256) void quantize_weight_kernel(const T *__restrict__ w,
                                                              e4m3_t *__restrict__ wq,
                                                              float *__restrict__ wscale,
                                                              int Kg, int Kp, int Cg, int K)
{
    __shared__ float wave_max[4];
    const int co = int(blockIdx.x);
    const T *row = w + size_t(co) * Kg;           // weight [Co][Cg][kh][kw]: Kg per row
    float mx = 0.0f;
    for (int t = int(threadIdx.x); t < Kg; t += 256)
        mx = fmaxf(mx, fabsf(to_f32(row[t])));    // fmaxf skips NaN
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1)
        mx = fmaxf(mx, __shfl_xor(mx, d, 64));
    if ((threadIdx.x & 63) == 0)
        wave_max[threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
    int e = 0;
    if (mx > 0.0f && !__builtin_isinf(mx)) {
        int ex;
        const float f = frexpf(mx, &ex);          // mx = f * 2^ex, f in [0.5, 1)
        e = (f <= 0.875f) ? 9 - ex : 8 - ex;      // 448 = 0.875 * 2^9
        e = min(126, max(-126, e));
    }
    e4m3_t *dst = wq + size_t(co) * Kp;
    for (int kk = int(threadIdx.x); kk < Kp; kk += 256) {
        e4m3_t q = 0;
        if (kk < Kg) {
            const int k = kk / Cg;
            const int cl = kk - k * Cg;
            q = to_e4m3(ldexpf(to_f32(row[cl * K + k]), e));
        }
        dst[kk] = q;
    }
    if (threadIdx.x == 0)
        wscale[co] = ldexpf(1.0f, -e);
}

template <typename T>
hipError_t quantize_t(const Problem &p, const Plan &plan, const void *w, void *wq, float *wscale,
                      hipStream_t s)
{
    if (p.Co == 0)
        return hipSuccess;
    hipLaunchKernelGGL((quantize_weight_kernel<T>), dim3(unsigned(p.Co)), dim3(256), 0, s,
                       static_cast<const T *>(w), static_cast<e4m3_t *>(wq), wscale, int(p.Kg),
                       int(plan.Kp), int(p.Cg), int(p.K));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_weight(const Problem &p, const Plan &plan, const void *weight,
                                  void *wq, float *wscale, hipStream_t stream)
{
    switch (p.dtype) {
    case MDCN_F32: return quantize_t<float>(p, plan, weight, wq, wscale, stream);
    case MDCN_F16: return quantize_t<half_t>(p, plan, weight, wq, wscale, stream);
    case MDCN_BF16: return quantize_t<bf16_t>(p, plan, weight, wq, wscale, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mdcn
