// prep.hip -- layout kernels of the gather + GEMM path: x to channels-last,
// and the weight repacked in the tap-major contraction order the gather
// writes.  Both only move data.
#include "device_common.h"
#include "launch.h"

namespace mdcn {

namespace {

constexpr int kTile = 64;

// One 64 (channels) x 64 (pixels) tile through LDS per workgroup.
template <typename T>
__global__ __launch_bounds__(256) void to_nhwc_kernel(const T *__restrict__ x, T *__restrict__ xt,
                                                      int C, int HW)
{
    __shared__ T tile[kTile][kTile + 1];
    const int p0 = blockIdx.x * kTile;
    const int c0 = blockIdx.y * kTile;
    const size_t img = size_t(blockIdx.z) * size_t(C) * size_t(HW);
    const int tx = threadIdx.x % kTile;
    const int ty = threadIdx.x / kTile;
    const T *src = x + img;
    T *dst = xt + img;
    for (int r = ty; r < kTile; r += 256 / kTile) {
        const int c = c0 + r, p = p0 + tx;
        tile[r][tx] = (c < C && p < HW) ? src[size_t(c) * HW + p] : T(0);
    }
    __syncthreads();
    for (int r = ty; r < kTile; r += 256 / kTile) {
        const int p = p0 + r, c = c0 + tx;
        if (p < HW && c < C)
            dst[size_t(p) * C + c] = tile[tx][r];
    }
}

// The same transpose with 16-byte global accesses on both sides (pixels
// along the load, channels along the store); requires C and H*W to be
// multiples of the vector width.
template <typename T>
__global__ __launch_bounds__(256) void to_nhwc_vec_kernel(const T *__restrict__ x,
                                                          T *__restrict__ xt, int C, int HW)
{
    constexpr int V = 16 / sizeof(T);
    constexpr int NV = kTile / V;                      // vectors per tile row
    __shared__ T tile[kTile][kTile + 1];
    const int p0 = blockIdx.x * kTile;
    const int c0 = blockIdx.y * kTile;
    const size_t img = size_t(blockIdx.z) * size_t(C) * size_t(HW);
    const T *src = x + img;
    T *dst = xt + img;
    for (int v = threadIdx.x; v < kTile * NV; v += 256) {
        const int r = v / NV, pv = (v % NV) * V;
        const int c = c0 + r, p = p0 + pv;
        Vec16<T> val;
        val.raw = make_uint4(0u, 0u, 0u, 0u);
        if (c < C && p < HW)
            val = load16(src + size_t(c) * HW + p);
#pragma unroll
        for (int e = 0; e < V; ++e)
            tile[r][pv + e] = val.e[e];
    }
    __syncthreads();
    for (int v = threadIdx.x; v < kTile * NV; v += 256) {
        const int r = v / NV, cv = (v % NV) * V;
        const int p = p0 + r, c = c0 + cv;
        if (p < HW && c < C) {
            Vec16<T> val;
#pragma unroll
            for (int e = 0; e < V; ++e)
                val.e[e] = tile[cv + e][r];
            store16(dst + size_t(p) * C + c, val);
        }
    }
}

template <typename T>
__global__ __launch_bounds__(256) void pack_weight_kernel(const T *__restrict__ w,
                                                          T *__restrict__ wp, int total, int Kp,
                                                          int Kg, int Cg, int K)
{
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= total)
        return;
    const int kk = t % Kp;
    const int co = t / Kp;
    T v = T(0);
    if (kk < Kg) {
        const int k = kk / Cg;
        const int cl = kk - k * Cg;
        v = w[(size_t(co) * Cg + cl) * K + k];
    }
    wp[t] = v;
}

template <typename T>
hipError_t to_nhwc_t(const Problem &p, int64_t cnt, const void *x, void *xt, hipStream_t s)
{
    const int HW = int(p.H * p.W);
    dim3 grid((HW + kTile - 1) / kTile, unsigned((p.C + kTile - 1) / kTile), 1);
    // The z dimension is limited to 65535; walk larger batches in slices.
    for (int64_t n0 = 0; n0 < cnt; n0 += 65535) {
        grid.z = unsigned(std::min<int64_t>(65535, cnt - n0));
        const size_t off = size_t(n0) * size_t(p.C) * size_t(HW);
        constexpr int V = 16 / sizeof(T);
        if (p.C % V == 0 && HW % V == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
            reinterpret_cast<uintptr_t>(xt) % 16 == 0)
            hipLaunchKernelGGL(to_nhwc_vec_kernel<T>, grid, dim3(256), 0, s,
                               static_cast<const T *>(x) + off, static_cast<T *>(xt) + off,
                               int(p.C), HW);
        else
            hipLaunchKernelGGL(to_nhwc_kernel<T>, grid, dim3(256), 0, s,
                               static_cast<const T *>(x) + off, static_cast<T *>(xt) + off,
                               int(p.C), HW);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

template <typename T>
hipError_t pack_weight_t(const Problem &p, const Plan &plan, const void *w, void *wp,
                         hipStream_t s)
{
    const int total = int(p.Co * plan.Kp);
    hipLaunchKernelGGL(pack_weight_kernel<T>, dim3((total + 255) / 256), dim3(256), 0, s,
                       static_cast<const T *>(w), static_cast<T *>(wp), total, int(plan.Kp),
                       int(p.Kg), int(p.Cg), int(p.K));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_to_nhwc(const Problem &p, int64_t cnt, const void *x, void *xt,
                          hipStream_t stream)
{
    switch (p.dtype) {
    case MDCN_F32: return to_nhwc_t<float>(p, cnt, x, xt, stream);
    case MDCN_F16: return to_nhwc_t<half_t>(p, cnt, x, xt, stream);
    case MDCN_BF16: return to_nhwc_t<bf16_t>(p, cnt, x, xt, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_pack_weight(const Problem &p, const Plan &plan, const void *weight,
                              void *wpack, hipStream_t stream)
{
    switch (p.dtype) {
    case MDCN_F32: return pack_weight_t<float>(p, plan, weight, wpack, stream);
    case MDCN_F16: return pack_weight_t<half_t>(p, plan, weight, wpack, stream);
    case MDCN_BF16: return pack_weight_t<bf16_t>(p, plan, weight, wpack, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mdcn
