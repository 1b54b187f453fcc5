// backward.hip -- gradients of the forward (fp32): with g = dL/dout,
//   grad_bias[co]          = sum_{n,p} g[n][co][p]
//   grad_weight[co][c'][k] = sum_{n,p} g[n][co][p] * col(n, c, k, p)
//   gcol(n, c, k, p)       = sum_{m in the group} weight[m][c'][k] * g[n][m][p]
// and, per (image, offset group, tap, pixel), from gcol of the group's
// channels: grad_mask += gcol * sample, grad_offset += gcol * mask *
// d sample / d(h, w), and grad_x gets gcol * mask * corner weight at each
// bilinear corner on the image.  col is the modulated sample the forward's
// im2col produces [plugin guide §五 step 1]; the derivative of the bilinear
// sample is taken on the cell floor() selects (corners off the image count
// as 0; a sample outside the open window, or with a non-finite coordinate,
// has zero derivatives).
//
// Kernels: a strided tiled fp32 GEMM for the two contractions (the weight
// gradient split over pixels with atomic adds into an fp32 accumulator), the
// sampling backward (a team of lanes per offset group, tap and pixel, spread
// over the group's channels, channels-last: grad_x by atomic adds into an
// NHWC buffer, transposed to NCHW per image), and small fill, reduce and
// permute kernels.  The images are processed one at a time.
#include <algorithm>
#include <cstdlib>

#include "device_common.h"
#include "launch.h"

namespace mdcn {

namespace {

constexpr int kBT = 64;     // GEMM tile (rows and columns)
constexpr int kBL = 16;     // GEMM contraction slice

// C(i, j) (+)= sum_l A(i, l) * B(l, j), element (i, l) of A at
// A[i*ai + l*al], and so on.  Rows i < M, columns j < N, l in
// [z*lchunk, min(L, (z+1)*lchunk)) for grid z.
struct GemmDesc {
    const void *A;            // TA elements
    int64_t ai, al;
    const void *B;            // TB elements
    int64_t bl, bj;
    float *C;
    int64_t ci, cj;
    int M, N, L, lchunk;
    int atomic;            // add into C atomically (split contraction) instead of storing
};

template <typename TA, typename TB>
__global__ __launch_bounds__(256) void sgemm_kernel(GemmDesc d)
{
    const TA *A = static_cast<const TA *>(d.A);
    const TB *B = static_cast<const TB *>(d.B);
    __shared__ float As[kBL][kBT + 4];
    __shared__ float Bs[kBL][kBT + 4];
    const int i0 = int(blockIdx.y) * kBT, j0 = int(blockIdx.x) * kBT;
    const int l_begin = int(blockIdx.z) * d.lchunk;
    const int l_end = min(d.L, l_begin + d.lchunk);
    const int tx = int(threadIdx.x) & 15, ty = int(threadIdx.x) >> 4;
    const bool a_i_fast = d.ai == 1, b_j_fast = d.bj == 1;   // coalesce along the contiguous index
    float acc[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            acc[u][v] = 0.0f;
    for (int l0 = l_begin; l0 < l_end; l0 += kBL) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int idx = int(threadIdx.x) + 256 * r;
            const int ii = a_i_fast ? idx % kBT : idx / kBL;
            const int la = a_i_fast ? idx / kBT : idx % kBL;
            const int gi = i0 + ii, gl = l0 + la;
            As[la][ii] = (gi < d.M && gl < l_end) ? to_f32(A[gi * d.ai + gl * d.al]) : 0.0f;
            const int jj = b_j_fast ? idx % kBT : idx / kBL;
            const int lb = b_j_fast ? idx / kBT : idx % kBL;
            const int gj = j0 + jj, glb = l0 + lb;
            Bs[lb][jj] = (gj < d.N && glb < l_end) ? to_f32(B[glb * d.bl + gj * d.bj]) : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int l = 0; l < kBL; ++l) {
            float a[4], b[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                a[u] = As[l][ty + 16 * u];
                b[u] = Bs[l][tx + 16 * u];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    acc[u][v] = fmaf(a[u], b[v], acc[u][v]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = i0 + ty + 16 * u, j = j0 + tx + 16 * v;
            if (i < d.M && j < d.N) {
                float *c = d.C + i * d.ci + j * d.cj;
                if (d.atomic)
                    atomicAdd(c, acc[u][v]);
                else
                    *c = acc[u][v];
            }
        }
}

template <typename TA, typename TB>
hipError_t run_gemm(const GemmDesc &d, int splits, hipStream_t s)
{
    if (d.M <= 0 || d.N <= 0 || d.L <= 0)
        return hipSuccess;
    const dim3 grid(unsigned((d.N + kBT - 1) / kBT), unsigned((d.M + kBT - 1) / kBT),
                    unsigned(splits));
    if (grid.y > 65535u || grid.z > 65535u)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((sgemm_kernel<TA, TB>), grid, dim3(256), 0, s, d);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float *p, int64_t n)
{
    const int64_t stride = int64_t(gridDim.x) * 256;
    for (int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x; t < n; t += stride)
        p[t] = 0.0f;
}

// grad_bias[co] = sum over images and pixels of g[n][co][p]; one workgroup per co.
// (1024 threads: one workgroup per output channel sums N*P values)
template <typename T>
__global__ __launch_bounds__(1024) void bias_grad_kernel(const T *__restrict__ g,
                                                         T *__restrict__ gb, int N, int Co, int P)
{
    __shared__ float part[16];
    const int co = int(blockIdx.x);
    float s = 0.0f;
    for (int n = 0; n < N; ++n) {
        const T *row = g + (int64_t(n) * Co + co) * P;
        for (int p = int(threadIdx.x); p < P; p += 1024)
            s += to_f32(row[p]);
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1)
        s += __shfl_xor(s, d, 64);
    if ((threadIdx.x & 63) == 0)
        part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.0f;
        for (int w = 0; w < 16; ++w)
            t += part[w];
        gb[co] = from_f32<T>(t);
    }
}

// grad_weight[g*Mg + m][c'][k] = acc[g][m][k*Cg + c'] (the accumulator is in
// the columns' tap-major order).
template <typename T>
__global__ __launch_bounds__(256) void weight_out_kernel(const float *__restrict__ acc,
                                                         T *__restrict__ gw, int Co, int Cg,
                                                         int K, int Kp)
{
    const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t total = int64_t(Co) * Cg * K;
    if (t >= total)
        return;
    const int k = int(t % K);
    const int cl = int((t / K) % Cg);
    const int64_t co = t / (int64_t(K) * Cg);
    gw[t] = from_f32<T>(acc[co * Kp + int64_t(k) * Cg + cl]);
}

struct SampleArgs {
    const void *xt;         // image n, NHWC (the gather's copy), dtype
    const void *off;        // image n, dtype
    const void *msk;        // image n, dtype
    const float *gcol;      // [G][P][Kp], column k*Cg + c' (tap-major)
    float *gxt;             // image n's grad_x, NHWC, fp32 (atomic adds)
    void *goff, *gmask;     // image n, dtype
    int C, H, W, Wo, P, K, kw, Cg, Cdg, DG, Kp;
    int sh, sw, ph, pw, dh, dw;
    int team_shift;         // lanes per (offset group, tap, pixel): 1 << team_shift (<= 64)
};

// Sampling geometry of (offset group q, tap k, output pixel p) for the
// backward: the cell floor() selects, its fractions, which corners lie on
// the image, and whether the sample has derivatives at all (inside the open
// window (-1, H) x (-1, W), finite coordinate).
struct BwdTaps {
    bool live;
    bool r0, r1, c0, c1;
    int y0, x0;
    float ay, ax;
};

__device__ __forceinline__ BwdTaps bwd_taps(float oh, float ow, int ho, int wo, int i, int j,
                                            int H, int W, int sh, int sw, int ph, int pw, int dh,
                                            int dw)
{
    BwdTaps t{};
    const float lim = 33554432.0f;                // 2^25: certainly off any valid image
    if (!(fabsf(oh) <= lim && fabsf(ow) <= lim))
        return t;
    const float fh = floorf(oh), fw = floorf(ow);
    t.ay = oh - fh;                               // fractions (the anchor is an integer)
    t.ax = ow - fw;
    t.y0 = ho * sh - ph + i * dh + int(fh);
    t.x0 = wo * sw - pw + j * dw + int(fw);
    // inside the open window (-1, H) x (-1, W): h > -1 is y0 >= 0, or
    // y0 == -1 with a nonzero fraction; h < H is y0 <= H-1 (same for w)
    t.live = (t.y0 >= 0 || (t.y0 == -1 && t.ay > 0.0f)) && t.y0 < H &&
             (t.x0 >= 0 || (t.x0 == -1 && t.ax > 0.0f)) && t.x0 < W;
    t.r0 = t.y0 >= 0;
    t.r1 = t.y0 + 1 < H;
    t.c0 = t.x0 >= 0;
    t.c1 = t.x0 + 1 < W;
    return t;
}

// A team of lanes per (offset group q, tap k, pixel p) of one image, its
// lanes spread over q's channels: the corner reads of x, the column
// gradients and (ATOMIC_X) the atomic adds into grad_x are contiguous across
// the team (channels-last), and the team reduces its mask and offset
// gradients with wave shuffles.  Without ATOMIC_X, grad_x is left to the
// binned gather (bin_corners_kernel, gather_gx_kernel).
template <typename T, bool ATOMIC_X>
__global__ __launch_bounds__(256) void sample_grad_kernel(SampleArgs a)
{
    const T *xt = static_cast<const T *>(a.xt);
    const T *offp = static_cast<const T *>(a.off);
    const T *mskp = static_cast<const T *>(a.msk);
    const int TS = 1 << a.team_shift;
    const int64_t gt = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t item = gt >> a.team_shift;
    const int lane = int(gt & (TS - 1));
    const bool live = item < int64_t(a.DG) * a.K * a.P;
    float gm = 0.0f, gh = 0.0f, gw = 0.0f, m = 0.0f;
    int64_t ohi = 0, mi = 0;
    if (live) {
        const int p = int(item % a.P);
        const int k = int((item / a.P) % a.K);
        const int q = int(item / (int64_t(a.P) * a.K));
        const int ho = p / a.Wo, wo = p - (p / a.Wo) * a.Wo;
        const int i = k / a.kw, j = k - (k / a.kw) * a.kw;
        ohi = (int64_t(q) * 2 * a.K + 2 * k) * a.P + p;
        const float oh = to_f32(offp[ohi]), ow = to_f32(offp[ohi + a.P]);
        mi = (int64_t(q) * a.K + k) * a.P + p;
        m = to_f32(mskp[mi]);
        const float lim = 33554432.0f;            // 2^25: certainly off any valid image
        if (fabsf(oh) <= lim && fabsf(ow) <= lim) {
            const float fh = floorf(oh), fw = floorf(ow);
            const float ay = oh - fh, ax = ow - fw;   // fractions (the anchor is an integer)
            const int y0 = ho * a.sh - a.ph + i * a.dh + int(fh);
            const int x0 = wo * a.sw - a.pw + j * a.dw + int(fw);
            // inside the open window (-1, H) x (-1, W): h > -1 is y0 >= 0, or
            // y0 == -1 with a nonzero fraction; h < H is y0 <= H-1 (same for w)
            if ((y0 >= 0 || (y0 == -1 && ay > 0.0f)) && y0 < a.H &&
                (x0 >= 0 || (x0 == -1 && ax > 0.0f)) && x0 < a.W) {
                const bool r0 = y0 >= 0, r1 = y0 + 1 < a.H, c0 = x0 >= 0, c1 = x0 + 1 < a.W;
                const float w00 = (1.0f - ay) * (1.0f - ax), w01 = (1.0f - ay) * ax;
                const float w10 = ay * (1.0f - ax), w11 = ay * ax;
                const int64_t e00 = (int64_t(y0) * a.W + x0) * a.C;   // NHWC entry of (y0, x0)
                const int64_t e01 = e00 + a.C, e10 = e00 + int64_t(a.W) * a.C, e11 = e10 + a.C;
                for (int c = q * a.Cdg + lane; c < (q + 1) * a.Cdg; c += TS) {
                    const int grp = c / a.Cg, cl = c - grp * a.Cg;
                    const float gc =
                        a.gcol[(int64_t(grp) * a.P + p) * a.Kp + int64_t(k) * a.Cg + cl];
                    const float v00 = (r0 && c0) ? to_f32(xt[e00 + c]) : 0.0f;
                    const float v01 = (r0 && c1) ? to_f32(xt[e01 + c]) : 0.0f;
                    const float v10 = (r1 && c0) ? to_f32(xt[e10 + c]) : 0.0f;
                    const float v11 = (r1 && c1) ? to_f32(xt[e11 + c]) : 0.0f;
                    const float v = w00 * v00 + w01 * v01 + w10 * v10 + w11 * v11;
                    gm = fmaf(gc, v, gm);
                    gh = fmaf(gc, (1.0f - ax) * (v10 - v00) + ax * (v11 - v01), gh);
                    gw = fmaf(gc, (1.0f - ay) * (v01 - v00) + ay * (v11 - v10), gw);
                    if constexpr (ATOMIC_X) {
                        const float s = gc * m;
                        if (r0 && c0) atomicAdd(a.gxt + e00 + c, s * w00);
                        if (r0 && c1) atomicAdd(a.gxt + e01 + c, s * w01);
                        if (r1 && c0) atomicAdd(a.gxt + e10 + c, s * w10);
                        if (r1 && c1) atomicAdd(a.gxt + e11 + c, s * w11);
                    }
                }
            }
        }
    }
    // team reduction (teams are aligned groups of TS lanes within a wave)
    for (int d = TS >> 1; d >= 1; d >>= 1) {
        gm += __shfl_xor(gm, d, 64);
        gh += __shfl_xor(gh, d, 64);
        gw += __shfl_xor(gw, d, 64);
    }
    if (live && lane == 0) {
        static_cast<T *>(a.gmask)[mi] = from_f32<T>(gm);
        static_cast<T *>(a.goff)[ohi] = from_f32<T>(gh * m);
        static_cast<T *>(a.goff)[ohi + a.P] = from_f32<T>(gw * m);
    }
}

// Four consecutive channels of element type T at p (aligned to four
// elements) as floats.
template <typename T>
__device__ __forceinline__ float4 load4f(const T *p)
{
    if constexpr (sizeof(T) == 4) {
        return *reinterpret_cast<const float4 *>(p);
    } else {
        const uint2 r = *reinterpret_cast<const uint2 *>(p);
        T e[4];
        __builtin_memcpy(e, &r, 8);
        return make_float4(to_f32(e[0]), to_f32(e[1]), to_f32(e[2]), to_f32(e[3]));
    }
}

// The mask and offset gradients alone (grad_x by the binned gather), four
// channels a lane: one 16-byte column-gradient load and four corner loads
// of four channels per step.  Requires C/group and C/deformable_group to be
// multiples of 4.
template <typename T>
__global__ __launch_bounds__(256) void sample_grad_vec_kernel(SampleArgs a)
{
    const T *xt = static_cast<const T *>(a.xt);
    const T *offp = static_cast<const T *>(a.off);
    const T *mskp = static_cast<const T *>(a.msk);
    const int TS = 1 << a.team_shift;
    const int64_t gt = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t item = gt >> a.team_shift;
    const int lane = int(gt & (TS - 1));
    const bool live = item < int64_t(a.DG) * a.K * a.P;
    float gm = 0.0f, gh = 0.0f, gw = 0.0f, m = 0.0f;
    int64_t ohi = 0, mi = 0;
    if (live) {
        const int p = int(item % a.P);
        const int k = int((item / a.P) % a.K);
        const int q = int(item / (int64_t(a.P) * a.K));
        const int ho = p / a.Wo, wo = p - (p / a.Wo) * a.Wo;
        const int i = k / a.kw, j = k - (k / a.kw) * a.kw;
        ohi = (int64_t(q) * 2 * a.K + 2 * k) * a.P + p;
        mi = (int64_t(q) * a.K + k) * a.P + p;
        m = to_f32(mskp[mi]);
        const BwdTaps t = bwd_taps(to_f32(offp[ohi]), to_f32(offp[ohi + a.P]), ho, wo, i, j, a.H,
                                   a.W, a.sh, a.sw, a.ph, a.pw, a.dh, a.dw);
        if (t.live) {
            const float ay = t.ay, ax = t.ax;
            const float w00 = (1.0f - ay) * (1.0f - ax), w01 = (1.0f - ay) * ax;
            const float w10 = ay * (1.0f - ax), w11 = ay * ax;
            const int64_t e00 = (int64_t(t.y0) * a.W + t.x0) * a.C;   // NHWC entry of (y0, x0)
            const int64_t e01 = e00 + a.C, e10 = e00 + int64_t(a.W) * a.C, e11 = e10 + a.C;
            const float4 z = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            for (int c = q * a.Cdg + lane * 4; c < (q + 1) * a.Cdg; c += TS * 4) {
                const int grp = c / a.Cg, cl = c - grp * a.Cg;
                const float4 g4 = *reinterpret_cast<const float4 *>(
                    a.gcol + (int64_t(grp) * a.P + p) * a.Kp + int64_t(k) * a.Cg + cl);
                const float4 a00 = (t.r0 && t.c0) ? load4f(xt + e00 + c) : z;
                const float4 a01 = (t.r0 && t.c1) ? load4f(xt + e01 + c) : z;
                const float4 a10 = (t.r1 && t.c0) ? load4f(xt + e10 + c) : z;
                const float4 a11 = (t.r1 && t.c1) ? load4f(xt + e11 + c) : z;
                const float gcv[4] = {g4.x, g4.y, g4.z, g4.w};
                const float v00[4] = {a00.x, a00.y, a00.z, a00.w};
                const float v01[4] = {a01.x, a01.y, a01.z, a01.w};
                const float v10[4] = {a10.x, a10.y, a10.z, a10.w};
                const float v11[4] = {a11.x, a11.y, a11.z, a11.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float v = w00 * v00[u] + w01 * v01[u] + w10 * v10[u] + w11 * v11[u];
                    gm = fmaf(gcv[u], v, gm);
                    gh = fmaf(gcv[u], (1.0f - ax) * (v10[u] - v00[u]) + ax * (v11[u] - v01[u]),
                              gh);
                    gw = fmaf(gcv[u], (1.0f - ay) * (v01[u] - v00[u]) + ay * (v11[u] - v10[u]),
                              gw);
                }
            }
        }
    }
    for (int d = TS >> 1; d >= 1; d >>= 1) {
        gm += __shfl_xor(gm, d, 64);
        gh += __shfl_xor(gh, d, 64);
        gw += __shfl_xor(gw, d, 64);
    }
    if (live && lane == 0) {
        static_cast<T *>(a.gmask)[mi] = from_f32<T>(gm);
        static_cast<T *>(a.goff)[ohi] = from_f32<T>(gh * m);
        static_cast<T *>(a.goff)[ohi + a.P] = from_f32<T>(gw * m);
    }
}

// grad_x without atomics: every on-image corner of every live sample is an
// entry (source column k*P + p, weight mask * corner weight) in the bucket of
// its (offset group, input pixel) cell.  A counting pass (FILL = false)
// counts the entries of each cell, a scan turns the counts into bucket
// starts, and a fill pass (FILL = true) places each entry at
// start + (count after a decrement), which also leaves every count at zero
// for the next image.  Then one thread per (cell, channel) sums its bucket:
//   grad_x[c][cell] = sum over entries (k, p, w) of w * gcol(c, k, p).
struct BinArgs {
    const void *off;        // image n, dtype
    const void *msk;        // image n, dtype
    uint32_t *cnt;          // [DG][H*W]: zero before the counting pass and after the fill
    const uint32_t *start;  // [DG][H*W] + 1: bucket starts
    uint2 *entries;         // {k*P + p, weight bits}
    int H, W, Wo, P, K, kw, DG;
    int sh, sw, ph, pw, dh, dw;
};

template <typename T, bool FILL>
__global__ __launch_bounds__(256) void bin_corners_kernel(BinArgs a)
{
    const int64_t item = int64_t(blockIdx.x) * 256 + threadIdx.x;   // (q, k, p)
    if (item >= int64_t(a.DG) * a.K * a.P)
        return;
    const int p = int(item % a.P);
    const int k = int((item / a.P) % a.K);
    const int q = int(item / (int64_t(a.P) * a.K));
    const int ho = p / a.Wo, wo = p - (p / a.Wo) * a.Wo;
    const int i = k / a.kw, j = k - (k / a.kw) * a.kw;
    const T *offp = static_cast<const T *>(a.off);
    const int64_t ohi = (int64_t(q) * 2 * a.K + 2 * k) * a.P + p;
    const BwdTaps t = bwd_taps(to_f32(offp[ohi]), to_f32(offp[ohi + a.P]), ho, wo, i, j, a.H,
                               a.W, a.sh, a.sw, a.ph, a.pw, a.dh, a.dw);
    if (!t.live)
        return;
    const float m = to_f32(static_cast<const T *>(a.msk)[(int64_t(q) * a.K + k) * a.P + p]);
    const float wt[4] = {(1.0f - t.ay) * (1.0f - t.ax), (1.0f - t.ay) * t.ax,
                         t.ay * (1.0f - t.ax), t.ay * t.ax};
    const bool on[4] = {t.r0 && t.c0, t.r0 && t.c1, t.r1 && t.c0, t.r1 && t.c1};
    const int64_t base = int64_t(q) * a.H * a.W;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        if (!on[s])
            continue;
        const int64_t cell = base + int64_t(t.y0 + (s >> 1)) * a.W + t.x0 + (s & 1);
        if constexpr (!FILL) {
            atomicAdd(a.cnt + cell, 1u);
        } else {
            const uint32_t slot = atomicSub(a.cnt + cell, 1u) - 1u;
            a.entries[a.start[cell] + slot] =
                make_uint2(uint32_t(k * a.P + p), __float_as_uint(m * wt[s]));
        }
    }
}

// Exclusive scan of n counts into start[0..n] (start[n] = total), in three
// launches: per 4096-element block (1024 threads, 4 elements each) the local
// scan and the block's total; the scan of the block totals (one workgroup,
// at most 4096 blocks); the block offsets added.
constexpr int kScanBlock = 4096;

__device__ __forceinline__ uint32_t block_scan_1024(uint32_t v, uint32_t *sh, uint32_t *total)
{
    // inclusive scan within the wave, then across the 16 waves
    const int lane = int(threadIdx.x) & 63, wave = int(threadIdx.x) >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t u = __shfl_up(v, d, 64);
        if (lane >= d)
            v += u;
    }
    if (lane == 63)
        sh[wave] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t run = 0;
        for (int w = 0; w < 16; ++w) {
            const uint32_t x = sh[w];
            sh[w] = run;
            run += x;
        }
        sh[16] = run;
    }
    __syncthreads();
    const uint32_t r = v + sh[wave];
    *total = sh[16];
    __syncthreads();
    return r;                                    // inclusive
}

__global__ __launch_bounds__(1024) void scan_blocks_kernel(const uint32_t *__restrict__ cnt,
                                                           uint32_t *__restrict__ start,
                                                           uint32_t *__restrict__ bsum,
                                                           int64_t n)
{
    __shared__ uint32_t sh[17];
    const int64_t i0 = int64_t(blockIdx.x) * kScanBlock + int64_t(threadIdx.x) * 4;
    uint32_t v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        v[e] = i0 + e < n ? cnt[i0 + e] : 0u;
    const uint32_t mine = v[0] + v[1] + v[2] + v[3];
    uint32_t total;
    const uint32_t incl = block_scan_1024(mine, sh, &total);
    uint32_t run = incl - mine;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (i0 + e < n)
            start[i0 + e] = run;
        run += v[e];
    }
    if (threadIdx.x == 0)
        bsum[blockIdx.x] = total;
}

__global__ __launch_bounds__(1024) void scan_sums_kernel(uint32_t *__restrict__ bsum, int nb,
                                                         uint32_t *__restrict__ last)
{
    __shared__ uint32_t sh[17];
    uint32_t v[4];
    const int i0 = int(threadIdx.x) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        v[e] = i0 + e < nb ? bsum[i0 + e] : 0u;
    const uint32_t mine = v[0] + v[1] + v[2] + v[3];
    uint32_t total;
    const uint32_t incl = block_scan_1024(mine, sh, &total);
    uint32_t run = incl - mine;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (i0 + e < nb)
            bsum[i0 + e] = run;
        run += v[e];
    }
    if (threadIdx.x == 0)
        *last = total;
}

__global__ __launch_bounds__(256) void scan_add_kernel(uint32_t *__restrict__ start,
                                                       const uint32_t *__restrict__ bsum,
                                                       int64_t n)
{
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i < n)
        start[i] += bsum[i / kScanBlock];
}

struct GatherGxArgs {
    const uint32_t *start;  // [DG][H*W] + 1
    const uint2 *entries;
    const float *gcol;      // [G][P][Kp], column k*Cg + c'
    float *gxt;             // image n's grad_x, NHWC, fp32 (every element written)
    int C, HW, P, Cg, Cdg, Kp, DG;
};

// One wave per (offset group q, input cell): its lanes run over q's
// channels, V consecutive channels a lane (one 16-byte column-gradient load
// when V = 4), in slices of 64*V.  The bucket's entries are read 64 at a
// time, one per lane, and handed to the whole wave one by one (readlane), so
// that the column-gradient loads of several entries are in flight together.
template <int V>
__global__ __launch_bounds__(256) void gather_gx_kernel(GatherGxArgs a)
{
    const int64_t wv = (int64_t(blockIdx.x) * 256 + threadIdx.x) >> 6;   // (q, cell)
    const int lane = int(threadIdx.x) & 63;
    if (wv >= int64_t(a.DG) * a.HW)
        return;
    const int q = int(wv / a.HW);
    const int64_t cell = wv - int64_t(q) * a.HW;
    const uint32_t e0 = a.start[wv], e1 = a.start[wv + 1];
    for (int cs = 0; cs < a.Cdg; cs += 64 * V) {
        const int cq = cs + lane * V;               // the lane's first channel within q
        const bool on = cq < a.Cdg;
        const int c = q * a.Cdg + (on ? cq : 0);
        const int grp = c / a.Cg, cl = c - grp * a.Cg;
        const float *gc = a.gcol + int64_t(grp) * a.P * a.Kp + cl;
        float acc[V];
#pragma unroll
        for (int v = 0; v < V; ++v)
            acc[v] = 0.0f;
        for (uint32_t eb = e0; eb < e1; eb += 64) {
            const int n = int(min(64u, e1 - eb));
            const uint2 my = lane < n ? a.entries[eb + lane] : make_uint2(0u, 0u);
#pragma unroll 4
            for (int j = 0; j < n; ++j) {
                const int kp = __builtin_amdgcn_readlane(int(my.x), j);
                const float w = __uint_as_float(uint32_t(__builtin_amdgcn_readlane(int(my.y), j)));
                const int k = kp / a.P, p = kp - k * a.P;
                const float *src = gc + int64_t(p) * a.Kp + int64_t(k) * a.Cg;
                if (on) {
                    if constexpr (V == 4) {
                        const float4 g4 = *reinterpret_cast<const float4 *>(src);
                        acc[0] = fmaf(w, g4.x, acc[0]);
                        acc[1] = fmaf(w, g4.y, acc[1]);
                        acc[2] = fmaf(w, g4.z, acc[2]);
                        acc[3] = fmaf(w, g4.w, acc[3]);
                    } else {
                        acc[0] = fmaf(w, *src, acc[0]);
                    }
                }
            }
        }
        if (on) {
            float *dst = a.gxt + cell * a.C + c;
            if constexpr (V == 4)
                *reinterpret_cast<float4 *>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
            else
                *dst = acc[0];
        }
    }
}

// acc[t] += sum over s < S of part[s * n + t] (the pixel chunks' partial
// weight gradients).
__global__ __launch_bounds__(256) void reduce_parts_kernel(const float *__restrict__ part,
                                                           float *__restrict__ acc, int64_t n,
                                                           int S)
{
    const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (t >= n)
        return;
    float v = acc[t];
    for (int s = 0; s < S; ++s)
        v += part[int64_t(s) * n + t];
    acc[t] = v;
}

template <typename T>
__global__ __launch_bounds__(256) void convert_kernel(const float *__restrict__ src,
                                                      T *__restrict__ dst, int64_t n)
{
    const int64_t stride = int64_t(gridDim.x) * 256;
    for (int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x; t < n; t += stride)
        dst[t] = from_f32<T>(src[t]);
}

}  // namespace

BackwardLayout backward_layout(const Problem &p)
{
    BackwardLayout l{};
    auto al = [](size_t b) { return (b + kAlign - 1) / kAlign * kAlign; };
    l.Kp = (p.Kg + 63) / 64 * 64;
    l.wpack_off = 0;
    l.xt_off = l.wpack_off + al(size_t(p.Co * l.Kp) * p.elem);
    l.gxt_off = l.xt_off + al(size_t(p.C * p.H * p.W) * p.elem);
    l.gxn_off = l.gxt_off + al(size_t(p.C * p.H * p.W) * 4);
    l.col_off = l.gxn_off + (p.dtype == MDCN_F32 ? 0 : al(size_t(p.C * p.H * p.W) * 4));
    l.gcol_off = l.col_off + al(size_t(p.G * p.P * l.Kp) * 4);
    l.wacc_off = l.gcol_off + al(size_t(p.G * p.P * l.Kp) * 4);
    l.goT_off = l.wacc_off + al(size_t(p.Co * l.Kp) * 4);
    l.wT_off = l.goT_off;
    l.bytes = l.goT_off;
    // the column gradient on the MFMA GEMM (fp32, one group, rows of Co
    // floats that are whole 128-byte lines): grad_out and the packed weight
    // transposed so that both operands run along the output channels
    l.mfma_col = p.dtype == MDCN_F32 && p.G == 1 && p.Co % 32 == 0 && p.P >= 1;
    // the weight gradient on the MFMA GEMM as well: the image's pixels split
    // into S chunks of Pc (a multiple of 32 floats = whole 128-byte K steps,
    // at most 1024; MDCN_BWD_PC_MAX=<floats> lowers the cap) that run as the
    // GEMM's groups; the columns gathered transposed, [Kp][P] (into the
    // column-gradient buffer, written later), and the S partial [Co][Kp]
    // results (in the column buffer).  (OCDNet-like stage, P = 25600:
    // Pc = 1024 takes 270 us, 512 307 us, 640-1600 331-411 us.)
    l.wsplit = 0;
    if (l.mfma_col && p.P % 32 == 0) {
        int64_t dmax = 32;
        if (const char *env = std::getenv("MDCN_BWD_PC_MAX")) {
            const int64_t v = std::atoll(env) / 32;
            if (v >= 1 && v <= 256)
                dmax = v;
        }
        for (int64_t d = dmax; d >= 1; --d) {
            const int64_t pc = 32 * d;
            if (p.P % pc == 0 && (p.P / pc) * p.Co <= p.P) {
                l.wsplit = p.P / pc;
                break;
            }
        }
    }
    if (l.mfma_col) {
        l.wT_off = l.goT_off + al(size_t(p.P * p.Co) * 4);
        l.bytes = l.wT_off + al(size_t(l.Kp * p.Co) * 4);
    }
    // grad_x binned by input cell (no atomics on grad_x): counts, bucket
    // starts, scan block totals and up to four entries per sample, after
    // everything else (counts zeroed once per call, left zero by each image)
    const int64_t cells = p.DG * p.H * p.W;
    const int64_t entries = 4 * p.DG * p.K * p.P;
    l.binned = cells > 0 && cells <= int64_t(kScanBlock) * kScanBlock &&
               entries < (int64_t(1) << 32) && p.K * p.P < (int64_t(1) << 32);
    if (l.binned) {
        l.bins_off = l.bytes;
        l.cnt_off = 0;
        l.start_off = l.cnt_off + al(size_t(cells) * 4);
        l.bsum_off = l.start_off + al(size_t(cells + 1) * 4);
        l.entries_off = l.bsum_off + al(size_t(kScanBlock + 1) * 4);
        l.bytes = l.bins_off + l.entries_off + al(size_t(entries) * 8);
    }
    return l;
}

hipError_t launch_bwd_fill_zero(float *ptr, int64_t n, hipStream_t s)
{
    if (n <= 0)
        return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 65536);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, ptr, n);
    return hipGetLastError();
}

namespace {

template <typename T>
__global__ __launch_bounds__(256) void fill_zero_t_kernel(T *p, int64_t n)
{
    const int64_t stride = int64_t(gridDim.x) * 256;
    for (int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x; t < n; t += stride)
        p[t] = T(0);
}

template <typename T>
hipError_t fill_zero_t(void *ptr, int64_t n, hipStream_t s)
{
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 65536);
    hipLaunchKernelGGL((fill_zero_t_kernel<T>), dim3(unsigned(blocks)), dim3(256), 0, s,
                       static_cast<T *>(ptr), n);
    return hipGetLastError();
}

template <typename T>
hipError_t bias_t(const Problem &p, const void *g, void *gb, hipStream_t s)
{
    hipLaunchKernelGGL((bias_grad_kernel<T>), dim3(unsigned(p.Co)), dim3(1024), 0, s,
                       static_cast<const T *>(g), static_cast<T *>(gb), int(p.N), int(p.Co),
                       int(p.P));
    return hipGetLastError();
}

template <typename T>
hipError_t weight_gemm_t(const Problem &p, const BackwardLayout &l, const void *g_n,
                         const float *col, float *acc, hipStream_t s)
{
    // split the pixels so that the launch has about 1024 workgroups
    const int64_t tiles = ((p.Mg + kBT - 1) / kBT) * ((p.Kg + kBT - 1) / kBT);
    int64_t splits = std::max<int64_t>(1, std::min<int64_t>(1024 / std::max<int64_t>(tiles, 1),
                                                            (p.P + 255) / 256));
    const int64_t lchunk = ((p.P + splits - 1) / splits + kBL - 1) / kBL * kBL;
    splits = (p.P + lchunk - 1) / lchunk;
    for (int64_t grp = 0; grp < p.G; ++grp) {
        GemmDesc d{};
        d.A = static_cast<const T *>(g_n) + grp * p.Mg * p.P;  d.ai = p.P;  d.al = 1;
        d.B = col + grp * p.P * l.Kp;                          d.bl = l.Kp; d.bj = 1;
        d.C = acc + grp * p.Mg * l.Kp;                         d.ci = l.Kp; d.cj = 1;
        d.M = int(p.Mg); d.N = int(p.Kg); d.L = int(p.P); d.lchunk = int(lchunk);
        d.atomic = 1;
        hipError_t e = run_gemm<T, float>(d, int(splits), s);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

template <typename T>
hipError_t col_gemm_t(const Problem &p, const BackwardLayout &l, const void *wpack,
                      const void *g_n, float *gcol, hipStream_t s)
{
    for (int64_t grp = 0; grp < p.G; ++grp) {
        GemmDesc d{};
        d.A = static_cast<const T *>(g_n) + grp * p.Mg * p.P;    d.ai = 1;    d.al = p.P;
        d.B = static_cast<const T *>(wpack) + grp * p.Mg * l.Kp; d.bl = l.Kp; d.bj = 1;
        d.C = gcol + grp * p.P * l.Kp;                           d.ci = l.Kp; d.cj = 1;
        d.M = int(p.P); d.N = int(p.Kg); d.L = int(p.Mg); d.lchunk = int(p.Mg);
        d.atomic = 0;
        hipError_t e = run_gemm<T, T>(d, 1, s);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

template <typename T>
hipError_t sample_t(const Problem &p, const SampleArgs &a, int64_t threads, bool atomic_x,
                    hipStream_t s)
{
    if (!atomic_x && p.Cg % 4 == 0 && p.Cdg % 4 == 0) {
        // four channels a lane: a team of at most 64 lanes covers Cdg/4 slots
        SampleArgs v = a;
        int shift = 0;
        while ((1 << shift) * 4 < p.Cdg && shift < 6)
            ++shift;
        v.team_shift = shift;
        const int64_t n = (p.DG * p.K * p.P) << shift;
        hipLaunchKernelGGL((sample_grad_vec_kernel<T>), dim3(unsigned((n + 255) / 256)),
                           dim3(256), 0, s, v);
        return hipGetLastError();
    }
    if (atomic_x)
        hipLaunchKernelGGL((sample_grad_kernel<T, true>), dim3(unsigned((threads + 255) / 256)),
                           dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((sample_grad_kernel<T, false>), dim3(unsigned((threads + 255) / 256)),
                           dim3(256), 0, s, a);
    return hipGetLastError();
}

template <typename T>
hipError_t bin_t(const BinArgs &b, int64_t items, bool fill, hipStream_t s)
{
    if (fill)
        hipLaunchKernelGGL((bin_corners_kernel<T, true>), dim3(unsigned((items + 255) / 256)),
                           dim3(256), 0, s, b);
    else
        hipLaunchKernelGGL((bin_corners_kernel<T, false>), dim3(unsigned((items + 255) / 256)),
                           dim3(256), 0, s, b);
    return hipGetLastError();
}

template <typename T>
hipError_t convert_t(const float *src, void *dst, int64_t n, hipStream_t s)
{
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 65536);
    hipLaunchKernelGGL((convert_kernel<T>), dim3(unsigned(blocks)), dim3(256), 0, s, src,
                       static_cast<T *>(dst), n);
    return hipGetLastError();
}

template <typename T>
hipError_t weight_out_t(const Problem &p, const BackwardLayout &l, const float *acc, void *gw,
                        hipStream_t s)
{
    const int64_t total = p.Co * p.Cg * p.K;
    hipLaunchKernelGGL((weight_out_kernel<T>), dim3(unsigned((total + 255) / 256)), dim3(256), 0,
                       s, acc, static_cast<T *>(gw), int(p.Co), int(p.Cg), int(p.K), int(l.Kp));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bias(const Problem &p, const void *g, void *gb, hipStream_t s)
{
    if (p.Co == 0)
        return hipSuccess;
    switch (p.dtype) {
    case MDCN_F32: return bias_t<float>(p, g, gb, s);
    case MDCN_F16: return bias_t<half_t>(p, g, gb, s);
    case MDCN_BF16: return bias_t<bf16_t>(p, g, gb, s);
    }
    return hipErrorInvalidValue;
}

// acc[g][m][kk] += sum_p g_n[g*Mg + m][p] * col[g][p][kk], all groups.
hipError_t launch_bwd_weight_gemm(const Problem &p, const BackwardLayout &l, const void *g_n,
                                  const float *col, float *acc, hipStream_t s)
{
    switch (p.dtype) {
    case MDCN_F32: return weight_gemm_t<float>(p, l, g_n, col, acc, s);
    case MDCN_F16: return weight_gemm_t<half_t>(p, l, g_n, col, acc, s);
    case MDCN_BF16: return weight_gemm_t<bf16_t>(p, l, g_n, col, acc, s);
    }
    return hipErrorInvalidValue;
}

// gcol[g][p][kk] = sum_m g_n[g*Mg + m][p] * wpack[g][m][kk] (kk tap-major).
hipError_t launch_bwd_col_gemm(const Problem &p, const BackwardLayout &l, const void *wpack,
                               const void *g_n, float *gcol, hipStream_t s)
{
    switch (p.dtype) {
    case MDCN_F32: return col_gemm_t<float>(p, l, wpack, g_n, gcol, s);
    case MDCN_F16: return col_gemm_t<half_t>(p, l, wpack, g_n, gcol, s);
    case MDCN_BF16: return col_gemm_t<bf16_t>(p, l, wpack, g_n, gcol, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_sample(const Problem &p, const BackwardLayout &l, const void *xt_n,
                             const void *off_n, const void *msk_n, const float *gcol,
                             float *gxt_n, void *goff_n, void *gmask_n, char *bins,
                             hipStream_t s)
{
    SampleArgs a;
    a.xt = xt_n; a.off = off_n; a.msk = msk_n; a.gcol = gcol; a.gxt = gxt_n;
    a.goff = goff_n; a.gmask = gmask_n;
    a.C = int(p.C); a.H = int(p.H); a.W = int(p.W); a.Wo = int(p.Wo); a.P = int(p.P);
    a.K = int(p.K); a.kw = int(p.kw); a.Cg = int(p.Cg); a.Cdg = int(p.Cdg); a.DG = int(p.DG);
    a.Kp = int(l.Kp);
    a.sh = int(p.sh); a.sw = int(p.sw); a.ph = int(p.ph); a.pw = int(p.pw);
    a.dh = int(p.dh); a.dw = int(p.dw);
    int shift = 0;                        // team: the offset group's channels, at most 64 lanes
    while ((1 << shift) < p.Cdg && shift < 6)
        ++shift;
    a.team_shift = shift;
    const int64_t items = p.DG * p.K * p.P;
    const int64_t threads = items << shift;
    if (threads == 0)
        return hipSuccess;
    if ((threads + 255) / 256 > 0x7fffffff)
        return hipErrorInvalidValue;
    hipError_t e = hipSuccess;
    if (l.binned) {
        const int64_t cells = p.DG * p.H * p.W;
        BinArgs b;
        b.off = off_n; b.msk = msk_n;
        b.cnt = reinterpret_cast<uint32_t *>(bins + l.cnt_off);
        b.start = reinterpret_cast<const uint32_t *>(bins + l.start_off);
        b.entries = reinterpret_cast<uint2 *>(bins + l.entries_off);
        b.H = int(p.H); b.W = int(p.W); b.Wo = int(p.Wo); b.P = int(p.P); b.K = int(p.K);
        b.kw = int(p.kw); b.DG = int(p.DG);
        b.sh = int(p.sh); b.sw = int(p.sw); b.ph = int(p.ph); b.pw = int(p.pw);
        b.dh = int(p.dh); b.dw = int(p.dw);
        uint32_t *start = reinterpret_cast<uint32_t *>(bins + l.start_off);
        uint32_t *bsum = reinterpret_cast<uint32_t *>(bins + l.bsum_off);
        const int nb = int((cells + kScanBlock - 1) / kScanBlock);
        auto bin = [&](bool fill) {
            switch (p.dtype) {
            case MDCN_F32: return bin_t<float>(b, items, fill, s);
            case MDCN_F16: return bin_t<half_t>(b, items, fill, s);
            case MDCN_BF16: return bin_t<bf16_t>(b, items, fill, s);
            }
            return hipErrorInvalidValue;
        };
        e = bin(false);
        if (e == hipSuccess) {
            hipLaunchKernelGGL(scan_blocks_kernel, dim3(unsigned(nb)), dim3(1024), 0, s, b.cnt,
                               start, bsum, cells);
            hipLaunchKernelGGL(scan_sums_kernel, dim3(1), dim3(1024), 0, s, bsum, nb,
                               start + cells);
            hipLaunchKernelGGL(scan_add_kernel, dim3(unsigned((cells + 255) / 256)), dim3(256),
                               0, s, start, bsum, cells);
            e = hipGetLastError();
        }
        if (e == hipSuccess)
            e = bin(true);
        if (e == hipSuccess) {
            GatherGxArgs g{start, b.entries, gcol, gxt_n, int(p.C), int(p.H * p.W), int(p.P),
                           int(p.Cg), int(p.Cdg), int(l.Kp), int(p.DG)};
            const int64_t waves = cells;           // one per (offset group, cell)
            const dim3 grid(unsigned((waves + 3) / 4));
            if (p.Cg % 4 == 0 && p.Cdg % 4 == 0 && l.Kp % 4 == 0)
                hipLaunchKernelGGL(gather_gx_kernel<4>, grid, dim3(256), 0, s, g);
            else
                hipLaunchKernelGGL(gather_gx_kernel<1>, grid, dim3(256), 0, s, g);
            e = hipGetLastError();
        }
        if (e != hipSuccess)
            return e;
    }
    switch (p.dtype) {
    case MDCN_F32: return sample_t<float>(p, a, threads, !l.binned, s);
    case MDCN_F16: return sample_t<half_t>(p, a, threads, !l.binned, s);
    case MDCN_BF16: return sample_t<bf16_t>(p, a, threads, !l.binned, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_fill_zero_dtype(const Problem &p, void *ptr, int64_t n, hipStream_t s)
{
    if (n <= 0)
        return hipSuccess;
    switch (p.dtype) {
    case MDCN_F32: return fill_zero_t<float>(ptr, n, s);
    case MDCN_F16: return fill_zero_t<half_t>(ptr, n, s);
    case MDCN_BF16: return fill_zero_t<bf16_t>(ptr, n, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_convert(const Problem &p, const float *src, void *dst, int64_t n,
                              hipStream_t s)
{
    if (n <= 0)
        return hipSuccess;
    switch (p.dtype) {
    case MDCN_F32: return convert_t<float>(src, dst, n, s);
    case MDCN_F16: return convert_t<half_t>(src, dst, n, s);
    case MDCN_BF16: return convert_t<bf16_t>(src, dst, n, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_reduce_parts(const float *part, float *acc, int64_t n, int S,
                                   hipStream_t s)
{
    if (n <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(reduce_parts_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, part,
                       acc, n, S);
    return hipGetLastError();
}

hipError_t launch_bwd_weight_out(const Problem &p, const BackwardLayout &l, const float *acc,
                                 void *gw, hipStream_t s)
{
    if (p.Co * p.Cg * p.K == 0)
        return hipSuccess;
    switch (p.dtype) {
    case MDCN_F32: return weight_out_t<float>(p, l, acc, gw, s);
    case MDCN_F16: return weight_out_t<half_t>(p, l, acc, gw, s);
    case MDCN_BF16: return weight_out_t<bf16_t>(p, l, acc, gw, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace mdcn
