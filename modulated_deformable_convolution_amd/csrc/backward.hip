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

// A team of lanes per (offset group q, tap k, pixel p) of one image, its
// lanes spread over q's channels: the corner reads of x, the column
// gradients and the atomic adds into grad_x are contiguous across the team
// (channels-last), and the team reduces its mask and offset gradients with
// wave shuffles.
template <typename T>
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
                    const float s = gc * m;
                    if (r0 && c0) atomicAdd(a.gxt + e00 + c, s * w00);
                    if (r0 && c1) atomicAdd(a.gxt + e01 + c, s * w01);
                    if (r1 && c0) atomicAdd(a.gxt + e10 + c, s * w10);
                    if (r1 && c1) atomicAdd(a.gxt + e11 + c, s * w11);
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
    // at most 512) that run as the GEMM's groups; the columns transposed to
    // [Kp][P] (in the column-gradient buffer, written later) and the S
    // partial [Co][Kp] results (in the column buffer, consumed by then)
    l.wsplit = 0;
    if (l.mfma_col && p.P % 32 == 0) {
        for (int64_t d = 16; d >= 1; --d) {
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
hipError_t sample_t(const Problem &p, const SampleArgs &a, int64_t threads, hipStream_t s)
{
    hipLaunchKernelGGL((sample_grad_kernel<T>), dim3(unsigned((threads + 255) / 256)), dim3(256),
                       0, s, a);
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
                             float *gxt_n, void *goff_n, void *gmask_n, hipStream_t s)
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
    const int64_t threads = (p.DG * p.K * p.P) << shift;
    if (threads == 0)
        return hipSuccess;
    if ((threads + 255) / 256 > 0x7fffffff)
        return hipErrorInvalidValue;
    switch (p.dtype) {
    case MDCN_F32: return sample_t<float>(p, a, threads, s);
    case MDCN_F16: return sample_t<half_t>(p, a, threads, s);
    case MDCN_BF16: return sample_t<bf16_t>(p, a, threads, s);
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
