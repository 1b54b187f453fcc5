// prep.hip -- layout kernels: x to channels-last (NHWC) or to 8-channel
// blocks ([C/8][H][W][8] per image), and the weight repacked in the order a
// path's contraction walks it (for the FP8 path also scaled and rounded to
// E4M3).  Apart from that rounding they only move data.
#include <algorithm>

#include "device_common.h"
#include "launch.h"
#include "transpose.h"

namespace mdcn {

namespace {

constexpr int kTile = 64;

// Destination of (channel c, pixel p) of one image: NHWC, or 8-channel
// blocks (block c/8 is a plane of HW x 8 channels).
template <bool BLK>
__device__ __forceinline__ size_t dst_index(int c, int p, int C, int HW)
{
    return BLK ? (size_t(c >> 3) * HW + p) * 8 + (c & 7) : size_t(p) * C + c;
}

// One 64 (channels) x 64 (pixels) tile through LDS per workgroup: tile
// (bx, by) of image bz.
template <typename T, bool BLK>
__device__ __forceinline__ void transpose_tile(const T *__restrict__ x, T *__restrict__ xt,
                                               int C, int HW, int bx, int by, int bz,
                                               T (*tile)[kTile + 1])
{
    const int p0 = bx * kTile;
    const int c0 = by * kTile;
    const size_t img = size_t(bz) * size_t(C) * size_t(HW);
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
            dst[dst_index<BLK>(c, p, C, HW)] = tile[tx][r];
    }
}

template <typename T, bool BLK>
__global__ __launch_bounds__(256) void to_nhwc_kernel(const T *__restrict__ x, T *__restrict__ xt,
                                                      int C, int HW)
{
    __shared__ T tile[kTile][kTile + 1];
    transpose_tile<T, BLK>(x, xt, C, HW, blockIdx.x, blockIdx.y, blockIdx.z, tile);
}

// Workgroups of the register transposes for cnt images: four block units,
// or one NHWC tile, a workgroup.
template <typename T, bool BLK>
inline int64_t transpose_groups(int64_t C, int64_t HW, int64_t cnt)
{
    if constexpr (BLK)
        return (cnt * (C / 8) * ((HW + 511) / 512) + 3) / 4;
    return cnt * ((HW + 63) / 64) * ((C + 63) / 64);
}

// Whether the register transposes apply.
template <typename T, bool BLK>
inline bool transpose_regs_ok(int64_t C, int64_t HW, const void *x, const void *xt)
{
    constexpr int64_t EV = 16 / int64_t(sizeof(T));
    return (!BLK || EV == 8) && C % EV == 0 && HW % EV == 0 &&
           reinterpret_cast<uintptr_t>(x) % 16 == 0 && reinterpret_cast<uintptr_t>(xt) % 16 == 0;
}

// Workgroup b of the register transpose of images [0, cnt): `units` block
// units (BLK) or NHWC tiles in all.
template <typename T, bool BLK>
__device__ __forceinline__ void transpose_group(const T *__restrict__ x, T *__restrict__ xt,
                                                int C, int HW, uint32_t b, uint32_t units,
                                                uint4 *lds)
{
    if constexpr (BLK) {
        if constexpr (sizeof(T) == 2) {
            const uint32_t u = b * 4u + (threadIdx.x >> 6);
            if (u < units)
                transpose_blocks_wave<T>(x, xt, C, HW, u);
        }
    } else {
        NhwcTile<T> tl;
        tl.load(x, C, HW, b, int(threadIdx.x));
        tl.put(lds, int(threadIdx.x));
        __syncthreads();
        tl.take(lds, C, HW, int(threadIdx.x), [&](const uint4 &v, size_t off) {
            *reinterpret_cast<uint4 *>(xt + off) = v;
        });
    }
}

template <typename T, bool BLK>
__global__ __launch_bounds__(256) void to_nhwc_regs_kernel(const T *__restrict__ x,
                                                           T *__restrict__ xt, int C, int HW,
                                                           uint32_t units)
{
    __shared__ uint4 lds[BLK ? 1 : 64 * 64 * sizeof(T) / 16];
    transpose_group<T, BLK>(x, xt, C, HW, blockIdx.x, units, lds);
}

template <typename T>
__device__ __forceinline__ void pack_weight_elem(const T *__restrict__ w, T *__restrict__ wp,
                                                 int t, int total, int Kp, int Kg, int Cg, int K)
{
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
__global__ __launch_bounds__(256) void pack_weight_kernel(const T *__restrict__ w,
                                                          T *__restrict__ wp, int total, int Kp,
                                                          int Kg, int Cg, int K)
{
    pack_weight_elem(w, wp, int(blockIdx.x * 256 + threadIdx.x), total, Kp, Kg, Cg, K);
}

// The window path's weight: for each group g, K step st = chunk*K + k
// (chunk of 16 channels, tap k) and half h, the plane of Mg rows of 8
// channels: wp[(((g*S + st)*2 + h)*Mg + m)*8 + e] =
// weight[g*Mg + m][16*chunk + 8*h + e][k], S = (Cg/16)*K.
template <typename T>
__device__ __forceinline__ void pack_steps_elem(const T *__restrict__ w, T *__restrict__ wp,
                                                int t, int total, int Mg, int Cg, int K, int S,
                                                uint32_t *__restrict__ flags, int nflags)
{
    if (t < nflags)
        flags[t] = 0u;
    if (t >= total)
        return;
    const int e = t & 7;
    int r = t >> 3;
    const int m = r % Mg;
    r /= Mg;
    const int h = r & 1;
    r >>= 1;
    const int st = r % S;
    const int g = r / S;
    const int chunk = st / K, k = st - chunk * K;
    const int cl = chunk * 16 + h * 8 + e;
    wp[t] = w[(size_t(g * Mg + m) * Cg + cl) * K + k];
}

template <typename T>
__global__ __launch_bounds__(256) void pack_weight_steps_kernel(const T *__restrict__ w,
                                                                T *__restrict__ wp, int total,
                                                                int Mg, int Cg, int K, int S,
                                                                uint32_t *__restrict__ flags,
                                                                int nflags)
{
    pack_steps_elem(w, wp, int(blockIdx.x * 256 + threadIdx.x), total, Mg, Cg, K, S, flags,
                    nflags);
}

// Eight consecutive elements of a packed weight (PK 1: [Co][Kp]; PK 2: the
// window path's step-major planes), elements 8*t8 .. 8*t8+7, one thread:
// eight loads and one (16-bit) or two (fp32) 16-byte stores.  Kp and the
// planes' 8-element rows keep every group of eight inside one row.
template <typename T, int PK>
__device__ __forceinline__ void pack8(const T *__restrict__ w, T *__restrict__ wp, int t8,
                                      int total, int Kp, int Kg, int Cg, int K, int Mg, int S)
{
    const int t = t8 * 8;
    if (t >= total)
        return;
    union {
        T e[8];
        uint4 q[8 * sizeof(T) / 16];
    } v;
    if constexpr (PK == 1) {
        const int kk0 = t % Kp;
        const int co = t / Kp;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int kk = kk0 + e;
            const int k = kk / Cg;
            const int cl = kk - k * Cg;
            v.e[e] = kk < Kg ? w[(size_t(co) * Cg + cl) * K + k] : T(0);
        }
    } else {
        int r = t8;
        const int m = r % Mg;
        r /= Mg;
        const int h = r & 1;
        r >>= 1;
        const int st = r % S;
        const int g = r / S;
        const int chunk = st / K, k = st - chunk * K;
        const T *src = w + (size_t(g * Mg + m) * Cg + chunk * 16 + h * 8) * K + k;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            v.e[e] = src[size_t(e) * K];
    }
    uint4 *dst = reinterpret_cast<uint4 *>(wp + t);
#pragma unroll
    for (int j = 0; j < int(8 * sizeof(T) / 16); ++j)
        dst[j] = v.q[j];
}

// The exponent e of an FP8 weight row: the largest integer with
// max|row| * 2^e <= 448 (0 for a row with no nonzero finite maximum; clamped
// to [-126, 126]).  One workgroup (256 threads) per row, contiguous reads;
// `red` is 4 floats of LDS.
template <typename T>
__device__ __forceinline__ int row_exponent(const T *__restrict__ row, int Kg, float *red)
{
    float mx = 0.0f;
    for (int t = int(threadIdx.x); t < Kg; t += 256)
        mx = fmaxf(mx, fabsf(to_f32(row[t])));        // fmaxf skips NaN
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1)
        mx = fmaxf(mx, __shfl_xor(mx, d, 64));
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    int e = 0;
    if (mx > 0.0f && !__builtin_isinf(mx)) {
        int ex;
        const float f = frexpf(mx, &ex);              // mx = f * 2^ex, f in [0.5, 1)
        e = (f <= 0.875f) ? 9 - ex : 8 - ex;          // 448 = 0.875 * 2^9
        e = min(126, max(-126, e));
    }
    return e;
}

// The FP8 path's weight, one workgroup (256 threads) per output channel co:
// the row's exponent e (row_exponent), wq[co][kk] = E4M3(w * 2^e) in
// tap-major order (kk = k*Cg + c', zero for kk >= Kg) and wscale[co] = 2^-e,
// which the GEMM epilogue applies to the row's sums.  Scaling by a power of
// two is exact, so the only rounding is E4M3's own.
template <typename T>
__device__ __forceinline__ void quantize_row(const T *__restrict__ w, e4m3_t *__restrict__ wq,
                                             float *__restrict__ wscale, int co, int Kg, int Kp,
                                             int Cg, int K, float *red)
{
    const T *row = w + size_t(co) * Kg;              // weight [Co][Cg][kh][kw]: Kg per row
    const int e = row_exponent(row, Kg, red);
    e4m3_t *dst = wq + size_t(co) * Kp;
    for (int kk = int(threadIdx.x); kk < Kp; kk += 256) {   // the row is in L1 by now
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

// The windowed FP8 kernel's weight, one workgroup per output channel
// co = g*Mg + m (3x3 taps): the same exponent and rounding as quantize_row,
// written per 16-channel chunk c as 144 bytes of the chunk's block
// [G][Cg/16][region]: an 8-byte piece (channels 16c + 8h .. +7 at tap k) goes
// to region k / 4 for k < 8, laid out [h][part][Mg][16 bytes] with part
// (k % 4) / 2 and the piece at byte 8 * (k % 2) of the 16, and to region 2,
// [h][Mg][8 bytes], for tap 8.  One thread per piece: eight loads and one
// 8-byte store.
template <typename T>
__device__ __forceinline__ void quantize_row_window(const T *__restrict__ w,
                                                    e4m3_t *__restrict__ wq,
                                                    float *__restrict__ wscale, int co, int Kg,
                                                    int Cg, int Mg, float *red)
{
    constexpr int K = 9;
    const T *row = w + size_t(co) * Kg;
    const int e = row_exponent(row, Kg, red);
    const int g = co / Mg, m = co - g * Mg;
    const int nch = Cg / 16;
    for (int t = int(threadIdx.x); t < nch * 2 * K; t += 256) {
        const int k = t % K;
        const int ch = t / K;                         // 8-channel piece of the row
        const int c = ch >> 1, h = ch & 1;
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            v[i] = ldexpf(to_f32(row[(ch * 8 + i) * K + k]), e);
        const uint2 q = make_uint2(pack4_e4m3(v[0], v[1], v[2], v[3]),
                                   pack4_e4m3(v[4], v[5], v[6], v[7]));
        const size_t blk = (size_t(g) * nch + c) * size_t(Mg) * 144;
        const size_t o = k < 8 ? blk + size_t(k / 4) * 64 * Mg +
                                     (size_t(h * 2 + (k % 4) / 2) * Mg + m) * 16 +
                                     size_t(k % 2) * 8
                               : blk + size_t(128) * Mg + (size_t(h) * Mg + m) * 8;
        *reinterpret_cast<uint2 *>(wq + o) = q;
    }
    if (threadIdx.x == 0)
        wscale[co] = ldexpf(1.0f, -e);
}

// Both set-up jobs of a forward in one launch (for small problems the
// launches cost more than the work): the first `nt` workgroups transpose
// x (VEC: register transpose units 4b .. 4b+3, one a wave; otherwise LDS
// tile b -> (b % gx, b / gx % gy, b / (gx*gy))), the rest repack the
// weight (PK 1: [G][Mg][Kp] tap-major; PK 2: the window path's step-major
// planes, and its hand-over flags cleared; PK 3: the FP8 path's E4M3 rows
// and scales, one workgroup per row; PK 4: the windowed FP8 kernel's E4M3
// chunk blocks and scales, one workgroup per row, and its hand-over flags
// cleared).
struct PrepArgs {
    const void *x;
    void *xt;
    const void *w;
    void *wp;
    uint32_t *flags;
    float *wscale;
    int C, HW, gx, gy, nt;
    uint32_t units;
    int total, Kp, Kg, Cg, K, Mg, S, nflags;
};

template <typename T, bool BLK, bool VEC, int PK>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a)
{
    __shared__ __attribute__((aligned(16))) T tile[kTile][kTile + 1];
    const int b = int(blockIdx.x);
    if (b < a.nt) {
        if constexpr (VEC) {
            transpose_group<T, BLK>(static_cast<const T *>(a.x), static_cast<T *>(a.xt), a.C,
                                    a.HW, uint32_t(b), a.units,
                                    reinterpret_cast<uint4 *>(&tile[0][0]));
        } else {
            const int bx = b % a.gx, by = (b / a.gx) % a.gy, bz = b / (a.gx * a.gy);
            transpose_tile<T, BLK>(static_cast<const T *>(a.x), static_cast<T *>(a.xt), a.C,
                                   a.HW, bx, by, bz, tile);
        }
        return;
    }
    if constexpr (PK == 3) {
        quantize_row(static_cast<const T *>(a.w), static_cast<e4m3_t *>(a.wp), a.wscale,
                     b - a.nt, a.Kg, a.Kp, a.Cg, a.K, reinterpret_cast<float *>(&tile[0][0]));
        return;
    }
    if constexpr (PK == 4) {
        // one row a workgroup; workgroups past the last row only clear flags
        const int r = b - a.nt;
        const int t = r * 256 + int(threadIdx.x);
        if (t < a.nflags)
            a.flags[t] = 0u;
        if (r < a.total)
            quantize_row_window(static_cast<const T *>(a.w), static_cast<e4m3_t *>(a.wp),
                                a.wscale, r, a.Kg, a.Cg, a.Mg,
                                reinterpret_cast<float *>(&tile[0][0]));
        return;
    }
    // eight weight elements a thread (and, window path, one flag)
    const int t8 = (b - a.nt) * 256 + int(threadIdx.x);
    if (PK == 2 && t8 < a.nflags)
        a.flags[t8] = 0u;
    pack8<T, PK>(static_cast<const T *>(a.w), static_cast<T *>(a.wp), t8, a.total, a.Kp, a.Kg,
                 a.Cg, a.K, a.Mg, a.S);
}

template <typename T, bool BLK>
hipError_t to_nhwc_t(const Problem &p, int64_t cnt, const void *x, void *xt, hipStream_t s)
{
    const int HW = int(p.H * p.W);
    const size_t img = size_t(p.C) * size_t(HW);
    if (transpose_regs_ok<T, BLK>(p.C, HW, x, xt)) {
        // images per launch: at most 2^29 workgroups
        const int64_t per = transpose_groups<T, BLK>(p.C, HW, 1);
        const int64_t step = std::max<int64_t>(1, (int64_t(1) << 29) / std::max<int64_t>(per, 1));
        for (int64_t n0 = 0; n0 < cnt; n0 += step) {
            const int64_t m = std::min(step, cnt - n0);
            const int64_t units = BLK ? m * (p.C / 8) * ((HW + 511) / 512) : 0;
            hipLaunchKernelGGL((to_nhwc_regs_kernel<T, BLK>),
                               dim3(unsigned(transpose_groups<T, BLK>(p.C, HW, m))), dim3(256), 0,
                               s, static_cast<const T *>(x) + size_t(n0) * img,
                               static_cast<T *>(xt) + size_t(n0) * img, int(p.C), HW,
                               uint32_t(units));
            hipError_t e = hipGetLastError();
            if (e != hipSuccess)
                return e;
        }
        return hipSuccess;
    }
    dim3 grid((HW + kTile - 1) / kTile, unsigned((p.C + kTile - 1) / kTile), 1);
    // The z dimension is limited to 65535; walk larger batches in slices.
    for (int64_t n0 = 0; n0 < cnt; n0 += 65535) {
        grid.z = unsigned(std::min<int64_t>(65535, cnt - n0));
        const size_t off = size_t(n0) * img;
        hipLaunchKernelGGL((to_nhwc_kernel<T, BLK>), grid, dim3(256), 0, s,
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
    case MDCN_F32: return to_nhwc_t<float, false>(p, cnt, x, xt, stream);
    case MDCN_F16: return to_nhwc_t<half_t, false>(p, cnt, x, xt, stream);
    case MDCN_BF16: return to_nhwc_t<bf16_t, false>(p, cnt, x, xt, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_to_channel_blocks(const Problem &p, int64_t cnt, const void *x, void *xb,
                                    hipStream_t stream)
{
    if (p.C % 8 != 0)
        return hipErrorInvalidValue;
    switch (p.dtype) {
    case MDCN_F32: return to_nhwc_t<float, true>(p, cnt, x, xb, stream);
    case MDCN_F16: return to_nhwc_t<half_t, true>(p, cnt, x, xb, stream);
    case MDCN_BF16: return to_nhwc_t<bf16_t, true>(p, cnt, x, xb, stream);
    }
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t pack_weight_steps_t(const Problem &p, const void *w, void *wp, uint32_t *flags,
                               int nflags, hipStream_t s)
{
    const int S = int(p.Cg / 16 * p.K);
    const int total = int(p.G * S * 2 * p.Mg * 8);
    const int n = std::max(total, flags ? nflags : 0);
    hipLaunchKernelGGL(pack_weight_steps_kernel<T>, dim3((n + 255) / 256), dim3(256), 0, s,
                       static_cast<const T *>(w), static_cast<T *>(wp), total, int(p.Mg),
                       int(p.Cg), int(p.K), S, flags, flags ? nflags : 0);
    return hipGetLastError();
}

hipError_t launch_pack_weight_steps(const Problem &p, const void *weight, void *wpack,
                                    uint32_t *flags, int nflags, hipStream_t stream)
{
    if (p.Cg % 16 != 0)
        return hipErrorInvalidValue;
    switch (p.dtype) {
    case MDCN_F32: return pack_weight_steps_t<float>(p, weight, wpack, flags, nflags, stream);
    case MDCN_F16: return pack_weight_steps_t<half_t>(p, weight, wpack, flags, nflags, stream);
    case MDCN_BF16: return pack_weight_steps_t<bf16_t>(p, weight, wpack, flags, nflags, stream);
    }
    return hipErrorInvalidValue;
}

namespace {

template <typename T, bool BLK, int PK>
hipError_t prep_t(const Problem &p, const Plan &plan, int64_t cnt, const void *x, void *xt,
                  const void *w, void *wp, uint32_t *flags, int nflags, float *wscale,
                  hipStream_t s)
{
    const int HW = int(p.H * p.W);
    PrepArgs a{};
    a.x = x; a.xt = xt; a.w = w; a.wp = wp; a.flags = flags; a.wscale = wscale;
    a.C = int(p.C); a.HW = HW;
    a.gx = (HW + kTile - 1) / kTile;
    a.gy = int((p.C + kTile - 1) / kTile);
    a.Cg = int(p.Cg); a.K = int(p.K);
    int64_t npack;
    if constexpr (PK == 3) {
        a.Kp = int(plan.Kp);
        a.Kg = int(p.Kg);
        npack = p.Co * 256;                   // one workgroup per row
    } else if constexpr (PK == 4) {
        if (p.Cg % 16 != 0 || p.K != 9 || reinterpret_cast<uintptr_t>(wp) % 8 != 0)
            return hipErrorInvalidValue;
        a.total = int(p.Co);                  // rows
        a.Kg = int(p.Kg);
        a.Mg = int(p.Mg);
        a.nflags = flags ? nflags : 0;
        npack = std::max<int64_t>(p.Co * 256, a.nflags);   // one workgroup per row
    } else if constexpr (PK == 1) {
        a.total = int(p.Co * plan.Kp);
        a.Kp = int(plan.Kp);
        a.Kg = int(p.Kg);
        if (a.Kp % 8 != 0 || reinterpret_cast<uintptr_t>(wp) % 32 != 0)
            return hipErrorInvalidValue;
        npack = a.total / 8;                  // threads: eight elements each
    } else {
        if (p.Cg % 16 != 0 || reinterpret_cast<uintptr_t>(wp) % 32 != 0)
            return hipErrorInvalidValue;
        a.S = int(p.Cg / 16 * p.K);
        a.total = int(p.G * a.S * 2 * p.Mg * 8);
        a.Mg = int(p.Mg);
        a.nflags = flags ? nflags : 0;
        npack = std::max<int64_t>(a.total / 8, a.nflags);
    }
    const bool vec = transpose_regs_ok<T, BLK>(p.C, HW, x, xt);
    const int64_t units = vec ? (BLK ? cnt * (p.C / 8) * ((HW + 511) / 512) : 0) : 0;
    const int64_t nt = vec ? transpose_groups<T, BLK>(p.C, HW, cnt) : int64_t(a.gx) * a.gy * cnt;
    const int64_t blocks = nt + (npack + 255) / 256;
    if (blocks > 0x7fffffffll)
        return hipErrorInvalidValue;
    a.nt = int(nt);
    a.units = uint32_t(units);
    if (vec)
        hipLaunchKernelGGL((prep_kernel<T, BLK, true, PK>), dim3(unsigned(blocks)), dim3(256), 0,
                           s, a);
    else
        hipLaunchKernelGGL((prep_kernel<T, BLK, false, PK>), dim3(unsigned(blocks)), dim3(256), 0,
                           s, a);
    return hipGetLastError();
}

template <typename T>
hipError_t prep_dtype(const Problem &p, const Plan &plan, int64_t cnt, const void *x, void *xt,
                      const void *w, void *wp, uint32_t *flags, int nflags, float *wscale,
                      hipStream_t s)
{
    if (plan.path == Path::Window)
        return prep_t<T, true, 2>(p, plan, cnt, x, xt, w, wp, flags, nflags, nullptr, s);
    if (plan.path == Path::WindowFp8)
        return prep_t<T, true, 4>(p, plan, cnt, x, xt, w, wp, flags, nflags, wscale, s);
    if (plan.path == Path::GatherGemmFp8)
        return prep_t<T, false, 3>(p, plan, cnt, x, xt, w, wp, nullptr, 0, wscale, s);
    return prep_t<T, false, 1>(p, plan, cnt, x, xt, w, wp, flags, nflags, nullptr, s);
}

}  // namespace

hipError_t launch_prep(const Problem &p, const Plan &plan, int64_t cnt, const void *x, void *xt,
                       const void *weight, void *wpack, uint32_t *flags, int nflags,
                       float *wscale, hipStream_t stream)
{
    if ((plan.path == Path::GatherGemmFp8 || plan.path == Path::WindowFp8) && !wscale)
        return hipErrorInvalidValue;
    if ((plan.path == Path::Window || plan.path == Path::WindowFp8) && p.C % 8 != 0)
        return hipErrorInvalidValue;
    switch (p.dtype) {
    case MDCN_F32:
        return prep_dtype<float>(p, plan, cnt, x, xt, weight, wpack, flags, nflags, wscale,
                                stream);
    case MDCN_F16:
        return prep_dtype<half_t>(p, plan, cnt, x, xt, weight, wpack, flags, nflags, wscale,
                                stream);
    case MDCN_BF16:
        return prep_dtype<bf16_t>(p, plan, cnt, x, xt, weight, wpack, flags, nflags, wscale,
                                stream);
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
