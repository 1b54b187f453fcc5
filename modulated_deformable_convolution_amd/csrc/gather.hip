// gather.hip -- deformable im2col: for every (group, image, output pixel,
// tap, channel) the modulated bilinear sample of the input
// [plugin guide §五 step 1: anchor = out*stride - pad, sample = anchor +
// tap*dilation + learned offset, bilinear interpolation reading 0 off the
// image, times the mask, into the column buffer].
//
// The FP8 path writes the columns as OCP E4M3 bytes (each value saturated to
// +-448, rounded to nearest even) instead of elements of T.
//
// Layout choice (this library's, not the page's): x is read channels-last
// (NHWC, prepared by to_nhwc) and the columns are written K-contiguous,
// col[g][n*P + pix][k*Cg + c'], so that
//  - the 16-byte vector of channels c'..c'+VEC-1 at one bilinear corner is a
//    single contiguous load, and consecutive lanes (consecutive channel
//    vectors, then taps) read and write consecutive memory;
//  - the GEMM reads both of its operands K-contiguous, which is the register
//    layout of the MFMA A and B fragments.
//
// Workgroups are numbered so that consecutive pixel tiles of one image run
// on the same XCD: the corner reads of a band of output rows then hit a band
// of input rows in that XCD's L2.
//
// A workgroup owns tp consecutive output pixels of one image and one group,
// and kc consecutive taps (all of them unless the geometry table would not fit
// in 64 KB of LDS).  Phase 1 computes, once per (offset group, tap, pixel), the
// four corner offsets and the four bilinear weights with the mask folded in
// (fp32) and keeps them in LDS; phase 2 streams the channel vectors.  A corner off the
// image gets an offset past the end of the image's buffer range, which the
// buffer load returns as 0, so phase 2 has no branches.
#include "device_common.h"
#include "launch.h"

namespace mdcn {

namespace {

constexpr int kMaxTP = 32;       // output pixels per workgroup (at most)
constexpr int kThreads = 256;
constexpr size_t kGeoBytes = 64 * 1024;
constexpr uint32_t kOffImage = 0x80000000u;   // a byte offset no image reaches

struct GatherArgs {
    int Cg, Cdg, C, H, W, Wo, kw, K, P;
    int sh, sw, ph, pw, dh, dw;
    int offC, mskC;              // channels of offset and mask: 2*DG*K, DG*K
    int Kg, Kp, cnt;
    int tp, tiles;               // pixels per workgroup, pixel tiles per image
    int kc, kchunks;             // taps per workgroup, tap chunks
    int nq;                      // offset groups one group's channels can span
};

struct Geo {
    uint32_t off[4];             // byte offsets of the corners within the image
    float wt[4];
};

template <typename T>
__device__ __forceinline__ void vec_fma(float *acc, const uint4 &raw, float w)
{
    Vec16<T> v;
    v.raw = raw;
#pragma unroll
    for (int e = 0; e < Vec16<T>::N; ++e)
        acc[e] = fmaf(w, to_f32(v.e[e]), acc[e]);
}

// Buffer resource over `bytes` bytes at `base`, built from scalar copies of
// its inputs so that it provably lives in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t v = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
    void *p = reinterpret_cast<void *>((uint64_t(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, int(n), 0x00020000);
}

// One column element of output type O: T, or E4M3 for the FP8 path.
template <typename O> __device__ __forceinline__ O col_elem(float v) { return from_f32<O>(v); }
template <> __device__ __forceinline__ e4m3_t col_elem<e4m3_t>(float v) { return to_e4m3(v); }

// One output vector: VEC channels (c'..c'+VEC-1 of group g) at (pixel p0+pl,
// tap k0+kl), the four corners read with buffer loads (0 off the image),
// written as VEC elements of O (T, or E4M3 bytes for the FP8 path).
template <typename T, typename O, bool VECTOR>
__device__ __forceinline__ void gather_item(const GatherArgs &a, const Geo *geo,
                                            __amdgpu_buffer_rsrc_t rs, const char *img,
                                            O *col_g, int g, int q0, int p0, int k0, int pl,
                                            int kl, int cv)
{
    constexpr int VEC = VECTOR ? 16 / int(sizeof(T)) : 1;
    const int c = g * a.Cg + cv * VEC;
    const Geo gd = geo[((c / a.Cdg - q0) * a.kc + kl) * a.tp + pl];
    const uint32_t cb = uint32_t(c) * uint32_t(sizeof(T));
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e)
        acc[e] = 0.0f;
    O *dst = col_g + size_t(p0 + pl) * a.Kp + (k0 + kl) * a.Cg + cv * VEC;
    if constexpr (VECTOR) {
        uint4 v[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint32_t o = gd.off[s] == kOffImage ? kOffImage : gd.off[s] + cb;
            const auto r = __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 0);
            __builtin_memcpy(&v[s], &r, 16);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
            vec_fma<T>(acc, v[s], gd.wt[s]);
        if constexpr (sizeof(O) == 1) {
            // VEC E4M3 bytes: 8 (fp16/bf16 input) or 4 (fp32)
            uint32_t w[VEC / 4];
#pragma unroll
            for (int h = 0; h < VEC / 4; ++h)
                w[h] = pack4_e4m3(acc[4 * h], acc[4 * h + 1], acc[4 * h + 2], acc[4 * h + 3]);
            if constexpr (VEC == 8)
                *reinterpret_cast<uint2 *>(dst) = make_uint2(w[0], w[1]);
            else
                *reinterpret_cast<uint32_t *>(dst) = w[0];
        } else if constexpr (sizeof(O) == 4 && sizeof(T) == 2) {
            // fp32 columns of fp16/bf16 input (the backward's): 8 floats
            *reinterpret_cast<float4 *>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
            *reinterpret_cast<float4 *>(dst + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
        } else {
            Vec16<T> o;
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                o.e[e] = from_f32<T>(acc[e]);
            store16(dst, o);
        }
    } else {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            if (gd.off[s] != kOffImage)
                acc[0] = fmaf(gd.wt[s],
                              to_f32(*reinterpret_cast<const T *>(img + gd.off[s] + cb)), acc[0]);
        dst[0] = col_elem<O>(acc[0]);
    }
}

template <typename T, typename O, bool VECTOR>
__global__ __launch_bounds__(kThreads) void deform_gather_kernel(const T *__restrict__ xt,
                                                                 const T *__restrict__ off,
                                                                 const T *__restrict__ msk,
                                                                 O *__restrict__ col, GatherArgs a)
{
    constexpr int VEC = VECTOR ? 16 / int(sizeof(T)) : 1;
    extern __shared__ __attribute__((aligned(16))) char geo_raw[];
    Geo *geo = reinterpret_cast<Geo *>(geo_raw);

    // Block coordinates, kept in scalar registers (the buffer resource built
    // from them must be provably wave-uniform).  Consecutive logical blocks
    // (consecutive pixel tiles of one image) run on one XCD, so each XCD's L2
    // holds a band of rows of the image instead of all of it.
    uint32_t b = xcd_swizzle(blockIdx.x, gridDim.x);
    const int tile = __builtin_amdgcn_readfirstlane(int(b % uint32_t(a.tiles)));
    b /= uint32_t(a.tiles);
    const int kch = __builtin_amdgcn_readfirstlane(int(b % uint32_t(a.kchunks)));
    b /= uint32_t(a.kchunks);
    const int nl = __builtin_amdgcn_readfirstlane(int(b % uint32_t(a.cnt)));
    const int g = __builtin_amdgcn_readfirstlane(int(b / uint32_t(a.cnt)));
    const int p0 = tile * a.tp;
    const int np = min(a.tp, a.P - p0);
    const int k0 = kch * a.kc;
    const int nk = min(a.kc, a.K - k0);
    const int q0 = (g * a.Cg) / a.Cdg;                   // offset groups of this group:
    const int q1 = ((g + 1) * a.Cg - 1) / a.Cdg;         // q0 .. q1

    // Phase 1: geometry of (offset group q0+qq, tap k0+kl, pixel p0+pl)
    // -> geo[(qq*kc + kl)*tp + pl].
    const int entries = a.nq * a.kc * a.tp;
    const uint32_t elem_c = uint32_t(a.C) * uint32_t(sizeof(T));   // bytes per NHWC pixel
    for (int e = int(threadIdx.x); e < entries; e += kThreads) {
        const int pl = e % a.tp;
        const int kl = (e / a.tp) % a.kc;
        const int q = q0 + e / (a.tp * a.kc);
        Geo gd;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            gd.off[s] = kOffImage;
            gd.wt[s] = 0.0f;
        }
        if (pl < np && kl < nk && q <= q1) {
            const int pix = p0 + pl;
            const int k = k0 + kl;
            const int ho = pix / a.Wo, wo = pix - (pix / a.Wo) * a.Wo;
            const int i = k / a.kw, j = k - (k / a.kw) * a.kw;
            const size_t ob = (size_t(nl) * a.offC + size_t(q) * 2 * a.K + 2 * k) * a.P + pix;
            const float oh = to_f32(off[ob]);
            const float ow = to_f32(off[ob + a.P]);
            const float m = to_f32(msk[(size_t(nl) * a.mskC + size_t(q) * a.K + k) * a.P + pix]);
            const Taps tp = make_taps(ho * a.sh - a.ph + i * a.dh, wo * a.sw - a.pw + j * a.dw,
                                      oh, ow, m, a.H, a.W);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                gd.off[s] = tp.valid[s] ? uint32_t(tp.idx[s]) * elem_c : kOffImage;
                gd.wt[s] = tp.wt[s];
            }
        }
        geo[e] = gd;
    }
    __syncthreads();

    // Phase 2: items (pixel, tap, channel vector), channel vector fastest, so a
    // wave writes consecutive 16-byte pieces of one column row.
    const int CV = a.Cg / VEC;
    const size_t img_bytes = size_t(a.H) * a.W * elem_c;
    const char *img = reinterpret_cast<const char *>(xt) + size_t(nl) * img_bytes;
    const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(img, uint32_t(img_bytes));
    O *col_g = col + (size_t(g) * a.cnt + nl) * size_t(a.P) * a.Kp;

    if (CV <= kThreads && kThreads % CV == 0) {
        // Each thread keeps one channel vector and walks (pixel, tap) rows.
        const int cv = int(threadIdx.x) % CV;
        const int stride = kThreads / CV;
        int r = int(threadIdx.x) / CV;                   // row = pl*nk + kl
        int pl = r / nk, kl = r - (r / nk) * nk;
        while (pl < np) {
            gather_item<T, O, VECTOR>(a, geo, rs, img, col_g, g, q0, p0, k0, pl, kl, cv);
            kl += stride;
            while (kl >= nk) {
                kl -= nk;
                ++pl;
            }
        }
    } else {
        const int items = np * nk * CV;
        for (int it = int(threadIdx.x); it < items; it += kThreads) {
            const int cv = it % CV;
            const int kl = (it / CV) % nk;
            gather_item<T, O, VECTOR>(a, geo, rs, img, col_g, g, q0, p0, k0, it / (CV * nk), kl,
                                      cv);
        }
    }
    // Zero each row's padding [Kg, Kp) (once per row: by the first tap chunk).
    const int pad = a.Kp - a.Kg;
    if (kch == 0) {
        for (int it = int(threadIdx.x); it < np * pad; it += kThreads) {
            const int pl = it / pad;
            col_g[size_t(p0 + pl) * a.Kp + a.Kg + it % pad] = O(0);
        }
    }
}

// The backward's columns of one image, transposed: colT[g][k*Cg + c'][pix]
// (fp32, pixels contiguous), the layout the weight gradient's GEMM reads
// (contraction over pixels).  A workgroup owns 64 consecutive pixels, one
// tap and a slice of up to 64 channels of one group: phase 1 as above (the
// geometry of its pixels), phase 2 samples them channel vector by channel
// vector as the gather does (corner reads of whole 16-byte vectors) into an
// LDS tile [pixel][channel] (row pitch CS + 4 floats), phase 3 writes the
// tile out row by row (a wave stores 64 pixels of one channel row).  Rows
// kk in [Kg, Kp) are zeroed by the tap-0 workgroups.
constexpr int kTPX = 64;         // pixels per workgroup of the transposed gather
constexpr int kTCS = 64;         // channels per slice

template <typename T, bool VECTOR>
__global__ __launch_bounds__(kThreads) void deform_gather_t_kernel(const T *__restrict__ xt,
                                                                   const T *__restrict__ off,
                                                                   const T *__restrict__ msk,
                                                                   float *__restrict__ colT,
                                                                   GatherArgs a, int slices)
{
    constexpr int VEC = VECTOR ? 16 / int(sizeof(T)) : 1;
    extern __shared__ __attribute__((aligned(16))) char lds_raw[];
    Geo *geo = reinterpret_cast<Geo *>(lds_raw);                    // nq * kTPX entries
    float *tile = reinterpret_cast<float *>(lds_raw + size_t(a.nq) * kTPX * sizeof(Geo));

    uint32_t b = xcd_swizzle(blockIdx.x, gridDim.x);
    const int ptile = __builtin_amdgcn_readfirstlane(int(b % uint32_t(a.tiles)));
    b /= uint32_t(a.tiles);
    const int sl = __builtin_amdgcn_readfirstlane(int(b % uint32_t(slices)));
    b /= uint32_t(slices);
    const int k = __builtin_amdgcn_readfirstlane(int(b % uint32_t(a.K)));
    const int g = __builtin_amdgcn_readfirstlane(int(b / uint32_t(a.K)));
    const int p0 = ptile * kTPX;
    const int np = min(kTPX, a.P - p0);
    const int c_lo = sl * kTCS;                          // channel slice within the group
    const int cs = min(kTCS, a.Cg - c_lo);
    const int pitch = kTCS + 4;
    const int q0 = (g * a.Cg) / a.Cdg;

    // Phase 1: geometry of (offset group q0+qq, tap k, pixel p0+pl)
    const uint32_t elem_c = uint32_t(a.C) * uint32_t(sizeof(T));
    for (int e = int(threadIdx.x); e < a.nq * kTPX; e += kThreads) {
        const int pl = e % kTPX;
        const int q = q0 + e / kTPX;
        Geo gd;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            gd.off[s] = kOffImage;
            gd.wt[s] = 0.0f;
        }
        if (pl < np && q < a.offC / (2 * a.K)) {
            const int pix = p0 + pl;
            const int ho = pix / a.Wo, wo = pix - (pix / a.Wo) * a.Wo;
            const int i = k / a.kw, j = k - (k / a.kw) * a.kw;
            const size_t ob = (size_t(q) * 2 * a.K + 2 * k) * a.P + pix;
            const float oh = to_f32(off[ob]);
            const float ow = to_f32(off[ob + a.P]);
            const float m = to_f32(msk[(size_t(q) * a.K + k) * a.P + pix]);
            const Taps tp = make_taps(ho * a.sh - a.ph + i * a.dh, wo * a.sw - a.pw + j * a.dw,
                                      oh, ow, m, a.H, a.W);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                gd.off[s] = tp.valid[s] ? uint32_t(tp.idx[s]) * elem_c : kOffImage;
                gd.wt[s] = tp.wt[s];
            }
        }
        geo[e] = gd;
    }
    __syncthreads();

    // Phase 2: (pixel, channel vector) items, channel vector fastest
    const size_t img_bytes = size_t(a.H) * a.W * elem_c;
    const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(xt, uint32_t(img_bytes));
    const int CV = cs / VEC;
    for (int it = int(threadIdx.x); it < np * CV; it += kThreads) {
        const int pl = it / CV, cv = it - (it / CV) * CV;
        const int c = g * a.Cg + c_lo + cv * VEC;        // input channel
        const Geo gd = geo[(c / a.Cdg - q0) * kTPX + pl];
        const uint32_t cb = uint32_t(c) * uint32_t(sizeof(T));
        float acc[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            acc[e] = 0.0f;
        if constexpr (VECTOR) {
            uint4 v[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint32_t o = gd.off[s] == kOffImage ? kOffImage : gd.off[s] + cb;
                const auto r = __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 0);
                __builtin_memcpy(&v[s], &r, 16);
            }
#pragma unroll
            for (int s = 0; s < 4; ++s)
                vec_fma<T>(acc, v[s], gd.wt[s]);
        } else {
            const char *img = reinterpret_cast<const char *>(xt);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                if (gd.off[s] != kOffImage)
                    acc[0] = fmaf(gd.wt[s],
                                  to_f32(*reinterpret_cast<const T *>(img + gd.off[s] + cb)),
                                  acc[0]);
        }
        float *row = tile + pl * pitch + cv * VEC;
#pragma unroll
        for (int e = 0; e < VEC; e += 4) {
            if constexpr (VEC >= 4)
                *reinterpret_cast<float4 *>(row + e) =
                    make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
        }
        if constexpr (VEC < 4)
            row[0] = acc[0];
    }
    __syncthreads();

    // Phase 3: channel rows out, 64 pixels a wave; a lane reads four
    // channels of its pixel at once (16 lanes of a 16-byte read hit 16
    // distinct bank groups: the row pitch is 4 floats past a multiple of 64)
    const int lane = int(threadIdx.x) & 63, wave = int(threadIdx.x) >> 6;
    float *dst = colT + size_t(g) * a.Kp * a.P + size_t(k * a.Cg + c_lo) * a.P + p0;
    if (cs % 4 == 0) {
        for (int c = wave * 4; c < cs; c += kThreads / 16) {
            const float4 v = *reinterpret_cast<const float4 *>(tile + lane * pitch + c);
            if (lane < np) {
                dst[size_t(c) * a.P + lane] = v.x;
                dst[size_t(c + 1) * a.P + lane] = v.y;
                dst[size_t(c + 2) * a.P + lane] = v.z;
                dst[size_t(c + 3) * a.P + lane] = v.w;
            }
        }
    } else {
        for (int c = wave; c < cs; c += kThreads / 64)
            if (lane < np)
                dst[size_t(c) * a.P + lane] = tile[lane * pitch + c];
    }
    if (k == 0 && sl == 0)
        for (int r = a.Kg + wave; r < a.Kp; r += kThreads / 64)
            if (lane < np)
                colT[size_t(g) * a.Kp * a.P + size_t(r) * a.P + p0 + lane] = 0.0f;
}

template <typename T, typename O>
hipError_t gather_t(const Problem &p, const Plan &plan, int64_t cnt, const void *xt,
                    const void *offset, const void *mask, void *col, hipStream_t s)
{
    constexpr int V = 16 / sizeof(T);
    const bool vec = (p.Cg % V == 0) && (p.Cdg % V == 0);
    GatherArgs a;
    a.Cg = int(p.Cg); a.Cdg = int(p.Cdg); a.C = int(p.C);
    a.H = int(p.H); a.W = int(p.W); a.Wo = int(p.Wo); a.kw = int(p.kw); a.K = int(p.K);
    a.P = int(p.P);
    a.sh = int(p.sh); a.sw = int(p.sw); a.ph = int(p.ph); a.pw = int(p.pw);
    a.dh = int(p.dh); a.dw = int(p.dw);
    a.offC = int(2 * p.DG * p.K); a.mskC = int(p.DG * p.K);
    a.Kg = int(p.Kg); a.Kp = int(plan.Kp); a.cnt = int(cnt);
    // offset groups one group's channels can touch (a channel range of length
    // Cg overlaps at most ceil(Cg / Cdg) + 1 blocks), capped by their count
    a.nq = int(std::min<int64_t>(p.DG, (p.Cg + p.Cdg - 1) / p.Cdg + 1));
    // pixels and taps per workgroup: shrink until the geometry table fits
    int tp = kMaxTP, kc = int(p.K);
    while (size_t(a.nq) * kc * tp * sizeof(Geo) > kGeoBytes) {
        if (kc > 1)
            kc = (kc + 1) / 2;
        else if (tp > 1)
            tp /= 2;
        else
            return hipErrorInvalidValue;   // excluded by validation (offset groups)
    }
    a.tp = tp;
    a.tiles = int((p.P + tp - 1) / tp);
    a.kc = kc;
    a.kchunks = int((p.K + kc - 1) / kc);
    const size_t lds = size_t(a.nq) * kc * tp * sizeof(Geo);
    const dim3 grid(unsigned(uint64_t(p.G) * cnt * a.kchunks * a.tiles));
    if (vec)
        hipLaunchKernelGGL((deform_gather_kernel<T, O, true>), grid, dim3(kThreads), lds, s,
                           static_cast<const T *>(xt), static_cast<const T *>(offset),
                           static_cast<const T *>(mask), static_cast<O *>(col), a);
    else
        hipLaunchKernelGGL((deform_gather_kernel<T, O, false>), grid, dim3(kThreads), lds, s,
                           static_cast<const T *>(xt), static_cast<const T *>(offset),
                           static_cast<const T *>(mask), static_cast<O *>(col), a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gather_f32(const Problem &p, const Plan &plan, int64_t cnt, const void *xt,
                             const void *offset, const void *mask, float *col,
                             hipStream_t stream)
{
    switch (p.dtype) {
    case MDCN_F32: return gather_t<float, float>(p, plan, cnt, xt, offset, mask, col, stream);
    case MDCN_F16: return gather_t<half_t, float>(p, plan, cnt, xt, offset, mask, col, stream);
    case MDCN_BF16: return gather_t<bf16_t, float>(p, plan, cnt, xt, offset, mask, col, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gather_f32_t(const Problem &p, const Plan &plan, const void *xt,
                               const void *offset, const void *mask, float *colT,
                               hipStream_t stream)
{
    GatherArgs a{};
    a.Cg = int(p.Cg); a.Cdg = int(p.Cdg); a.C = int(p.C);
    a.H = int(p.H); a.W = int(p.W); a.Wo = int(p.Wo); a.kw = int(p.kw); a.K = int(p.K);
    a.P = int(p.P);
    a.sh = int(p.sh); a.sw = int(p.sw); a.ph = int(p.ph); a.pw = int(p.pw);
    a.dh = int(p.dh); a.dw = int(p.dw);
    a.offC = int(2 * p.DG * p.K); a.mskC = int(p.DG * p.K);
    a.Kg = int(p.Kg); a.Kp = int(plan.Kp); a.cnt = 1;
    a.nq = int(std::min<int64_t>(p.DG, (p.Cg + p.Cdg - 1) / p.Cdg + 1));
    a.tiles = int((p.P + kTPX - 1) / kTPX);
    const int slices = int((p.Cg + kTCS - 1) / kTCS);
    const size_t lds = size_t(a.nq) * kTPX * sizeof(Geo) + size_t(kTPX) * (kTCS + 4) * 4;
    if (lds > size_t(160) * 1024)
        return hipErrorInvalidValue;
    const uint64_t blocks = uint64_t(p.G) * p.K * slices * a.tiles;
    if (blocks > 0x7fffffffull)
        return hipErrorInvalidValue;
    const dim3 grid{unsigned(blocks), 1u, 1u};
    auto run = [&](auto tag) -> hipError_t {
        using T = decltype(tag);
        constexpr int V = 16 / sizeof(T);
        auto kv = deform_gather_t_kernel<T, true>;
        auto ks = deform_gather_t_kernel<T, false>;
        const bool vec = (p.Cg % V == 0) && (p.Cdg % V == 0) && (p.Cg >= kTCS || p.Cg % V == 0);
        static const hipError_t av = hipFuncSetAttribute(
            reinterpret_cast<const void *>(kv), hipFuncAttributeMaxDynamicSharedMemorySize,
            160 * 1024);
        static const hipError_t as = hipFuncSetAttribute(
            reinterpret_cast<const void *>(ks), hipFuncAttributeMaxDynamicSharedMemorySize,
            160 * 1024);
        if (av != hipSuccess || as != hipSuccess)
            return av != hipSuccess ? av : as;
        if (vec)
            hipLaunchKernelGGL(kv, grid, dim3(kThreads), lds, stream, static_cast<const T *>(xt),
                               static_cast<const T *>(offset), static_cast<const T *>(mask),
                               colT, a, slices);
        else
            hipLaunchKernelGGL(ks, grid, dim3(kThreads), lds, stream, static_cast<const T *>(xt),
                               static_cast<const T *>(offset), static_cast<const T *>(mask),
                               colT, a, slices);
        return hipGetLastError();
    };
    switch (p.dtype) {
    case MDCN_F32: return run(float{});
    case MDCN_F16: return run(half_t{});
    case MDCN_BF16: return run(bf16_t{});
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gather(const Problem &p, const Plan &plan, int64_t cnt, const void *xt,
                         const void *offset, const void *mask, void *col, hipStream_t stream)
{
    if (plan.path == Path::GatherGemmFp8) {
        switch (p.dtype) {
        case MDCN_F32: return gather_t<float, e4m3_t>(p, plan, cnt, xt, offset, mask, col, stream);
        case MDCN_F16: return gather_t<half_t, e4m3_t>(p, plan, cnt, xt, offset, mask, col, stream);
        case MDCN_BF16:
            return gather_t<bf16_t, e4m3_t>(p, plan, cnt, xt, offset, mask, col, stream);
        }
        return hipErrorInvalidValue;
    }
    switch (p.dtype) {
    case MDCN_F32: return gather_t<float, float>(p, plan, cnt, xt, offset, mask, col, stream);
    case MDCN_F16: return gather_t<half_t, half_t>(p, plan, cnt, xt, offset, mask, col, stream);
    case MDCN_BF16: return gather_t<bf16_t, bf16_t>(p, plan, cnt, xt, offset, mask, col, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mdcn
