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
// fastest memory for random reads is LDS, and on gfx950 a random LDS read
// costs about the same per lane up to 8 bytes and less than twice that for
// 16: wider entries are nearly free.  A workgroup therefore stages CH
// channels of one image interleaved, one ENT-byte entry (4 fp32 or 8 fp16
// channels for ENT = 16) per plane position.  Channels that share an offset
// group share every sample position, so one sampling geometry (corner
// address and four weights with the mask folded in) serves all CH channels,
// and the four corners of a sample are four aligned entry reads.
//
// The staged plane has a zero ring two entries wide.  A sample's top-left
// corner (h0, w0) is clamped to [-2, H] x [-2, W]: a sample with -1 <= h0 <=
// H-1 and -1 <= w0 <= W-1 is unchanged (its off-image corners read the ring's
// zeros, the zero that bilinear interpolation reads off the image), and any
// other sample lies entirely off the image and lands on a window of ring
// zeros, so it contributes 0 whatever its weights.  Taps need no validity
// test, and no input value can leak into an off-image sample.
//
// The geometry of a sample depends on the image, offset group, tap and
// pixel, not on the channel, so a small kernel computes it once per image
// (dw_geometry_kernel, one 16-byte record per sample) and every channel
// block of the image reads it back instead of recomputing it from offsets
// and masks.  A sample entirely off the image gets the record of one fixed
// window of ring zeros: the lanes holding such samples then read the same
// LDS addresses, which costs no bank conflicts (random samples spread over
// the plane are what bounds this kernel).
// Workgroups are ordered so that those of one image run on one XCD: the
// image's geometry, read by every channel block, stays in that L2.
// When not even a one-channel plane fits in LDS, a plain kernel reading x,
// offsets and masks from global memory is used instead (no workspace).
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
    int DG;
    uint32_t w_magic;        // floor(2^32 / W) + 1 for W > 1: pos / W = umulhi(pos, w_magic)
};

// Sampling geometry: rows r = (img*DG + q)*K + k of P records, one per
// (image, offset group, tap, pixel).  A record holds the index of the
// sample's top-left corner in the zero-ringed (H+4) x (W+4) plane, the
// fractional row part ly, and the two column weights with the mask folded in,
// lx*m and (1-lx)*m; the four bilinear weights are their products with ly
// and 1-ly.
struct DwGeoArgs {
    uint32_t groups;         // cnt * DG
    int P, Wo, K, kw, DG, H, W, PW;
    int sh, sw, ph, pw, dh, dw;
    int offC, mskC;
};

constexpr int kGeoThreads = 128;
constexpr int kGeoTaps = 3;                  // taps per thread, their inputs loaded at once

// One thread per (image, offset group, pixel, group of kGeoTaps taps): the
// loads of its taps are issued together, and the grid holds enough waves
// (one per 64 pixels, image, offset group and tap group) to keep HBM busy.
template <typename T>
__global__ __launch_bounds__(kGeoThreads) void dw_geometry_kernel(const T *__restrict__ off,
                                                                  const T *__restrict__ msk,
                                                                  uint4 *__restrict__ geo,
                                                                  DwGeoArgs a)
{
    const int pix = int(blockIdx.x) * kGeoThreads + int(threadIdx.x);
    if (pix >= a.P)
        return;
    const int ho = pix / a.Wo, wo = pix - (pix / a.Wo) * a.Wo;
    const int bh = ho * a.sh - a.ph, bw = wo * a.sw - a.pw;
    const uint32_t tgroups = uint32_t(a.K + kGeoTaps - 1) / uint32_t(kGeoTaps);
    // grid y over (image, offset group, tap group), strided when there are more
    for (uint32_t gy = blockIdx.y; gy < a.groups * tgroups; gy += gridDim.y) {
        const uint32_t g = gy / tgroups;
        const int k0 = int(gy - g * tgroups) * kGeoTaps;
        const int q = int(g % uint32_t(a.DG));
        const int img = int(g / uint32_t(a.DG));
        const T *ob = off + (size_t(img) * a.offC + size_t(q) * 2 * a.K) * a.P + pix;
        const T *mb = msk + (size_t(img) * a.mskC + size_t(q) * a.K) * a.P + pix;
        uint4 *gb = geo + size_t(g) * a.K * a.P + pix;
        float oh[kGeoTaps], ow[kGeoTaps], m[kGeoTaps];
#pragma unroll
        for (int t = 0; t < kGeoTaps; ++t) {
            const int k = min(k0 + t, a.K - 1);
            oh[t] = to_f32(ob[size_t(2 * k) * a.P]);
            ow[t] = to_f32(ob[size_t(2 * k + 1) * a.P]);
            m[t] = to_f32(mb[size_t(k) * a.P]);
        }
#pragma unroll
        for (int t = 0; t < kGeoTaps; ++t) {
            const int k = k0 + t;
            if (k >= a.K)
                break;
            const int i = k / a.kw, j = k - (k / a.kw) * a.kw;
            const int ah = bh + i * a.dh, aw = bw + j * a.dw;
            // Offsets clamped to +-2^24 (a NaN becomes -2^24): farther is
            // off any image, and the integer parts stay exact.  A sample
            // whose top-left corner (h0, w0) lies outside [-1, H-1] x
            // [-1, W-1] has no corner on the image; it gets entry 0, whose
            // 2 x 2 window (ring rows and columns 0 and 1) is all zeros,
            // so it contributes 0 whatever its weights.
            const float lim = 16777216.0f;
            const float vh = fminf(fmaxf(oh[t], -lim), lim);
            const float vw = fminf(fmaxf(ow[t], -lim), lim);
            const float fh = floorf(vh), fw = floorf(vw);
            const float h0 = float(ah) + fh, w0 = float(aw) + fw;
            const bool on = (h0 >= -1.0f) & (h0 <= float(a.H - 1)) & (w0 >= -1.0f) &
                            (w0 <= float(a.W - 1));
            const uint32_t e = on ? uint32_t((int(h0) + 2) * a.PW + (int(w0) + 2)) : 0u;
            const float ly = vh - fh, lx = vw - fw;
            gb[size_t(k) * a.P] = make_uint4(e, __builtin_bit_cast(uint32_t, ly),
                                             __builtin_bit_cast(uint32_t, lx * m[t]),
                                             __builtin_bit_cast(uint32_t, (1.0f - lx) * m[t]));
        }
    }
}

constexpr int kStagedThreads = 512;
constexpr int kMaxMg = 4;                    // output channels per input channel per pass

template <int ENT> struct EntryType;
template <> struct EntryType<16> { typedef uint4 type; };
template <> struct EntryType<8> { typedef uint2 type; };
template <> struct EntryType<4> { typedef uint32_t type; };
template <> struct EntryType<2> { typedef uint16_t type; };

// Channel ch of a staged entry, as fp32.
template <typename T, int ENT>
__device__ __forceinline__ float entry_at(const typename EntryType<ENT>::type &e, int ch)
{
    T v[ENT / sizeof(T)];
    __builtin_memcpy(v, &e, ENT);
    return to_f32(v[ch]);
}

// Buffer resource over `bytes` bytes at a uniform `base` (scalar registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dw_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t v = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
    void *p = reinterpret_cast<void *>((uint64_t(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, int(__builtin_amdgcn_readfirstlane(bytes)),
                                             0x00020000);
}

// One element at byte offset vo + so of a buffer.
template <typename T>
__device__ __forceinline__ T dw_load(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so)
{
    T v;
    if constexpr (sizeof(T) == 4) {
        const uint32_t b = __builtin_amdgcn_raw_buffer_load_b32(r, vo, int(so), 0);
        __builtin_memcpy(&v, &b, 4);
    } else {
        const uint16_t b = __builtin_amdgcn_raw_buffer_load_b16(r, vo, int(so), 0);
        __builtin_memcpy(&v, &b, 2);
    }
    return v;
}

template <typename T, int ENT, int UP, bool KT9, bool MG1>
__global__ __launch_bounds__(kStagedThreads) void depthwise_staged_kernel(
    const T *__restrict__ x, const uint4 *__restrict__ geo, const T *__restrict__ w,
    const T *__restrict__ bias, T *__restrict__ out, DwArgs a)
{
    constexpr int CH = ENT / int(sizeof(T));        // channels per entry
    using Ent = typename EntryType<ENT>::type;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int PW = a.W + 4, PH = a.H + 4;            // staged plane, entries
    const int tid = int(threadIdx.x);

    const uint32_t lid = xcd_swizzle(blockIdx.x, gridDim.x);
    const int n = __builtin_amdgcn_readfirstlane(int(lid / uint32_t(a.cblocks)));
    const int c0 = __builtin_amdgcn_readfirstlane(int(lid % uint32_t(a.cblocks)) * CH);
    const int ncb = min(CH, a.C - c0);

    // Stage: entry [r][cc] = channels c0 .. c0+CH-1 of x[r-2][cc-2], or 0 in
    // the ring (r < 2 or r >= H+2, cc < 2 or cc >= W+2) and past the last
    // channel.
    // Each thread takes SU entries kStagedThreads apart at a time and issues
    // all of their loads before writing any, so a whole batch of HBM reads is
    // in flight (one entry at a time would pay the full latency each time).
    {
        constexpr int SU = 8;
        const int NE = PH * PW;
        for (int e0 = tid; e0 < NE; e0 += SU * kStagedThreads) {
            T v[SU][CH];
#pragma unroll
            for (int su = 0; su < SU; ++su) {
                const int e = e0 + su * kStagedThreads;
                const int r = e / PW, cc = e - (e / PW) * PW;
                const int xr = r - 2, xc = cc - 2;
                const bool in = (e < NE) & (xr >= 0) & (xr < a.H) & (xc >= 0) & (xc < a.W);
#pragma unroll
                for (int ch = 0; ch < CH; ++ch)
                    v[su][ch] = (in && ch < ncb)
                                    ? x[(size_t(n) * a.C + c0 + ch) * a.HW + size_t(xr) * a.W + xc]
                                    : from_f32<T>(0.0f);
            }
#pragma unroll
            for (int su = 0; su < SU; ++su) {
                const int e = e0 + su * kStagedThreads;
                if (e < NE) {
                    Ent en;
                    __builtin_memcpy(&en, v[su], ENT);
                    *reinterpret_cast<Ent *>(lds + size_t(e) * ENT) = en;
                }
            }
        }
    }
    // With one output per channel and 3x3 taps, the workgroup's weights go
    // to LDS too, as fp32 [tap][channel], after the plane: one uniform read
    // per tap (in scalar registers, 9*CH of them would crowd out the rest).
    float *wtab = reinterpret_cast<float *>(lds + size_t(PH) * PW * ENT);
    if constexpr (MG1 && KT9) {
        for (int e = tid; e < 9 * CH; e += kStagedThreads) {
            const int k = e / CH, ch = e - (e / CH) * CH;
            wtab[e] = to_f32(w[size_t(min(c0 + ch, a.C - 1)) * 9 + k]);
        }
    }
    __syncthreads();

    const int q = c0 / a.Cdg;                        // every staged channel is in block q
    // This image's geometry of offset group q: per tap a row of P records.
    const uint32_t rowb = uint32_t(a.P) * 16u;
    const __amdgpu_buffer_rsrc_t rgeo =
        dw_rsrc(geo + (size_t(n) * a.DG + q) * size_t(a.K) * size_t(a.P), uint32_t(a.K) * rowb);
    const int mg_pass = MG1 ? 1 : kMaxMg;
    for (int m0 = 0; m0 < a.Mg; m0 += mg_pass) {
        const int nm = MG1 ? 1 : min(kMaxMg, a.Mg - m0);
        // One sample of one pixel for all CH channels: its four corner
        // entries and weights.  sample() issues the reads, blend()
        // accumulates.  A sample entirely off the image lands on ring zeros.
        struct Smp {
            Ent e00, e01, e10, e11;
            float w[4];
            float wk[CH];                            // tap weights (staged weights only)
        };
        auto sample = [&](Smp &sm, int k, const uint4 &g) {
            const float ly = __builtin_bit_cast(float, g.y);
            const float lxm = __builtin_bit_cast(float, g.z), hxm = __builtin_bit_cast(float, g.w);
            sm.w[0] = fmaf(-ly, hxm, hxm);
            sm.w[1] = fmaf(-ly, lxm, lxm);
            sm.w[2] = ly * hxm;
            sm.w[3] = ly * lxm;
            const char *pe = lds + g.x * uint32_t(ENT);
            sm.e00 = *reinterpret_cast<const Ent *>(pe);
            sm.e01 = *reinterpret_cast<const Ent *>(pe + ENT);
            sm.e10 = *reinterpret_cast<const Ent *>(pe + size_t(PW) * ENT);
            sm.e11 = *reinterpret_cast<const Ent *>(pe + size_t(PW + 1) * ENT);
            if constexpr (MG1 && KT9)
                __builtin_memcpy(sm.wk, wtab + k * CH, sizeof(sm.wk));
        };
        auto blend = [&](float (&acc)[CH][kMaxMg], const Smp &sm, int k) {
#pragma unroll
            for (int ch = 0; ch < CH; ++ch) {
                float v = sm.w[0] * entry_at<T, ENT>(sm.e00, ch);
                v = fmaf(sm.w[1], entry_at<T, ENT>(sm.e01, ch), v);
                v = fmaf(sm.w[2], entry_at<T, ENT>(sm.e10, ch), v);
                v = fmaf(sm.w[3], entry_at<T, ENT>(sm.e11, ch), v);
                if constexpr (MG1 && KT9) {
                    acc[ch][0] = fmaf(sm.wk[ch], v, acc[ch][0]);
                } else {
                    const int co = min(c0 + ch, a.C - 1) * a.Mg + m0;
#pragma unroll
                    for (int mm = 0; mm < kMaxMg; ++mm)
                        if (mm < nm)
                            acc[ch][mm] = fmaf(to_f32(w[size_t(co + mm) * a.K + k]), v,
                                               acc[ch][mm]);
                }
            }
        };
        // The accumulators are pinned after every blend (an empty asm that
        // claims to change them): their only use, the store, is conditional,
        // and the compiler would otherwise sink every blend into it, keeping
        // all the taps' corners live.
        auto pin = [&](float (&acc)[CH][kMaxMg]) {
#pragma unroll
            for (int ch = 0; ch < CH; ++ch)
#pragma unroll
                for (int mm = 0; mm < (MG1 ? 1 : kMaxMg); ++mm)
                    asm volatile("" : "+v"(acc[ch][mm]));
        };
        auto store = [&](const float (&acc)[CH][kMaxMg], int pix) {
#pragma unroll
            for (int ch = 0; ch < CH; ++ch) {
                if (ch >= ncb)
                    break;
#pragma unroll
                for (int mm = 0; mm < kMaxMg; ++mm) {
                    if (mm >= nm)
                        break;
                    const int co = (c0 + ch) * a.Mg + m0 + mm;
                    const float b = a.has_bias ? to_f32(bias[co]) : 0.0f;
                    out[(size_t(n) * a.Co + co) * a.P + pix] = from_f32<T>(acc[ch][mm] + b);
                }
            }
        };
        // One tap's geometry record: vector offset vo = the pixel's record in
        // row 0, scalar offset so = the tap's row.
        auto load_tap = [&](uint4 &g, uint32_t vo, uint32_t so) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rgeo, vo, int(so), 0);
            g = make_uint4(v[0], v[1], v[2], v[3]);
        };
        if constexpr (KT9) {
            // 3x3 taps, UP pixels per thread at a time.  One register set of
            // geometry records: as a tap's record is consumed, the same tap's
            // record of the next group of pixels is loaded into its place, so
            // each record has about a pixel's worth of taps to arrive.
            constexpr int STRIDE = UP * kStagedThreads;
            uint4 g[UP][9];
            int pb = tid;
#pragma unroll
            for (int u = 0; u < UP; ++u) {
                const uint32_t vo = uint32_t(min(pb + u * kStagedThreads, a.P - 1)) * 16u;
                // in tap order (the scheduler would otherwise reverse them,
                // and the first wait would then be for all of them)
#pragma unroll
                for (int k = 0; k < 9; ++k) {
                    load_tap(g[u][k], vo, uint32_t(k) * rowb);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            for (; pb < a.P; pb += STRIDE) {
#pragma unroll
                for (int u = 0; u < UP; ++u) {
                    // the next group's records (clamped: past the last pixel
                    // they are loaded and never used)
                    const uint32_t vn =
                        uint32_t(min(pb + STRIDE + u * kStagedThreads, a.P - 1)) * 16u;
                    float acc[CH][kMaxMg];
#pragma unroll
                    for (int ch = 0; ch < CH; ++ch)
#pragma unroll
                        for (int mm = 0; mm < kMaxMg; ++mm)
                            acc[ch][mm] = 0.0f;
                    // Taps software-pipelined: tap k+1's corner reads are
                    // issued before tap k's blend, so the LDS latency overlaps
                    // arithmetic.
                    Smp sp[2];
                    sample(sp[0], 0, g[u][0]);
                    load_tap(g[u][0], vn, 0u);
#pragma unroll
                    for (int k = 0; k < 9; ++k) {
                        if (k < 8) {
                            sample(sp[(k + 1) & 1], k + 1, g[u][k + 1]);
                            load_tap(g[u][k + 1], vn, uint32_t(k + 1) * rowb);
                        }
                        blend(acc, sp[k & 1], k);
                        pin(acc);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    if (pb + u * kStagedThreads < a.P)
                        store(acc, pb + u * kStagedThreads);
                }
            }
        } else {
            for (int pix = tid; pix < a.P; pix += kStagedThreads) {
                float acc[CH][kMaxMg];
#pragma unroll
                for (int ch = 0; ch < CH; ++ch)
#pragma unroll
                    for (int mm = 0; mm < kMaxMg; ++mm)
                        acc[ch][mm] = 0.0f;
                const uint32_t vo = uint32_t(pix) * 16u;
                uint32_t so = 0;
                for (int k = 0; k < a.K; ++k) {
                    uint4 g;
                    load_tap(g, vo, so);
                    so += rowb;
                    Smp sm;
                    sample(sm, k, g);
                    blend(acc, sm, k);
                    pin(acc);
                }
                store(acc, pix);
            }
        }
    }
}

// Persistent kernel for the common depthwise case: 3x3 taps and one output
// per input channel, at most 4 channels per staged entry.  A workgroup takes
// a run of consecutive channel blocks (of one image, where the run allows)
// and keeps its LDS plane busy: 8 waves compute one block while 4 loader
// waves read the next block's plane into their registers (kPersLoadBytes per
// loader thread), so that after the first block the HBM reads of x overlap
// the LDS-bound sampling; between blocks the loaders write the plane's
// interior (the zero ring stays).
//
// Compute waves take groups of 64 pixels (one per lane) from a counter in
// LDS, so that waves slowed by LDS contention take fewer; the geometry
// records of a wave's next group are loaded tap by tap as the current
// group's records are used, and tap k+1's corner reads go out before tap
// k's blend.  The tap weights and the bias live in scalar registers, not in
// LDS: a broadcast LDS read still returns a whole wave's worth of data.
constexpr int kPersCompute = 512;
constexpr int kPersLoad = 256;
constexpr int kPersThreads = kPersCompute + kPersLoad;
constexpr int kPersLoadBytes = 576;

template <typename T, int ENT>
__global__ __launch_bounds__(kPersThreads) void depthwise_persistent_kernel(
    const T *__restrict__ x, const uint4 *__restrict__ geo, const T *__restrict__ w,
    const T *__restrict__ bias, T *__restrict__ out, DwArgs a)
{
    constexpr int CH = ENT / int(sizeof(T));         // channels per entry
    constexpr int SLOTS = kPersLoadBytes / ENT;      // plane positions per loader thread
    static_assert(CH <= 4, "tap weights of at most 4 channels stay in registers");
    using Ent = typename EntryType<ENT>::type;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int PW = a.W + 4, PH = a.H + 4;
    const int tid = int(threadIdx.x);
    // pixel-group counter of the compute waves, after the plane
    uint32_t *ctr = reinterpret_cast<uint32_t *>(lds + size_t(PH) * PW * ENT);

    // this workgroup's channel blocks [b_lo, b_hi) of the (image, block) sequence
    const uint32_t lid = xcd_swizzle(blockIdx.x, gridDim.x);
    const uint64_t nblk = uint64_t(a.N) * uint64_t(a.cblocks);
    const int b_lo = __builtin_amdgcn_readfirstlane(int(uint64_t(lid) * nblk / gridDim.x));
    const int b_hi = __builtin_amdgcn_readfirstlane(int(uint64_t(lid + 1) * nblk / gridDim.x));
    if (b_lo >= b_hi)
        return;

    // First block: the whole plane, ring included, by every thread (as in
    // the staged kernel: SU entries per thread in flight at a time).
    if (tid == 0)
        *ctr = 0u;
    {
        const int n = b_lo / a.cblocks, c0 = (b_lo % a.cblocks) * CH;
        const int ncb = min(CH, a.C - c0);
        constexpr int SU = 8;
        const int NE = PH * PW;
        for (int e0 = tid; e0 < NE; e0 += SU * kPersThreads) {
            T v[SU][CH];
#pragma unroll
            for (int su = 0; su < SU; ++su) {
                const int e = e0 + su * kPersThreads;
                const int r = e / PW, cc = e - (e / PW) * PW;
                const int xr = r - 2, xc = cc - 2;
                const bool in = (e < NE) & (xr >= 0) & (xr < a.H) & (xc >= 0) & (xc < a.W);
#pragma unroll
                for (int ch = 0; ch < CH; ++ch)
                    v[su][ch] = (in && ch < ncb)
                                    ? x[(size_t(n) * a.C + c0 + ch) * a.HW + size_t(xr) * a.W + xc]
                                    : from_f32<T>(0.0f);
            }
#pragma unroll
            for (int su = 0; su < SU; ++su) {
                const int e = e0 + su * kPersThreads;
                if (e < NE) {
                    Ent en;
                    __builtin_memcpy(&en, v[su], ENT);
                    *reinterpret_cast<Ent *>(lds + size_t(e) * ENT) = en;
                }
            }
        }
    }
    __syncthreads();

    const uint32_t rowb = uint32_t(a.P) * 16u;
    // The two roles run loops of their own (their registers never overlap)
    // with the same barriers: after each block's sampling, and after the
    // next block's plane is in LDS.
    if (__builtin_amdgcn_readfirstlane(tid) >= kPersCompute) {
        const int lt = tid - kPersCompute;
        // plane row of a position (exact for pos * W < 2^32)
        auto row_of = [&](int pos) {
            return a.W > 1 ? int(__umulhi(uint32_t(pos), a.w_magic)) : pos;
        };
        for (int b = b_lo; b + 1 < b_hi; ++b) {
            // the next block's plane interior into registers; position
            // j*kPersLoad + lt of the image plane, all CH channels
            const int n = (b + 1) / a.cblocks, c0 = ((b + 1) % a.cblocks) * CH;
            const int ncb = min(CH, a.C - c0);
            // one buffer per channel plane: reads past the plane, and every
            // read of a channel past the last, return 0
            __amdgpu_buffer_rsrc_t rx[CH];
#pragma unroll
            for (int ch = 0; ch < CH; ++ch)
                rx[ch] = dw_rsrc(x + (size_t(n) * a.C + c0 + min(ch, ncb - 1)) * a.HW,
                                 ch < ncb ? uint32_t(a.HW) * uint32_t(sizeof(T)) : 0u);
            if constexpr (sizeof(T) == 4) {
                Ent R[SLOTS];
                uint32_t vo = uint32_t(lt) * 4u;
#pragma unroll
                for (int j = 0; j < SLOTS; ++j) {
                    T v[CH];
#pragma unroll
                    for (int ch = 0; ch < CH; ++ch)
                        v[ch] = dw_load<T>(rx[ch], vo, 0);
                    __builtin_memcpy(&R[j], v, ENT);
                    // one offset register, stepped (not one per slot)
                    vo += uint32_t(kPersLoad) * 4u;
                    asm volatile("" : "+v"(vo));
                }
                __syncthreads();                     // block b's sampling is done
                int pos = lt;
#pragma unroll
                for (int j = 0; j < SLOTS; ++j, pos += kPersLoad) {
                    // addresses one slot at a time (not all hoisted beside R)
                    asm volatile("" : "+v"(pos));
                    if (pos < a.HW) {
                        const int xr = row_of(pos), xc = pos - xr * a.W;
                        const size_t e = size_t(xr + 2) * PW + xc + 2;
                        *reinterpret_cast<Ent *>(lds + e * ENT) = R[j];
                    }
                }
            } else {
                // 16-bit values: one 4-byte read per channel covers the
                // positions 2p and 2p+1 (the plane has an even size); the
                // halves are sorted into the two entries when written
                constexpr int PAIRS = kPersLoadBytes / 4 / CH;
                uint32_t R[PAIRS][CH];
                uint32_t vo = uint32_t(lt) * 4u;
#pragma unroll
                for (int j = 0; j < PAIRS; ++j) {
#pragma unroll
                    for (int ch = 0; ch < CH; ++ch)
                        R[j][ch] = __builtin_amdgcn_raw_buffer_load_b32(rx[ch], vo, 0, 0);
                    vo += uint32_t(kPersLoad) * 4u;
                    asm volatile("" : "+v"(vo));
                }
                __syncthreads();                     // block b's sampling is done
                int pos = 2 * lt;
#pragma unroll
                for (int j = 0; j < PAIRS; ++j, pos += 2 * kPersLoad) {
                    asm volatile("" : "+v"(pos));
                    if (pos < a.HW) {
                        uint32_t lo[CH / 2], hi[CH / 2];
#pragma unroll
                        for (int c = 0; c < CH / 2; ++c) {
                            const uint32_t u = R[j][2 * c], v = R[j][2 * c + 1];
                            lo[c] = __builtin_amdgcn_perm(v, u, 0x05040100u);
                            hi[c] = __builtin_amdgcn_perm(v, u, 0x07060302u);
                        }
                        Ent e0, e1;
                        __builtin_memcpy(&e0, lo, ENT);
                        __builtin_memcpy(&e1, hi, ENT);
                        const int xr = row_of(pos), xc = pos - xr * a.W;
                        const size_t f0 = size_t(xr + 2) * PW + xc + 2;
                        *reinterpret_cast<Ent *>(lds + f0 * ENT) = e0;
                        const int p1 = pos + 1;
                        const int yr = row_of(p1), yc = p1 - yr * a.W;
                        const size_t f1 = size_t(yr + 2) * PW + yc + 2;
                        *reinterpret_cast<Ent *>(lds + f1 * ENT) = e1;
                    }
                }
            }
            __syncthreads();                         // block b+1's plane is staged
        }
        return;
    }
    for (int b = b_lo; b < b_hi; ++b) {
        const int n = b / a.cblocks, c0 = (b % a.cblocks) * CH;
        const int ncb = min(CH, a.C - c0);
        const int q = c0 / a.Cdg;
        const __amdgpu_buffer_rsrc_t rgeo =
            dw_rsrc(geo + (size_t(n) * a.DG + q) * 9 * size_t(a.P), 9u * rowb);
        float wk[9][CH];                             // tap weights
#pragma unroll
        for (int k = 0; k < 9; ++k)
#pragma unroll
            for (int ch = 0; ch < CH; ++ch)
                wk[k][ch] = to_f32(w[size_t(min(c0 + ch, a.C - 1)) * 9 + k]);
        float bz[CH];                                // bias (scalar loads before the loop)
#pragma unroll
        for (int ch = 0; ch < CH; ++ch)
            bz[ch] = a.has_bias ? to_f32(bias[min(c0 + ch, a.C - 1)]) : 0.0f;
        if constexpr (sizeof(T) == 4) {
            // the scalar loads land before the sampling loop: a scalar load
            // still in flight there would make every LDS wait a full drain
#pragma unroll
            for (int k = 0; k < 9; ++k)
#pragma unroll
                for (int ch = 0; ch < CH; ++ch)
                    asm volatile("" : "+s"(wk[k][ch]));
#pragma unroll
            for (int ch = 0; ch < CH; ++ch)
                asm volatile("" : "+s"(bz[ch]));
        }

        struct Smp {
            Ent e00, e01, e10, e11;
            float w[4];
        };
        auto sample = [&](Smp &sm, const uint4 &g) {
            const float ly = __builtin_bit_cast(float, g.y);
            const float lxm = __builtin_bit_cast(float, g.z);
            const float hxm = __builtin_bit_cast(float, g.w);
            sm.w[0] = fmaf(-ly, hxm, hxm);
            sm.w[1] = fmaf(-ly, lxm, lxm);
            sm.w[2] = ly * hxm;
            sm.w[3] = ly * lxm;
            // computed here, while the record is live (not sunk to the blend)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                asm volatile("" : "+v"(sm.w[c]));
            const char *pe = lds + g.x * uint32_t(ENT);
            sm.e00 = *reinterpret_cast<const Ent *>(pe);
            sm.e01 = *reinterpret_cast<const Ent *>(pe + ENT);
            sm.e10 = *reinterpret_cast<const Ent *>(pe + size_t(PW) * ENT);
            sm.e11 = *reinterpret_cast<const Ent *>(pe + size_t(PW + 1) * ENT);
        };
        auto blend = [&](float (&acc)[CH], const Smp &sm, int k) {
#pragma unroll
            for (int ch = 0; ch < CH; ++ch) {
                float v = sm.w[0] * entry_at<T, ENT>(sm.e00, ch);
                v = fmaf(sm.w[1], entry_at<T, ENT>(sm.e01, ch), v);
                v = fmaf(sm.w[2], entry_at<T, ENT>(sm.e10, ch), v);
                v = fmaf(sm.w[3], entry_at<T, ENT>(sm.e11, ch), v);
                acc[ch] = fmaf(wk[k][ch], v, acc[ch]);
            }
        };
        auto load_tap = [&](uint4 &g, int pix, int k) {
            const uint32_t vo = uint32_t(min(pix, a.P - 1)) * 16u;
            const auto v =
                __builtin_amdgcn_raw_buffer_load_b128(rgeo, vo, int(uint32_t(k) * rowb), 0);
            g = make_uint4(v[0], v[1], v[2], v[3]);
        };
        auto store = [&](const float (&acc)[CH], int pix) {
#pragma unroll
            for (int ch = 0; ch < CH; ++ch)
                if (ch < ncb)
                    out[(size_t(n) * a.Co + c0 + ch) * a.P + pix] = from_f32<T>(acc[ch] + bz[ch]);
        };
        // Pixels go out in groups of 64 (one per lane of a wave) from a
        // counter in LDS, so that waves slowed by LDS contention take fewer
        // groups and all finish together.  A wave knows its next group
        // while it works on the current one (the next group's geometry
        // records are loaded tap by tap as the current ones are used) and
        // draws the one after that at the end of each group, when it has no
        // LDS reads in flight.
        const int lane = tid & 63;
        const uint32_t ngroups = uint32_t(a.P + 63) / 64u;
        auto draw = [&]() {
            uint32_t v = 0;
            if (lane == 0)
                v = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            return __builtin_amdgcn_readfirstlane(v);
        };
        uint32_t cur = draw();
        uint32_t nxt = draw();
        // g[k]: the record of tap k of the next sample of tap k, in tap order
        uint4 g[9];
#pragma unroll
        for (int k = 0; k < 9; ++k) {
            load_tap(g[k], int(cur * 64u) + lane, k);
            __builtin_amdgcn_sched_barrier(0);
        }
        while (cur < ngroups) {
            const int pix = int(cur * 64u) + lane;
            const int npix = int(nxt * 64u) + lane;
            float acc[CH];
#pragma unroll
            for (int ch = 0; ch < CH; ++ch)
                acc[ch] = 0.0f;
            // taps software-pipelined: tap k+1's corner reads go out before
            // tap k's blend
            Smp sp[2];
            sample(sp[0], g[0]);
            __builtin_amdgcn_sched_barrier(0);
            load_tap(g[0], npix, 0);
#pragma unroll
            for (int k = 0; k < 9; ++k) {
                if (k < 8) {
                    sample(sp[(k + 1) & 1], g[k + 1]);
                    // the record is consumed before its registers are reloaded
                    __builtin_amdgcn_sched_barrier(0);
                    load_tap(g[k + 1], npix, k + 1);
                }
                __builtin_amdgcn_sched_barrier(0);   // the reads go out first
                blend(acc, sp[k & 1], k);
#pragma unroll
                for (int ch = 0; ch < CH; ++ch)
                    asm volatile("" : "+v"(acc[ch]));
                __builtin_amdgcn_sched_barrier(0);
            }
            if (pix < a.P)
                store(acc, pix);
            cur = nxt;
            nxt = draw();
        }
        // the loaders wait here (twice per block but the last) until the
        // plane is no longer read, then stage the next one
        if (b + 1 < b_hi) {
            __syncthreads();                         // the plane is no longer read
            if (tid == 0)
                *ctr = 0u;
            __syncthreads();                         // the next block's plane is staged
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
using DwKernel = void (*)(const T *, const uint4 *, const T *, const T *, T *, DwArgs);

// The staged kernel instance for (entry bytes, pixels per thread, 3x3 taps,
// exactly one output per input channel).
template <typename T>
DwKernel<T> staged_fn(int ent, int up, bool kt9, bool mg1)
{
#define MDCN_DW_PICK(ENT_, UP_)                                                                \
    if (ent == ENT_ && up == UP_) {                                                            \
        if (kt9)                                                                               \
            return mg1 ? &depthwise_staged_kernel<T, ENT_, UP_, true, true>                    \
                       : &depthwise_staged_kernel<T, ENT_, UP_, true, false>;                  \
        return mg1 ? &depthwise_staged_kernel<T, ENT_, UP_, false, true>                       \
                   : &depthwise_staged_kernel<T, ENT_, UP_, false, false>;                     \
    }
    MDCN_DW_PICK(16, 1) MDCN_DW_PICK(16, 2) MDCN_DW_PICK(8, 1) MDCN_DW_PICK(8, 2)
    MDCN_DW_PICK(4, 1) MDCN_DW_PICK(4, 2)
    if constexpr (sizeof(T) == 2) {
        MDCN_DW_PICK(2, 1) MDCN_DW_PICK(2, 2)
    }
#undef MDCN_DW_PICK
    return nullptr;
}

// The persistent kernel instance for an entry width (4 bytes or more, at
// most 4 channels).
template <typename T>
DwKernel<T> pers_fn(int ent)
{
    if constexpr (sizeof(T) == 4) {
        if (ent == 16)
            return &depthwise_persistent_kernel<T, 16>;
    }
    if (ent == 8)
        return &depthwise_persistent_kernel<T, 8>;
    if (ent == 4)
        return &depthwise_persistent_kernel<T, 4>;
    return nullptr;
}

template <typename T>
hipError_t depthwise_t(const Problem &p, int64_t cnt, const void *x, const void *geo,
                       const void *offset, const void *mask, const void *weight, const void *bias,
                       void *out, hipStream_t s)
{
    DwArgs a;
    a.total = uint32_t(p.Co * p.P);
    a.N = int(cnt); a.C = int(p.C); a.H = int(p.H); a.W = int(p.W); a.HW = int(p.H * p.W);
    a.Co = int(p.Co); a.Mg = int(p.Mg); a.Cdg = int(p.Cdg); a.K = int(p.K); a.P = int(p.P);
    a.Wo = int(p.Wo); a.kw = int(p.kw);
    a.sh = int(p.sh); a.sw = int(p.sw); a.ph = int(p.ph); a.pw = int(p.pw);
    a.dh = int(p.dh); a.dw = int(p.dw);
    a.offC = int(2 * p.DG * p.K); a.mskC = int(p.DG * p.K);
    a.has_bias = bias != nullptr;
    a.DG = int(p.DG);
    a.w_magic = p.W > 1 ? uint32_t((uint64_t(1) << 32) / uint64_t(p.W) + 1) : 0u;
    // The widest allowed entry, one pixel per thread at a time with the next
    // one's geometry in flight.  MDCN_DW_ENTRY=<bytes> and MDCN_DW_PIXELS=1|2
    // override (for tuning), where allowed.
    int ent = dw_default_entry(p), up = 1;
    if (const char *env = std::getenv("MDCN_DW_ENTRY")) {
        const int v = std::atoi(env);
        if ((v == 16 || v == 8 || v == 4 || v == 2) && dw_entry_allowed(p, v))
            ent = v;
    }
    if (const char *env = std::getenv("MDCN_DW_PIXELS")) {
        const int v = std::atoi(env);
        if (v == 1 || v == 2)
            up = v;
    }
    const bool kt9 = p.kh == 3 && p.kw == 3, mg1 = p.Mg == 1;
    // 3x3 taps, one output per input channel, entries of 4 bytes or more and
    // a plane the loader waves can hold: the persistent kernel
    // (MDCN_DW_PERSISTENT=0 turns it off, for tuning)
    // (at most 4 channels per entry: 8-byte entries for fp16/bf16).
    // MDCN_DW_PERSISTENT=0 turns it off, MDCN_DW_PERSISTENT_BLOCKS=<n> sets
    // the channel blocks per workgroup (for tuning).
    const int pent = std::min(ent, 4 * int(sizeof(T)));
    bool pers = kt9 && mg1 && pent >= 4 && geo != nullptr &&
                p.H * p.W <= int64_t(kPersLoad) * (kPersLoadBytes / pent) &&
                (sizeof(T) == 4 || (p.H * p.W) % 2 == 0);
    if (const char *env = std::getenv("MDCN_DW_PERSISTENT"))
        pers = pers && std::atoi(env) != 0;
    if (pers) {
        const int ch = pent / int(sizeof(T));
        a.cblocks = int((p.C + ch - 1) / ch);
        const int64_t nblk = cnt * a.cblocks;
        const int64_t cus = std::max(1, device_cu_count());
        int64_t per = (nblk + cus - 1) / cus;
        if (const char *env = std::getenv("MDCN_DW_PERSISTENT_BLOCKS"))
            per = std::max<int64_t>(1, std::atoi(env));
        const dim3 grid(unsigned((nblk + per - 1) / per));
        const size_t lds = size_t(p.H + 4) * size_t(p.W + 4) * size_t(pent) + 16;
        const DwKernel<T> fn = pers_fn<T>(pent);
        if (fn != nullptr &&
            hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) == hipSuccess) {
            hipLaunchKernelGGL(fn, grid, dim3(kPersThreads), lds, s, static_cast<const T *>(x),
                               static_cast<const uint4 *>(geo),
                               static_cast<const T *>(weight), static_cast<const T *>(bias),
                               static_cast<T *>(out), a);
            return hipGetLastError();
        }
        (void)hipGetLastError();           // clear it; use the staged kernel below
    }
    if (ent > 0 && geo != nullptr) {
        const int ch = ent / int(sizeof(T));
        a.cblocks = int((p.C + ch - 1) / ch);
        const dim3 grid(unsigned(uint64_t(cnt) * a.cblocks));
        const size_t lds = size_t(p.H + 4) * size_t(p.W + 4) * size_t(ent) +
                           9 * size_t(ch) * sizeof(float);
        const DwKernel<T> fn = staged_fn<T>(ent, up, kt9, mg1);
        if (fn != nullptr &&
            hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) == hipSuccess) {
            hipLaunchKernelGGL(fn, grid, dim3(kStagedThreads), lds, s, static_cast<const T *>(x),
                               static_cast<const uint4 *>(geo),
                               static_cast<const T *>(weight), static_cast<const T *>(bias),
                               static_cast<T *>(out), a);
            return hipGetLastError();
        }
        (void)hipGetLastError();           // clear it; use the plain kernel below
    }
    const dim3 grid((a.total + 255u) / 256u, unsigned(std::min<int64_t>(cnt, 65535)));
    hipLaunchKernelGGL(depthwise_kernel<T>, grid, dim3(256), 0, s, static_cast<const T *>(x),
                       static_cast<const T *>(offset), static_cast<const T *>(mask),
                       static_cast<const T *>(weight), static_cast<const T *>(bias),
                       static_cast<T *>(out), a);
    return hipGetLastError();
}

template <typename T>
hipError_t dw_geometry_t(const Problem &p, int64_t cnt, const void *offset, const void *mask,
                         void *geo, hipStream_t s)
{
    DwGeoArgs a;
    a.groups = uint32_t(cnt * p.DG);
    a.P = int(p.P); a.Wo = int(p.Wo); a.K = int(p.K); a.kw = int(p.kw); a.DG = int(p.DG);
    a.H = int(p.H); a.W = int(p.W); a.PW = int(p.W + 4);
    a.sh = int(p.sh); a.sw = int(p.sw); a.ph = int(p.ph); a.pw = int(p.pw);
    a.dh = int(p.dh); a.dw = int(p.dw);
    a.offC = int(2 * p.DG * p.K); a.mskC = int(p.DG * p.K);
    const unsigned tgroups = unsigned((p.K + kGeoTaps - 1) / kGeoTaps);
    const dim3 grid(unsigned((p.P + kGeoThreads - 1) / kGeoThreads),
                    unsigned(std::min<uint64_t>(uint64_t(a.groups) * tgroups, 65535u)));
    hipLaunchKernelGGL(dw_geometry_kernel<T>, grid, dim3(kGeoThreads), 0, s,
                       static_cast<const T *>(offset), static_cast<const T *>(mask),
                       static_cast<uint4 *>(geo), a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_depthwise(const Problem &p, int64_t cnt, const void *x, const void *geo,
                            const void *offset, const void *mask, const void *weight,
                            const void *bias, void *out, hipStream_t stream)
{
    switch (p.dtype) {
    case MDCN_F32:
        return depthwise_t<float>(p, cnt, x, geo, offset, mask, weight, bias, out, stream);
    case MDCN_F16:
        return depthwise_t<half_t>(p, cnt, x, geo, offset, mask, weight, bias, out, stream);
    case MDCN_BF16:
        return depthwise_t<bf16_t>(p, cnt, x, geo, offset, mask, weight, bias, out, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_dw_geometry(const Problem &p, int64_t cnt, const void *offset,
                              const void *mask, void *geo, hipStream_t stream)
{
    switch (p.dtype) {
    case MDCN_F32: return dw_geometry_t<float>(p, cnt, offset, mask, geo, stream);
    case MDCN_F16: return dw_geometry_t<half_t>(p, cnt, offset, mask, geo, stream);
    case MDCN_BF16: return dw_geometry_t<bf16_t>(p, cnt, offset, mask, geo, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mdcn
