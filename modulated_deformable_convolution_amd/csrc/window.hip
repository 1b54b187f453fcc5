// window.hip -- the deformable gather fused into the MFMA GEMM, with the
// input window of each output tile staged in LDS.
//   out[n][g*Mg + m][ho][wo] = bias[g*Mg + m]
//       + sum_{k, c'} A[g][m][k*Cg + c'] * mask * bilinear0(x[n][g*Cg + c'], sample(k, ho, wo))
// [plugin guide §五 steps 1-3, without a columns buffer between step 1 and 2].
//
// A tile is 256 output channels of one image and group x 256 output pixels:
// a TH x TW rectangle, or (TH = 1, narrow images) 256 consecutive pixels in
// raster order.  The contraction runs chunk-major: for each chunk of 16 input
// channels, the rectangle of input pixels that the tile's samples can reach
// -- the anchors of all taps plus a margin of `margin` pixels on every side
// for the offsets -- is copied into LDS once (the "window", channels-last,
// two planes of 8 channels), and the 9 taps of the chunk are then 9 K-steps
// that read their bilinear corners from it.  A sample with a corner on the
// image that falls outside the window is rare with the margin sized for the
// offsets; its lane reads zeros from the window and its value is computed
// from global memory instead (the fallback), so the result does not depend
// on the margin.
//
// The grid is persistent, one workgroup (4 waves, one per SIMD) per CU.  The
// (tile, chunk) units are cut into contiguous per-workgroup ranges on the
// host (balanced for chunks plus a per-tile cost); a workgroup walks the
// tiles of its range from last to first.  A tile split between two
// workgroups is finished by the one holding its last chunks: the other
// publishes its accumulators (device-scope stores, then a flag) on the first
// tile it processes, and the finisher loads them into its accumulators on
// the last one.
//
// Every wave owns 64 pixels (two slabs of 32) and all 256 output channels:
// it makes the B fragments of its own pixels in registers (lane l of a slab
// owns pixel l%32 and channels 8*(l/32)..+8 of the chunk, which is exactly
// the MFMA B-fragment layout), so B never goes through LDS, and reads the A
// fragments (packed weight rows) from LDS stages filled by DMA LEAD steps
// ahead.  The per-lane sampling geometry of all taps (window address of the
// top-left corner, four weights with the mask folded in) is computed once per
// tile and kept in registers.  In each step the MFMAs of step s run beside
// the bilinear blend of step s+1 and the LDS reads of step s+2.
//
// Both operands come in layouts that make every LDS copy contiguous (a copy
// instruction's cost on the texture path grows with the cache lines it
// touches): x in 8-channel blocks [C/8][H][W][8] per image, so the window of
// one chunk is two planes of contiguous row runs, and the weight step-major,
// [G][S][2][Mg][8] (S = 9 * C/group/16 steps, two 8-channel halves), so the A
// tile of a step is two contiguous 4 KiB planes.
//
// The LDS copies are issued as inline-assembly DMA (buffer_load ... lds): the
// waits for them are explicit (s_waitcnt vmcnt + barrier), so the compiler,
// which does not see them, cannot make LDS reads wait for unrelated copies.
#include <algorithm>
#include <map>
#include <mutex>
#include <type_traits>

#include "launch.h"
#include "mfma_common.h"

namespace mdcn {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kCC = 16;                       // channels per chunk = one MFMA k-group
constexpr int kTaps = 9;                      // 3x3 kernels
constexpr uint32_t kOOB = 0x80000000u;        // a byte offset past every buffer range

// LDS layout (bytes):
//   window buffer b (b = 0, 1): [plane 0: kWinPx x 16][gap][plane 1: kWinPx x 16][zeros]
//   window copy table:          [instruction t][thread]: source byte offset of the
//                               thread's 16 bytes of window copy instruction t
//   parked tile index:          one word per wave (256 bytes reserved)
//   A stage s (s = 0..LEAD):    [plane 0: 256 rows x 16][plane 1: 256 rows x 16]
// Plane p of an entry holds channels 8p..8p+7 of the chunk.
constexpr int kWinPlane = kWindowPixels * 16;
// Plane 1 starts this many bytes past the end of plane 0, so that lanes
// reading the two planes at the same position use different LDS banks.
constexpr int kPlaneGap = 128;
constexpr int kPlane1 = kWinPlane + kPlaneGap;          // start of plane 1
constexpr int kWinZeroOff = kPlane1 + kWinPlane;        // start of the zero area
constexpr int kWinZero = kWindowZeroBytes;
constexpr int kWinBuf = kWinZeroOff + kWinZero;
constexpr int kAStage = 256 * 2 * 16;
constexpr int kWinInstr = 2 * kWindowPixels / 64 / 4;   // window DMA instructions per wave
constexpr int kWoffOff = 2 * kWinBuf;
constexpr int kParkOff = kWoffOff + kWinInstr * 256 * 4;  // 4 words: a tile index per wave
constexpr int kAOff = kParkOff + 256;
// A stages: the copy of step s+LEAD is issued in step s, into one of LEAD+1
// stages.
constexpr int lds_total(int lead) { return kAOff + (lead + 1) * kAStage; }
constexpr int kAInstr = kAStage / 1024 / 4;             // A DMA instructions per wave
constexpr int kEpRow = 256 + 4;                          // epilogue slice row, floats
// Cache-policy operand of a buffer access with device scope (the SC1 bit on
// gfx950): a store is written through to where every XCD sees it and a load
// is served from there.  The partial sums passed between workgroups use it,
// so no whole-L2 writeback or invalidate is needed on either side.
constexpr int kDevScope = 16;
static_assert(lds_total(kWindowMaxLead) <= int(kLdsBytes), "LDS budget");
static_assert(32 * kEpRow * 4 <= lds_total(2), "epilogue slice must fit");
static_assert(kWindowPixels % 128 == 0,
              "window DMA covers whole wave instructions, none straddling the two planes");

struct WinArgs {
    const void *A, *xt, *off, *msk, *bias;   // step-major weight, x blocks, offset, mask, bias|null
    void *out;
    float *partial;                          // partial-sum slots
    uint32_t *flags;                         // one flag per slot
    int Mg, Kp, Co, P, Ho, Wo;
    int C, H, W, Cg, nch;          // nch: chunks of 16 channels per group
    int sh, sw, ph, pw, dh, dw;
    int margin, WR, WC;            // window rows / columns
    int tiles_x, tiles_y, tiles_m, cnt, tiles;
    int epoch;                     // value that marks partial sums published by this launch
    int offC, mskC, Cdg;           // offset / mask channels per image; C / deformable_group
    int has_bias, vec_out;
    uint32_t img_bytes, chunk_bytes, a_bytes;
    // unit range of each workgroup slot (slot j = run * per + index in run)
    uint32_t bounds[kWindowSlots + 1];
};
static_assert(sizeof(WinArgs) <= 4096, "kernel arguments are at most 4 KiB");

// The kernel's only argument, read through a pointer into the kernarg
// segment that the compiler cannot see through at each use site: every
// region (set-up, tile prologue, fallback, epilogue) loads the fields it needs
// with scalar loads instead of keeping them in registers across the main
// loop, where scalar registers are scarce.
typedef const WinArgs __attribute__((address_space(4))) *KArgs;
__device__ __forceinline__ KArgs fresh_args(KArgs p)
{
    asm volatile("" : "+s"(p));
    return p;
}

// Buffer resource (4 scalar registers) over `bytes` bytes at `base`.
__device__ __forceinline__ v4i srd(const void *base, uint32_t bytes)
{
    const uint64_t v = reinterpret_cast<uint64_t>(base);
    v4i r;
    r.x = int(__builtin_amdgcn_readfirstlane(uint32_t(v)));
    r.y = int(__builtin_amdgcn_readfirstlane(uint32_t(v >> 32)));
    r.z = int(__builtin_amdgcn_readfirstlane(bytes));
    r.w = 0x00020000;
    return r;
}

// The same as a buffer resource value for the buffer load/store builtins.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t srd_b(const void *base, uint32_t bytes)
{
    const uint64_t v = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
    void *p = reinterpret_cast<void *>((uint64_t(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0,
                                             int(__builtin_amdgcn_readfirstlane(bytes)),
                                             0x00020000);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16 bytes per lane from buffer offset voff + soff into LDS at lds + 16*lane.
// The compiler does not see this write to LDS; callers wait with vmcnt and
// a barrier before any wave reads the data.
__device__ __forceinline__ void dma16(uint32_t lds, v4i rsrc, uint32_t voff, uint32_t soff)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return uint32_t(reinterpret_cast<uintptr_t>((const lds_void *)p));
}

typedef float float2v __attribute__((ext_vector_type(2)));

// Two fp32 values rounded (to nearest even) into one register of T pairs.
template <typename T> __device__ __forceinline__ uint32_t pack2(float a, float b);
template <> __device__ __forceinline__ uint32_t pack2<half_t>(float a, float b)
{
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 r = __builtin_convertvector((float2v){a, b}, h2);
    uint32_t o;
    __builtin_memcpy(&o, &r, 4);
    return o;
}
template <> __device__ __forceinline__ uint32_t pack2<bf16_t>(float a, float b)
{
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const b2 r = __builtin_convertvector((float2v){a, b}, b2);
    uint32_t o;
    __builtin_memcpy(&o, &r, 4);
    return o;
}

// Elements 2p, 2p+1 of the lane's 8 channels of a sample (see blend).
template <typename T>
__device__ __forceinline__ uint32_t blend_pair(const uint4 (&c)[4], const float (&w)[4],
                                               float zero, int p)
{
    float acc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int e = 2 * p + h;
        Vec16<T> v0, v1, v2, v3;
        v0.raw = c[0]; v1.raw = c[1]; v2.raw = c[2]; v3.raw = c[3];
        acc[h] = fmaf(to_f32(v0.e[e]), w[0], zero);
        acc[h] = fmaf(to_f32(v1.e[e]), w[1], acc[h]);
        acc[h] = fmaf(to_f32(v2.e[e]), w[2], acc[h]);
        acc[h] = fmaf(to_f32(v3.e[e]), w[3], acc[h]);
    }
    return pack2<T>(acc[0], acc[1]);
}

// The lane's 8 channels of a sample: four corner chunks weighted and summed
// in fp32, one rounding to T.  `zero` is 0.0f that the compiler cannot see
// through, so the first product is a mixed-precision FMA too (x*w + 0 is
// x*w up to the sign of a zero).
template <typename T>
__device__ __forceinline__ uint4 blend(const uint4 &c0, const uint4 &c1, const uint4 &c2,
                                       const uint4 &c3, const float (&w)[4], float zero)
{
    Vec16<T> v0, v1, v2, v3;
    v0.raw = c0; v1.raw = c1; v2.raw = c2; v3.raw = c3;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        acc[e] = fmaf(to_f32(v0.e[e]), w[0], zero);
        acc[e] = fmaf(to_f32(v1.e[e]), w[1], acc[e]);
        acc[e] = fmaf(to_f32(v2.e[e]), w[2], acc[e]);
        acc[e] = fmaf(to_f32(v3.e[e]), w[3], acc[e]);
    }
    return make_uint4(pack2<T>(acc[0], acc[1]), pack2<T>(acc[2], acc[3]),
                      pack2<T>(acc[4], acc[5]), pack2<T>(acc[6], acc[7]));
}

template <typename T, int TH, int TW, int LEAD>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void window_kernel(WinArgs args)
{
    (void)args;
    const KArgs pa = (KArgs)__builtin_amdgcn_kernarg_segment_ptr();
    KArgs a = fresh_args(pa);
    static_assert(TH * TW == 256 && TW % 8 == 0, "a tile is 256 pixels, rows of 8-pixel vectors");
    // TH = 1: a flat tile, 256 consecutive output pixels in raster order
    // (ho0 holds its first pixel's index, wo0 is 0)
    constexpr bool kFlat = TH == 1;
    // output pixel (ho, wo) of the tile's pixel n
    auto out_pixel = [](int n, int ho0, int wo0, int Wo, int &ho, int &wo) {
        if constexpr (kFlat) {
            const int pp = ho0 + n;
            ho = pp / Wo;
            wo = pp - ho * Wo;
        } else {
            ho = ho0 + n / TW;
            wo = wo0 + n % TW;
        }
    };
    static_assert(LEAD >= 2 && LEAD + 1 <= 9, "copies lead by 2..8 steps");
    constexpr int kAStages = LEAD + 1;
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    const uint32_t lds0 = lds_addr(smem);
    uint32_t *woff_tab = reinterpret_cast<uint32_t *>(smem + kWoffOff);

    // zero areas of both window buffers (read by lanes whose sample is not
    // in the window); no copy ever writes them
    for (int i = int(threadIdx.x); i < 2 * kWinZero / 8; i += 256) {
        const int b = i / (kWinZero / 8), o = i - b * (kWinZero / 8);
        *reinterpret_cast<uint2 *>(smem + b * kWinBuf + kWinZeroOff + o * 8) = make_uint2(0u, 0u);
    }

    // This workgroup's share of the (tile, chunk) units: [u0, u1), split
    // evenly.  A tile shared with the previous workgroup (its first chunks
    // are there) comes first in the range, a tile shared with the next one
    // last.  Tiles are processed from the last to the first:
    // the partial sums of the last tile are published at once, and the first
    // tile is finished with the previous workgroup's partial sums at the
    // very end, so a workgroup only ever waits for a lower-numbered one
    // (dispatched earlier, and publishing first).
    //
    // Workgroups are dealt round-robin to the 8 XCDs (each with its own L2),
    // so with a grid that is a multiple of 8 the tiles are first split into
    // 8 contiguous runs of whole tiles, one per XCD (neighbouring tiles share
    // window rows, which then stay in one L2), and each run is split evenly
    // over that XCD's workgroups cta = x, x+8, x+16, ...: the previous
    // workgroup of a run is cta-8.
    const uint32_t cta = blockIdx.x;
    // [u0, u1) and the run's previous workgroup, from the arguments
    // (recomputed where needed rather than kept in scalar registers)
    struct Range {
        uint32_t u0, u1, prev;
    };
    auto range_of = [&](KArgs a) {
        const uint32_t ncta = gridDim.x, tiles = uint32_t(a->tiles);
        const uint32_t ngrp = (ncta % 8u == 0u && tiles >= ncta) ? 8u : 1u;
        const uint32_t grp = cta % ngrp, per = ncta / ngrp, idx = cta / ngrp;
        const uint32_t j = grp * per + idx;
        Range r;
        r.u0 = a->bounds[j];
        r.u1 = a->bounds[j + 1];
        r.prev = cta - ngrp;
        return r;
    };
    // a tile's chunk segment [c_lo, c_hi) in this workgroup and its position
    struct TileInfo {
        int c_lo, c_hi, m0, ho0, wo0, img, g;
    };
    auto tile_info = [&](KArgs a, const Range &r, int tile) {
        const uint32_t nch = uint32_t(a->nch);
        TileInfo ti;
        ti.c_lo = int(max(r.u0, uint32_t(tile) * nch) - uint32_t(tile) * nch);
        ti.c_hi = int(min(r.u1, uint32_t(tile + 1) * nch) - uint32_t(tile) * nch);
        uint32_t bid = uint32_t(tile);
        ti.m0 = int(bid % uint32_t(a->tiles_m)) * 256;
        bid /= uint32_t(a->tiles_m);
        ti.wo0 = int(bid % uint32_t(a->tiles_x)) * TW;
        bid /= uint32_t(a->tiles_x);
        ti.ho0 = int(bid % uint32_t(a->tiles_y)) * (kFlat ? 256 : TH);
        bid /= uint32_t(a->tiles_y);
        ti.img = int(bid % uint32_t(a->cnt));
        ti.g = int(bid / uint32_t(a->cnt));
        return ti;
    };
    int tile;
    {
        const Range r = range_of(a);
        if (r.u0 >= r.u1)
            return;
        tile = int((r.u1 - 1) / uint32_t(a->nch));   // the range's last tile comes first
    }
    // per-wave LDS word that holds the tile index across the main loop
    int *tile_park = reinterpret_cast<int *>(smem + kParkOff) +
                     __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);

    for (;;) {
        // Every lane- and argument-derived value is derived afresh per tile
        // (the thread index passes through an empty asm): a value hoisted out
        // of the tile loop would be live across the main loop, where no
        // register is free, and its spill reloads would wait for every store
        // in flight.
        int tid = int(threadIdx.x);
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int half = lane >> 5;                  // plane: channels 8*half..+8 of a chunk
        KArgs a = fresh_args(pa);
        const v4i rx = srd(a->xt, a->chunk_bytes);
        const uint32_t hw16 = uint32_t(a->H * a->W) * 16;   // bytes of one 8-channel block plane
        const uint32_t wrow = uint32_t(a->WC * 16);
        const uint32_t a_lane = uint32_t(half * (kAStage / 2) + (lane & 31) * 16);
        float zero;
        asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
        const int nch = a->nch;
        const TileInfo ti = tile_info(a, range_of(a), tile);
        const int c_lo = ti.c_lo, c_hi = ti.c_hi;
        const int m0 = ti.m0, ho0 = ti.ho0, wo0 = ti.wo0, img = ti.img;
        const int g = __builtin_amdgcn_readfirstlane(ti.g);
        // window origin (input coordinates)
        const int r0 = (kFlat ? ho0 / a->Wo : ho0) * a->sh - a->ph - a->margin;
        const int c0 = wo0 * a->sw - a->pw - a->margin;
        const int q = (g * a->Cg) / a->Cdg;              // the group's offset group
        const v4i ra =
            srd(static_cast<const char *>(a->A) + size_t(g) * a->a_bytes, a->a_bytes);
        if (lane == 0)
            *tile_park = tile;

        // ---- per-lane DMA source offsets of the window (kept in LDS; each
        // thread reads back only its own entries) and of the A rows
        const float inv_wc = 1.0f / float(a->WC);
#pragma unroll
        for (int t = 0; t < kWinInstr; ++t) {
            const int S = (t * 4 + wave) * 64 + lane;          // 16-byte slot of the buffer
            const int pl = S >= kWindowPixels ? 1 : 0;       // S < 2 * kWindowPixels
            const int px = S - pl * kWindowPixels;
            // px / WC through a float reciprocal: px < 1280 and WC <= 64, so
            // px/WC is at least 1/128 away from the next integer, far above
            // the float error (the plane of slot S is S / 1280 likewise)
            const int r = int((float(px) + 0.5f) * inv_wc), c = px - r * a->WC;
            const int gr = r0 + r, gc = c0 + c;
            const bool ok = px < a->WR * a->WC && (unsigned)gr < (unsigned)a->H &&
                            (unsigned)gc < (unsigned)a->W;
            woff_tab[t * 256 + tid] = ok ? uint32_t(img) * a->img_bytes + uint32_t(pl) * hw16 +
                                               uint32_t(gr * a->W + gc) * 16
                                         : kOOB;
        }
        uint32_t aoff[kAInstr];
#pragma unroll
        for (int t = 0; t < kAInstr; ++t) {
            const int S = (t * 4 + wave) * 64 + lane;
            const int pl = S >> 8, row = S & 255;
            aoff[t] = (m0 + row < a->Mg) ? uint32_t(pl * a->Mg + m0 + row) * 16 : kOOB;
        }
        // the group's first 8-channel block plane, bytes
        const uint32_t ch_base = uint32_t(g * a->Cg / 8) * hw16;
        auto issue_window = [&](int chunk, int buf) {
            const uint32_t soff =
                __builtin_amdgcn_readfirstlane(ch_base + uint32_t(chunk * 2) * hw16);
            uint32_t wo[kWinInstr];                 // all table reads first: one LDS wait
#pragma unroll
            for (int t = 0; t < kWinInstr; ++t)
                wo[t] = woff_tab[t * 256 + tid];
#pragma unroll
            for (int t = 0; t < kWinInstr; ++t)
                dma16(lds0 + buf * kWinBuf + (t * 4 + wave) * 1024 +
                          ((t * 4 + wave) * 64 >= kWindowPixels ? kPlaneGap : 0),
                      rx, wo[t], soff);
        };
        // K steps of the segment: step s (relative to its first chunk c_lo)
        // is tap s % 9 of chunk c_lo + s / 9; its A tile is step
        // 9*c_lo + s of the group's step-major weight.
        const int steps = (c_hi - c_lo) * kTaps;
        const int s_base = c_lo * kTaps;
        // (bytes per step of the step-major weight, held in a register: the
        // compiler would otherwise reload the argument inside the main loop)
        uint32_t a_step = uint32_t(a->Mg) * 32;
        asm volatile("" : "+s"(a_step));
        auto issue_a = [&](int step) {
            const uint32_t soff = __builtin_amdgcn_readfirstlane(uint32_t(s_base + step) * a_step);
#pragma unroll
            for (int t = 0; t < kAInstr; ++t)
                dma16(lds0 + kAOff + (step % kAStages) * kAStage + (t * 4 + wave) * 1024, ra,
                      aoff[t], soff);
        };

        // ---- prologue copies: window of the first chunk, A of steps 0 .. LEAD-1
        issue_window(c_lo, 0);
#pragma unroll
        for (int s = 0; s < LEAD; ++s)
            if (s < steps)
                issue_a(s);

        // ---- sampling geometry of the lane's two pixels, all taps
        uint32_t gaddr[2][kTaps];
        float gw[2][kTaps][4];
        uint32_t fbl = 0;                            // lane: (slab, tap) needs the fallback
        {
            const int P = a->P;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int n = (wave * 2 + s) * 32 + (lane & 31);
                int ho, wo;
                out_pixel(n, ho0, wo0, a->Wo, ho, wo);
                const bool pv = ho < a->Ho && wo < a->Wo;
                const int pix = pv ? ho * a->Wo + wo : 0;
                const size_t ob = (size_t(img) * a->offC + size_t(q) * 2 * kTaps) * P + pix;
                const size_t mb = (size_t(img) * a->mskC + size_t(q) * kTaps) * P + pix;
                const T *off = static_cast<const T *>(a->off);
                const T *msk = static_cast<const T *>(a->msk);
                float oh[kTaps], ow[kTaps], mm[kTaps];
#pragma unroll
                for (int k = 0; k < kTaps; ++k) {
                    oh[k] = to_f32(off[ob + size_t(2 * k) * P]);
                    ow[k] = to_f32(off[ob + size_t(2 * k + 1) * P]);
                    mm[k] = to_f32(msk[mb + size_t(k) * P]);
                }
#pragma unroll
                for (int k = 0; k < kTaps; ++k) {
                    const int i = k / 3, j = k % 3;
                    const int ah = ho * a->sh - a->ph + i * a->dh;
                    const int aw = wo * a->sw - a->pw + j * a->dw;
                    const float lim = 33554432.0f;
                    const bool fin = fabsf(oh[k]) <= lim && fabsf(ow[k]) <= lim;
                    const float fh = fin ? floorf(oh[k]) : 0.0f;
                    const float fw = fin ? floorf(ow[k]) : 0.0f;
                    const float ly = fin ? oh[k] - fh : 0.0f;
                    const float lx = fin ? ow[k] - fw : 0.0f;
                    const int h0 = ah + int(fh), w0 = aw + int(fw);
                    const bool any = pv && fin && h0 >= -1 && h0 < a->H && w0 >= -1 && w0 < a->W;
                    const int lr = h0 - r0, lc = w0 - c0;
                    const bool inw = (unsigned)lr <= unsigned(a->WR - 2) &&
                                     (unsigned)lc <= unsigned(a->WC - 2);
                    const bool use = any && inw;
                    const float hy = 1.0f - ly, hx = 1.0f - lx, m = mm[k];
                    gw[s][k][0] = use ? hy * hx * m : 0.0f;
                    gw[s][k][1] = use ? hy * lx * m : 0.0f;
                    gw[s][k][2] = use ? ly * hx * m : 0.0f;
                    gw[s][k][3] = use ? ly * lx * m : 0.0f;
                    gaddr[s][k] = use ? uint32_t(half * kPlane1 + (lr * a->WC + lc) * 16)
                                      : uint32_t(kWinZeroOff);
                    fbl |= uint32_t(any && !inw) << (s * kTaps + k);
                }
            }
        }
        // wave-level: which (slab, tap) has a lane that needs the fallback
        uint32_t fbw = 0;
#pragma unroll
        for (int b = 0; b < 2 * kTaps; ++b)
            fbw |= uint32_t(__builtin_amdgcn_ballot_w64(((fbl >> b) & 1u) != 0u) != 0) << b;
        fbw = __builtin_amdgcn_readfirstlane(fbw);

        // Fallback: the lane's 8 channels of sample (slab s, tap k) in chunk
        // `chunk`, from global memory (rare).
        auto fallback = [&](int s, int k, int chunk, uint4 &bv) {
            if ((fbl >> (s * kTaps + k)) & 1u) {
                KArgs a = fresh_args(pa);
                const T *offp = static_cast<const T *>(a->off);
                const T *mskp = static_cast<const T *>(a->msk);
                const int n = (wave * 2 + s) * 32 + (lane & 31);
                int ho, wo;
                out_pixel(n, ho0, wo0, a->Wo, ho, wo);
                const int pix = ho * a->Wo + wo;
                const size_t ob =
                    (size_t(img) * a->offC + size_t(q) * 2 * kTaps + 2 * k) * a->P + pix;
                const float oh = to_f32(offp[ob]), ow = to_f32(offp[ob + a->P]);
                const float m =
                    to_f32(mskp[(size_t(img) * a->mskC + size_t(q) * kTaps + k) * a->P + pix]);
                const int i = k / 3, j = k % 3;
                const Taps tp = make_taps(ho * a->sh - a->ph + i * a->dh,
                                          wo * a->sw - a->pw + j * a->dw, oh, ow, m, a->H, a->W);
                const uint32_t cb = ch_base + uint32_t(chunk * 2 + half) * hw16;
                uint4 cv[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const uint32_t o = tp.valid[t] ? uint32_t(img) * a->img_bytes +
                                                         uint32_t(tp.idx[t]) * 16 + cb
                                                   : kOOB;
                    const auto r = __builtin_amdgcn_raw_buffer_load_b128(
                        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a->xt), (short)0,
                                                          int(a->chunk_bytes), 0x00020000),
                        o, 0, 0);
                    __builtin_memcpy(&cv[t], &r, 16);
                }
                const float w4[4] = {tp.wt[0], tp.wt[1], tp.wt[2], tp.wt[3]};
                bv = blend<T>(cv[0], cv[1], cv[2], cv[3], w4, 0.0f);
            }
        };

        // Accumulators: zero, or -- for a tile whose first chunks the
        // previous workgroup of the run computed -- its partial sums, which
        // that workgroup published first thing (so the wait is short; the
        // spin is bounded, so that a broken invariant gives a wrong result,
        // never a stuck GPU).  The slot holds each lane's accumulator
        // registers as they are: wave w's 64 KB, 16-byte group j of every
        // lane at w*64K + j*1K + lane*16.
        float16v acc[8][2];
        {
            const bool resume = c_lo > 0;
            const uint32_t prev = range_of(a).prev;
            if (resume && tid == 0) {
                for (uint32_t it = 0; it < (1u << 26); ++it) {
                    if (__hip_atomic_load(a->flags + prev, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) == uint32_t(a->epoch))
                        break;
                    __builtin_amdgcn_s_sleep(2);
                }
            }
            __builtin_amdgcn_s_barrier();
            // (a tile started here reads through an empty buffer: zeros, with
            // no memory access and no branch)
            const __amdgpu_buffer_rsrc_t rs =
                srd_b(a->partial + (resume ? size_t(prev) * 65536 : 0),
                      resume ? uint32_t(65536 * 4) : 0u);
            const uint32_t lo = uint32_t(wave * 65536 + lane * 16);
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const auto v = __builtin_amdgcn_raw_buffer_load_b128(
                            rs, lo + uint32_t(((i * 2 + s) * 4 + q) * 1024), 0, kDevScope);
                        float4v f;
                        __builtin_memcpy(&f, &v, 16);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[i][s][4 * q + e] = f[e];
                    }
        }

        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

        // A fragment of block i of step `step` (plane = half, row = 32i + lane%32)
        auto read_a = [&](uint4 (&fa)[8], int step) {
            const uint32_t so = __builtin_amdgcn_readfirstlane(
                uint32_t(kAOff + (step % kAStages) * kAStage));
            const char *st = smem + (a_lane + so);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                fa[i] = *reinterpret_cast<const uint4 *>(st + i * 32 * 16);
        };
        // corners of (slab s, tap k) from window buffer `buf`
        auto read_corners = [&](uint4 (&cr)[4], int s, int k, int buf) {
            const uint32_t bo = __builtin_amdgcn_readfirstlane(uint32_t(buf ? kWinBuf : 0));
            const char *p = smem + (gaddr[s][k] + bo);
            const char *p2 = p + wrow;
            cr[0] = *reinterpret_cast<const uint4 *>(p);
            cr[1] = *reinterpret_cast<const uint4 *>(p + 16);
            cr[2] = *reinterpret_cast<const uint4 *>(p2);
            cr[3] = *reinterpret_cast<const uint4 *>(p2 + 16);
        };

        uint4 fa[8];
        uint4 cr[2][4];
        uint4 b[2];
        // step 0's operands
        read_a(fa, 0);
        read_corners(cr[0], 0, 0, 0);
        read_corners(cr[1], 1, 0, 0);
        b[0] = blend<T>(cr[0][0], cr[0][1], cr[0][2], cr[0][3], gw[0][0], zero);
        b[1] = blend<T>(cr[1][0], cr[1][1], cr[1][2], cr[1][3], gw[1][0], zero);
        if (fbw & (1u | (1u << kTaps))) {
            fallback(0, 0, c_lo, b[0]);
            fallback(1, 0, c_lo, b[1]);
        }
        read_corners(cr[0], 0, 1, 0);
        read_corners(cr[1], 1, 1, 0);

        // One step: relative step s = rc*9 + k of chunk c_lo + rc.  The tap
        // k is a compile-time index so the geometry stays in registers.
        auto step_body = [&](int rc, auto kc) {
            constexpr int k = decltype(kc)::value;
            const int s = rc * kTaps + k;
            const int chunk = c_lo + rc;
            const bool last_chunk = chunk + 1 >= c_hi;
            // One barrier every other step (even s): it makes A of steps s+1
            // and s+2 visible to every wave (the next step, which has none,
            // reads A(s+2)), so A(s+2) and every older copy must have
            // landed.  Issued after A(s+2) and allowed to be in flight: the A
            // copies of the LEAD-3 steps after it, and the window copy of the
            // next chunk while its first reads (in step k == 7, after the
            // barrier of step 6 or 7) are still ahead -- k in [1, LEAD-2]
            // (younger than A(s+2)) and k <= 5.  In the last chunk no window
            // is issued and the A copies stop at the last step.  (No LDS wait:
            // every LDS read of an A stage or window buffer that a copy issued
            // in this or the next step overwrites was consumed -- so waited
            // for -- before the previous step ended, and every wave has passed
            // this barrier or the previous one.)
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            if (((rc + k) & 1) == 0) {                    // s = 9 rc + k is even
                constexpr int kNoLgkm = 0x70 | 0xF00;     // expcnt and lgkmcnt: no wait
                if (last_chunk) {
                    constexpr int NA = kAInstr * ((LEAD - 3) < (6 - k)
                                                      ? (LEAD - 3)
                                                      : (6 - k > 0 ? 6 - k : 0));
                    __builtin_amdgcn_s_waitcnt((NA & 15) | ((NA >> 4) << 14) | kNoLgkm);
                } else if (k >= 1 && k <= LEAD - 2 && k <= 5) {
                    constexpr int N = kAInstr * (LEAD - 3) + kWinInstr;
                    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | kNoLgkm);
                } else {
                    constexpr int N = kAInstr * (LEAD - 3);
                    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | kNoLgkm);
                }
                __builtin_amdgcn_s_barrier();
            }
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("" ::: "memory");
            if (s + LEAD < steps)
                issue_a(s + LEAD);
            if (k == 0 && !last_chunk)
                issue_window(chunk + 1, (rc + 1) & 1);

            // MFMAs of step s, interleaved group by group (the wave issues in
            // order and is the only one on its SIMD) with the reads of step
            // s+1's A fragments (block i as soon as its two MFMAs have issued),
            // the blend of step s+1's B (one element pair per group) and the
            // corner reads of step s+2 (a slab's, once its blend is done).
            // Reads past the last step hit valid (stale) LDS and are never used.
            constexpr int k1 = (k + 1) % kTaps, k2 = (k + 2) % kTaps;
            const int rc1 = (k + 1 >= kTaps) ? rc + 1 : rc;
            const int rc2 = (k + 2 >= kTaps) ? rc + 1 : rc;
            const uint32_t so = __builtin_amdgcn_readfirstlane(
                uint32_t(kAOff + ((s + 1) % kAStages) * kAStage));
            const char *st = smem + (a_lane + so);
            uint32_t bn[2][4];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                acc[i][0] = Mma<T>::step(fa[i], b[0], acc[i][0]);
                acc[i][1] = Mma<T>::step(fa[i], b[1], acc[i][1]);
                fa[i] = *reinterpret_cast<const uint4 *>(st + i * 32 * 16);
                const int sl = i >> 2, pr = i & 3;
                bn[sl][pr] = blend_pair<T>(cr[sl], gw[sl][k1], zero, pr);
                if (pr == 3)
                    read_corners(cr[sl], sl, k2, rc2 & 1);
                __builtin_amdgcn_sched_barrier(0);
            }
            b[0] = make_uint4(bn[0][0], bn[0][1], bn[0][2], bn[0][3]);
            b[1] = make_uint4(bn[1][0], bn[1][1], bn[1][2], bn[1][3]);
            if (s + 1 < steps && (fbw & ((1u << k1) | (1u << (kTaps + k1))))) {
                fallback(0, k1, c_lo + rc1, b[0]);
                fallback(1, k1, c_lo + rc1, b[1]);
            }
        };

        for (int rc = 0; rc < c_hi - c_lo; ++rc) {
            step_body(rc, std::integral_constant<int, 0>{});
            step_body(rc, std::integral_constant<int, 1>{});
            step_body(rc, std::integral_constant<int, 2>{});
            step_body(rc, std::integral_constant<int, 3>{});
            step_body(rc, std::integral_constant<int, 4>{});
            step_body(rc, std::integral_constant<int, 5>{});
            step_body(rc, std::integral_constant<int, 6>{});
            step_body(rc, std::integral_constant<int, 7>{});
            step_body(rc, std::integral_constant<int, 8>{});
        }
        __builtin_amdgcn_s_waitcnt(0);

        // the main loop is over: the tile's state comes back from LDS and
        // the arguments rather than from registers held across it
        asm volatile("" ::: "memory");
        tile = __builtin_amdgcn_readfirstlane(*tile_park);
        tid = int(threadIdx.x);
        asm volatile("" : "+v"(tid));
        a = fresh_args(pa);
        const Range rg = range_of(a);
        const TileInfo te = tile_info(a, rg, tile);

        if (te.c_hi < a->nch) {
            // ---- the tile's first chunks: publish the accumulators as they
            // are (the layout the next workgroup of the run loads them in),
            // then the flag once every store is complete
            const __amdgpu_buffer_rsrc_t rs =
                srd_b(a->partial + size_t(cta) * 65536, uint32_t(65536 * 4));
            const uint32_t lo = uint32_t((tid >> 6) * 65536 + (tid & 63) * 16);
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float4v f = {acc[i][s][4 * q], acc[i][s][4 * q + 1],
                                           acc[i][s][4 * q + 2], acc[i][s][4 * q + 3]};
                        u32x4 u;
                        __builtin_memcpy(&u, &f, 16);
                        __builtin_amdgcn_raw_buffer_store_b128(
                            u, rs, lo + uint32_t(((i * 2 + s) * 4 + q) * 1024), 0, kDevScope);
                    }
            // device-scope stores are complete (acknowledged where every XCD
            // sees them) once the counter drains; only then the flag
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_s_barrier();
            if (tid == 0)
                __hip_atomic_store(a->flags + cta, uint32_t(a->epoch), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        } else {
            // ---- the tile's last chunks: per block of 32 output channels,
            // through an LDS slice [row][pixel] of fp32 sums, + bias, one
            // rounding, 16-byte stores of 8 pixels along a tile row.  No load
            // is issued between the stores (on this GPU a load's wait also
            // waits for every older store).
            float *bias_l = reinterpret_cast<float *>(smem + kWoffOff);   // dead copy table
            {
                const T *bias = static_cast<const T *>(a->bias);
                const int m = te.m0 + tid;
                bias_l[tid] =
                    (bias && m < a->Mg) ? to_f32(bias[size_t(te.g) * a->Mg + m]) : 0.0f;
            }
            __syncthreads();
            // output planes of the tile's image and group, as a buffer (a
            // lane with nothing to store gets an out-of-range offset, so
            // every block issues the same stores with no branches)
            const int Mg = a->Mg, P = a->P, Ho = a->Ho, Wo = a->Wo;
            const __amdgpu_buffer_rsrc_t ro =
                srd_b(static_cast<const T *>(a->out) +
                          (size_t(te.img) * a->Co + size_t(te.g) * a->Mg) * a->P,
                      uint32_t(size_t(Mg) * P * sizeof(T)));
            const bool vec = a->vec_out != 0;
            float *slice = reinterpret_cast<float *>(smem);
            // this thread's 4 x 8 sums of a block: row tid/32 + 8*jj, pixels
            // 8*(tid%32) ..+8
            const int row0 = tid >> 5, n = (tid & 31) * 8;
            int ho, wo;
            out_pixel(n, te.ho0, te.wo0, Wo, ho, wo);
            const uint32_t pix_off = uint32_t(ho * Wo + wo) * sizeof(T);   // bytes in a plane
            // (with vec, Wo and wo are multiples of 8: wo < Wo keeps all 8 inside)
            const bool pix_ok = ho < Ho && wo < Wo;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        slice[(8 * (r >> 2) + 4 * ((tid >> 5) & 1) + (r & 3)) * kEpRow +
                              (__builtin_amdgcn_readfirstlane(tid >> 6) * 2 + s) * 32 +
                              (tid & 31)] = acc[i][s][r];
                lds_barrier();                       // LDS only: stores stay in flight
                // per-block bases behind an empty asm, so that the per-(i, jj)
                // LDS addresses become base + immediate instead of 32 hoisted
                // (and spilled) registers (integer offsets pass through the
                // asm: a pointer would lose its LDS address space)
                uint32_t sl_o = uint32_t(row0 * kEpRow + n), bl_o = uint32_t(i * 32 + row0);
                asm volatile("" : "+v"(sl_o), "+v"(bl_o));
                const float *sl_b = slice + sl_o;
                const float *bl_b = bias_l + bl_o;
                // all of the block's LDS reads first (16-byte reads: a slice
                // row is 1040 bytes and n a multiple of 8), then one wait
                float4v sv[4][2];
                float bvv[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    sv[jj][0] = *reinterpret_cast<const float4v *>(sl_b + 8 * jj * kEpRow);
                    sv[jj][1] = *reinterpret_cast<const float4v *>(sl_b + 8 * jj * kEpRow + 4);
                    bvv[jj] = bl_b[8 * jj];
                }
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int row = row0 + 8 * jj;
                    const float sp[8] = {sv[jj][0][0], sv[jj][0][1], sv[jj][0][2], sv[jj][0][3],
                                         sv[jj][1][0], sv[jj][1][1], sv[jj][1][2], sv[jj][1][3]};
                    const int m = te.m0 + i * 32 + row;
                    const bool ok = m < Mg && pix_ok;
                    const float bv = bvv[jj];
                    const uint32_t base =
                        ok ? uint32_t(m) * uint32_t(P) * sizeof(T) + pix_off : kOOB;
                    if (vec) {
                        Vec16<T> o;
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            o.e[e] = from_f32<T>(sp[e] + bv);
                        u32x4 ov;
                        __builtin_memcpy(&ov, &o.raw, 16);
                        __builtin_amdgcn_raw_buffer_store_b128(ov, ro, base, 0, 0);
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const T h = from_f32<T>(sp[e] + bv);
                            uint16_t hb;
                            __builtin_memcpy(&hb, &h, 2);
                            __builtin_amdgcn_raw_buffer_store_b16(
                                hb, ro,
                                (kFlat ? ho * Wo + wo + e < Ho * Wo : wo + e < Wo)
                                    ? base + uint32_t(e) * sizeof(T)
                                    : kOOB,
                                0, 0);
                        }
                    }
                }
                lds_barrier();
            }
        }
        if (tile <= int(rg.u0 / uint32_t(a->nch)))
            break;                                   // that was the range's first tile
        --tile;
    }
}

// window_split for the last sizes asked (the same for every forward of one
// problem), behind a lock.
bool split_cached(int64_t tiles, int64_t nch, int64_t ncta, int64_t seg_x4, uint32_t *bounds)
{
    static std::mutex mu;
    static int64_t key[4] = {-1, -1, -1, -1};
    static uint32_t cached[kWindowSlots + 1];
    std::lock_guard<std::mutex> lock(mu);
    if (key[0] != tiles || key[1] != nch || key[2] != ncta || key[3] != seg_x4) {
        if (!window_split(tiles, nch, ncta, seg_x4, cached)) {
            key[0] = -1;
            return false;
        }
        key[0] = tiles; key[1] = nch; key[2] = ncta; key[3] = seg_x4;
    }
    std::copy(cached, cached + ncta + 1, bounds);
    return true;
}

// Compute units of the current device (cached per device).
int cu_count()
{
    static std::mutex mu;
    static std::map<int, int> known;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 1;
    std::lock_guard<std::mutex> lock(mu);
    auto it = known.find(dev);
    if (it == known.end()) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 1;
        it = known.emplace(dev, n).first;
    }
    return it->second;
}

template <typename T, int TH, int TW, int LEAD>
hipError_t window_cfg(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                      const void *xt, const void *offset, const void *mask, const void *bias,
                      void *out, const WindowScratch &ws, hipStream_t s)
{
    WinArgs a;
    a.Mg = int(p.Mg); a.Kp = int(plan.Kp); a.Co = int(p.Co); a.P = int(p.P);
    a.Ho = int(p.Ho); a.Wo = int(p.Wo);
    a.C = int(p.C); a.H = int(p.H); a.W = int(p.W); a.Cg = int(p.Cg);
    a.nch = int(p.Cg / kCC);
    a.sh = int(p.sh); a.sw = int(p.sw); a.ph = int(p.ph); a.pw = int(p.pw);
    a.dh = int(p.dh); a.dw = int(p.dw);
    a.margin = int(plan.win_margin);
    constexpr bool flat = TH == 1;
    a.WR = int(window_extent(flat ? window_flat_rows(p.Wo) : TH, p.sh, p.kh, p.dh,
                             plan.win_margin));
    a.WC = int(window_extent(flat ? p.Wo : TW, p.sw, p.kw, p.dw, plan.win_margin));
    a.tiles_y = int(flat ? (p.P + 255) / 256 : (p.Ho + TH - 1) / TH);
    a.tiles_x = int(flat ? 1 : (p.Wo + TW - 1) / TW);
    a.tiles_m = int((p.Mg + 255) / 256);
    a.cnt = int(cnt);
    a.offC = int(2 * p.DG * p.K);
    a.mskC = int(p.DG * p.K);
    a.Cdg = int(p.Cdg);
    a.has_bias = bias != nullptr;
    // 8-pixel vectors stay inside the image: rows of a multiple of 8 pixels,
    // or (flat tiles, where a vector may run on into the next row) planes of
    // a multiple of 8 pixels
    a.vec_out = ((flat ? p.P : p.Wo) % 8 == 0) && reinterpret_cast<uintptr_t>(out) % 16 == 0;
    a.img_bytes = uint32_t(size_t(p.H) * p.W * p.C * sizeof(T));
    a.chunk_bytes = uint32_t(size_t(cnt) * a.img_bytes);
    a.a_bytes = uint32_t(size_t(p.Mg) * p.Kg * sizeof(T));     // one group's weight
    if (a.WR * a.WC > kWindowPixels || a.WC * 16 + 32 > kWinZero)
        return hipErrorInvalidValue;
    const uint64_t tiles = uint64_t(p.G) * cnt * a.tiles_y * a.tiles_x * a.tiles_m;
    if (tiles == 0)
        return hipSuccess;
    if (tiles * uint64_t(a.nch) > 0xffffffffull)
        return hipErrorInvalidValue;
    a.tiles = int(tiles);
    a.epoch = ws.epoch;
    // One workgroup per CU (at most one tile's worth of units each fewer:
    // every tile then spans at most two workgroups), and no more than the
    // workspace has partial-sum slots for.
    uint64_t blocks = std::min<uint64_t>(
        {tiles, uint64_t(std::max(1, cu_count())), uint64_t(std::max(1, ws.slots))});
    if (plan.win_max_ctas > 0)
        blocks = std::min<uint64_t>(blocks, uint64_t(plan.win_max_ctas));
    if (ws.epoch <= 0 || (blocks < tiles && (!ws.partial || !ws.flags)))
        return hipErrorInvalidValue;
    if (!split_cached(int64_t(tiles), int64_t(a.nch), int64_t(blocks), plan.win_seg_cost_x4,
                      a.bounds))
        return hipErrorInvalidValue;
    auto kern = window_kernel<T, TH, TW, LEAD>;
    constexpr int lds = lds_total(LEAD);
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (attr != hipSuccess)
        return attr;
    a.A = wpack; a.xt = xt; a.off = offset; a.msk = mask; a.bias = bias; a.out = out;
    a.partial = ws.partial; a.flags = ws.flags;
    hipLaunchKernelGGL(kern, dim3(uint32_t(blocks)), dim3(256), lds, s, a);
    return hipGetLastError();
}

template <typename T, int TH, int TW>
hipError_t window_lead(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                       const void *xt, const void *offset, const void *mask, const void *bias,
                       void *out, const WindowScratch &ws, hipStream_t s)
{
    switch (plan.win_lead) {
    case 3:
        return window_cfg<T, TH, TW, 3>(p, plan, cnt, wpack, xt, offset, mask, bias, out, ws,
                                          s);
    case 5:
        return window_cfg<T, TH, TW, 5>(p, plan, cnt, wpack, xt, offset, mask, bias, out, ws,
                                          s);
    case 7:
        return window_cfg<T, TH, TW, 7>(p, plan, cnt, wpack, xt, offset, mask, bias, out, ws,
                                          s);
    }
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t window_t(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                    const void *xt, const void *offset, const void *mask, const void *bias,
                    void *out, const WindowScratch &ws, hipStream_t s)
{
    switch (plan.win_tile) {
    case WindowTile::H16_W16:
        return window_lead<T, 16, 16>(p, plan, cnt, wpack, xt, offset, mask, bias, out, ws, s);
    case WindowTile::H8_W32:
        return window_lead<T, 8, 32>(p, plan, cnt, wpack, xt, offset, mask, bias, out, ws, s);
    case WindowTile::H32_W8:
        return window_lead<T, 32, 8>(p, plan, cnt, wpack, xt, offset, mask, bias, out, ws, s);
    case WindowTile::FLAT:
        return window_lead<T, 1, 256>(p, plan, cnt, wpack, xt, offset, mask, bias, out, ws, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_window(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                         const void *xt, const void *offset, const void *mask, const void *bias,
                         void *out, const WindowScratch &ws, hipStream_t stream)
{
    switch (p.dtype) {
    case MDCN_F16:
        return window_t<half_t>(p, plan, cnt, wpack, xt, offset, mask, bias, out, ws, stream);
    case MDCN_BF16:
        return window_t<bf16_t>(p, plan, cnt, wpack, xt, offset, mask, bias, out, ws, stream);
    case MDCN_F32:
        break;
    }
    return hipErrorInvalidValue;
}

}  // namespace mdcn
