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
// The grid is persistent, one workgroup (8 waves, two per SIMD) per CU.  The
// (tile, chunk) units are cut into contiguous per-workgroup ranges on the
// host (balanced for chunks plus a per-tile cost, keeping tiles whole where
// the counts allow); a workgroup walks the tiles of its range from last to
// first.  A tile split between two workgroups is finished by the one holding
// its last chunks: the other publishes its accumulators (device-scope
// stores, then a flag) on the first tile it processes, and the finisher
// loads them into its accumulators on the last one (a bounded wait: a
// hand-over that never comes is recorded in a status word, never a hang).
//
// Every wave owns one slab of 32 pixels and all 256 output channels: it
// makes the B fragments of its own pixels in registers (lane l owns pixel
// l%32 and channels 8*(l/32)..+8 of the chunk, which is exactly the MFMA
// fragment layout), so B never goes through LDS, and reads the A fragments
// (packed weight rows) from LDS stages filled by DMA LEAD steps ahead.  The
// per-lane sampling geometry of all taps (window address of the top-left
// corner as packed 16-bit offsets, the bilinear factors with the mask folded
// in) is computed once per tile and kept in registers.  A step is a blend
// half (this step's B from the corners read one step before, then the next
// step's corner reads) and an MFMA half (8 MFMAs, then the next step's A
// fragment reads); the two waves of a SIMD run opposite halves, and the
// MFMA half runs at raised wave priority so that its issue is not starved
// by the partner's blend.
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
//
// The E4M3 variant (F8) keeps the window, geometry, work split and
// hand-overs, and changes the contraction: each sample is blended in fp32,
// saturated to +-448 and rounded to E4M3, and a 16-channel chunk's 9 taps run
// as three MFMA groups on the FP8 matrix cores -- taps 0-3 and 4-7 as one
// 64-deep v_mfma_f32_32x32x64_f8f6f4 each (the lane's 8 channels of four taps,
// 32 bytes, per 32x32 block), tap 8 as one 16-deep v_mfma_f32_32x32x16_fp8_fp8
// -- with the weight rows scaled by 2^e (e per output channel) and rounded to
// E4M3 by the set-up kernel, and 2^-e applied in the epilogue.  Its main loop
// is software-pipelined: every wave blends group q while the MFMAs of group
// q-1 run, with one barrier per group and one chunk's weight (36 KiB) in LDS.
// On groups of more than 256 output channels it runs wide tiles, 128 pixels
// x 512 output channels (72 KiB of weight, windows of kWindowPixelsWide
// positions): waves w and w+4 share 32 pixels and take one 256-channel half
// each, and each blends half of every group's samples and passes its E4M3
// bytes to the other through LDS, so that every sample is blended once for
// all 512 channels.
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
constexpr int kWaves = 8;                     // two waves per SIMD, 32 pixels each
constexpr int kThreads = 64 * kWaves;
constexpr int kTaps = 9;                      // 3x3 kernels
constexpr uint32_t kOOB = 0x80000000u;        // a byte offset past every buffer range

// LDS layout (bytes):
//   A stage s (s = 0..LEAD):    [plane 0: 256 rows x 16][plane 1: 256 rows x 16]
//                               (eight stages reserved whatever LEAD is, so that every
//                               A-fragment read is a base register plus an immediate
//                               offset below 64 KiB)
//   window buffer b (b = 0, 1): [plane 0: kWinPx x 16][gap][plane 1: kWinPx x 16][zeros]
//   window copy table:          [instruction t][thread]: source byte offset of the
//                               thread's 16 bytes of window copy instruction t
//   parked tile index:          one word per wave (256 bytes reserved)
// Plane p of an entry holds channels 8p..8p+7 of the chunk.  At the start of
// a tile, window buffer 1 (not yet in use) first receives the tile's offsets
// and masks: [channel of the offset group's 3K][256 tile pixels] elements.
constexpr int kWinPlane = kWindowPixels * 16;
// Plane 1 starts this many bytes past the end of plane 0, so that lanes
// reading the two planes at the same position use different LDS banks.
constexpr int kPlaneGap = 128;
constexpr int kPlane1 = kWinPlane + kPlaneGap;          // start of plane 1
constexpr int kWinZeroOff = kPlane1 + kWinPlane;        // start of the zero area
constexpr int kWinZero = kWindowZeroBytes;
constexpr int kWinBuf = kWinZeroOff + kWinZero;
constexpr int kAStage = 256 * 2 * 16;
constexpr int kAOff = 0;
constexpr int kWin0 = 8 * kAStage;                      // window buffer 0
constexpr int kWinInstr = 2 * kWindowPixels / 64 / kWaves;   // window DMA instructions per wave
constexpr int kWoffOff = kWin0 + 2 * kWinBuf;
constexpr int kParkOff = kWoffOff + kWinInstr * kThreads * 4;  // a tile index per wave, a flag
constexpr int kLdsTotal = kParkOff + 256;
constexpr int kOmOff = kWin0 + kWinBuf;                 // offsets and masks of a tile
constexpr int kOmPlanes = 3 * kTaps;                    // 2K offset + K mask channels
static_assert(kOmPlanes * 256 * 2 <= kWinPlane, "a tile's offsets and masks fit plane 0");
// A stages: the copy of step s+LEAD is issued in step s, into one of LEAD+1
// stages.
constexpr int kAInstr = kAStage / 1024 / kWaves;        // A DMA instructions per wave
// Cache-policy operand of a buffer access with device scope (the SC1 bit on
// gfx950): a store is written through to where every XCD sees it and a load
// is served from there.  The partial sums passed between workgroups use it,
// so no whole-L2 writeback or invalidate is needed on either side.
constexpr int kDevScope = 16;
static_assert(kLdsTotal <= int(kLdsBytes), "LDS budget");
static_assert(8 * kAStage <= kWin0, "A stages below the window buffers");
static_assert(kWindowPixels % 64 == 0 && (2 * kWindowPixels / 64) % kWaves == 0,
              "window DMA covers whole wave instructions, none straddling the two planes");
static_assert(kAStage % (1024 * kWaves) == 0, "A DMA covers whole wave instructions");

// The E4M3 variant (F8) keeps one chunk's weight in LDS, in three slots that
// the chunk's three MFMA groups read in turn: taps 0-3 and taps 4-7, each
// [half h][16-byte part][rows][16 bytes] (part 0: taps 0 and 1 of the row's
// 32 bytes, part 1: taps 2 and 3), and tap 8, [half h][rows][8 bytes], for
// the tile's 256 (wide tiles: 512) output channels.  Every part is the 8
// channels 8h..8h+7 of one tap as E4M3 bytes.  The window buffers, copy
// table and parked words follow the slots.
//
// The wide tiles (128 pixels x 512 output channels, E4M3 only) need 72 KiB of
// weight slots, so their window buffers hold kWindowPixelsWide positions, the
// window copy offsets stay in registers instead of the table, and in its
// place is the exchange area through which the two waves of a SIMD pass each
// other their halves of a group's E4M3 operand: [parity 2][wave pair 4]
// [half 2][64 lanes][16 bytes].
template <bool F8, bool WIDE> struct WinLds {
    static constexpr int px = WIDE ? kWindowPixelsWide : kWindowPixels;  // window positions
    static constexpr int plane = px * 16;                      // bytes of one window plane
    static constexpr int plane1 = plane + kPlaneGap;           // start of plane 1
    static constexpr int zero = plane1 + plane;                // start of the zero area
    static constexpr int buf = zero + kWinZero;                // one window buffer
    static constexpr int instr = 2 * px / 64 / kWaves;         // window DMA instructions per wave
    static constexpr int rows = WIDE ? 512 : 256;              // output channels of a tile
    static constexpr int quad = 2 * rows * 32;                 // E4M3 slot of four taps
    static constexpr int single = 2 * rows * 8;                // E4M3 slot of the ninth tap
    static constexpr int a8 = quad / 1024 / kWaves;            // E4M3 DMA instructions per wave and slot
    static constexpr int win0 = F8 ? 2 * quad + single : kWin0;   // window buffer 0
    static constexpr int woff = win0 + 2 * buf;                // window copy table (not WIDE)
    static constexpr int xch = woff + (WIDE ? 0 : instr * kThreads * 4);   // exchange (WIDE)
    static constexpr int park = xch + (WIDE ? 2 * 8192 : 0);   // tile index per wave, flag
    static constexpr int total = park + 256;
    static constexpr int om = win0 + buf;                      // offsets and masks of a tile
    static_assert(!WIDE || F8, "wide tiles are E4M3 only");
    static_assert(total <= int(kLdsBytes), "LDS budget");
    static_assert(win0 % 1024 == 0, "window buffers start on a 1 KiB boundary");
    static_assert(buf <= 65536, "window offsets fit 16 bits");
    static_assert(px % 64 == 0 && (2 * px / 64) % kWaves == 0,
                  "window DMA covers whole wave instructions, none straddling the two planes");
    static_assert(quad % (1024 * kWaves) == 0 && single / 256 / kWaves == a8,
                  "E4M3 weight DMA covers whole wave instructions");
    static_assert(kOmPlanes * (WIDE ? 128 : 256) * 2 <= plane, "a tile's offsets and masks fit plane 0");
};
static_assert(WinLds<false, false>::total == kLdsTotal && WinLds<false, false>::om == kOmOff &&
                  WinLds<false, false>::buf == kWinBuf && WinLds<false, false>::instr == kWinInstr,
              "layout");

struct WinArgs {
    const void *A, *xt, *off, *msk, *bias;   // step-major weight, x blocks, offset, mask, bias|null
    void *out;
    float *partial;                          // partial-sum slots
    uint32_t *flags;                         // one flag per slot
    uint32_t *status;                        // set to kWindowGaveUp by a hand-over wait that gave up
    int Mg, Kp, Co, P, Ho, Wo;
    int C, H, W, Cg, nch;          // nch: chunks of 16 channels per group
    int sh, sw, ph, pw, dh, dw;
    int margin, WR, WC;            // window rows / columns
    int tiles_x, tiles_y, tiles_m, cnt, tiles;
    int epoch;                     // value that marks partial sums published by this launch
    int offC, mskC, Cdg;           // offset / mask channels per image; C / deformable_group
    int has_bias, vec_out;
    int om_lds;                    // offsets and masks reach LDS by DMA (4-byte aligned pairs)
    uint32_t spin_limit;           // polls of a hand-over flag before giving up
    uint32_t img_bytes, chunk_bytes, a_bytes;
    uint32_t off_bytes, msk_bytes; // offsets / masks of the chunk's images
    // unit range of each workgroup slot (slot j = run * per + index in run)
    uint32_t bounds[kWindowSlots + 1];
    const float *wscale;           // F8: 2^-e of each output channel's weight row
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

// 4 bytes per lane from buffer offset voff + soff into LDS at lds + 4*lane
// (the same contract as dma16).
__device__ __forceinline__ void dma4(uint32_t lds, v4i rsrc, uint32_t voff, uint32_t soff)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
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

// The same sample as `blend`, as 8 E4M3 bytes (channel 0 in the lowest
// byte): the fp32 values saturated to +-448 -- only where some lane of the
// wave holds a value beyond that (or an infinity; a NaN stays NaN) -- and
// rounded to nearest even by the converter.
template <typename T>
__device__ __forceinline__ void blend_f32(const uint4 (&c)[4], const float (&w)[4], float zero,
                                          float (&acc)[8])
{
    Vec16<T> v0, v1, v2, v3;
    v0.raw = c[0]; v1.raw = c[1]; v2.raw = c[2]; v3.raw = c[3];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        acc[e] = fmaf(to_f32(v0.e[e]), w[0], zero);
        acc[e] = fmaf(to_f32(v1.e[e]), w[1], acc[e]);
        acc[e] = fmaf(to_f32(v2.e[e]), w[2], acc[e]);
        acc[e] = fmaf(to_f32(v3.e[e]), w[3], acc[e]);
    }
}

// Four channels (elements 0..3 of each corner chunk) of a sample in fp32.
template <typename T>
__device__ __forceinline__ void blend_f32_4(const uint4 (&c)[4], const float (&w)[4], float zero,
                                            float (&acc)[4])
{
    Vec16<T> v0, v1, v2, v3;
    v0.raw = c[0]; v1.raw = c[1]; v2.raw = c[2]; v3.raw = c[3];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        acc[e] = fmaf(to_f32(v0.e[e]), w[0], zero);
        acc[e] = fmaf(to_f32(v1.e[e]), w[1], acc[e]);
        acc[e] = fmaf(to_f32(v2.e[e]), w[2], acc[e]);
        acc[e] = fmaf(to_f32(v3.e[e]), w[3], acc[e]);
    }
}

// Four fp32 values as E4M3 bytes, saturated as in e4m3_of.
__device__ __forceinline__ uint32_t e4m3_of4(float (&acc)[4])
{
    const float m = fmaxf(fmaxf(fabsf(acc[0]), fabsf(acc[1])), fmaxf(fabsf(acc[2]), fabsf(acc[3])));
    if (__builtin_amdgcn_ballot_w64(m > 448.0f) != 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc[e] = sat_e4m3(acc[e]);
    }
    return pack4_e4m3_unsat(acc[0], acc[1], acc[2], acc[3]);
}

__device__ __forceinline__ uint2 e4m3_of(float (&acc)[8])
{
    const float m = fmaxf(fmaxf(fmaxf(fabsf(acc[0]), fabsf(acc[1])),
                                fmaxf(fabsf(acc[2]), fabsf(acc[3]))),
                          fmaxf(fmaxf(fabsf(acc[4]), fabsf(acc[5])),
                                fmaxf(fabsf(acc[6]), fabsf(acc[7]))));
    if (__builtin_amdgcn_ballot_w64(m > 448.0f) != 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[e] = sat_e4m3(acc[e]);
    }
    return make_uint2(pack4_e4m3_unsat(acc[0], acc[1], acc[2], acc[3]),
                      pack4_e4m3_unsat(acc[4], acc[5], acc[6], acc[7]));
}

template <typename T>
__device__ __forceinline__ uint2 blend_e4m3(const uint4 (&c)[4], const float (&w)[4], float zero)
{
    float acc[8];
    blend_f32<T>(c, w, zero, acc);
    return e4m3_of(acc);
}

template <typename T, int TH, int TW, int LEAD, bool F8, bool WIDE>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(2, 2)))
void window_kernel(WinArgs args)
{
    (void)args;
    const KArgs pa = (KArgs)__builtin_amdgcn_kernarg_segment_ptr();
    KArgs a = fresh_args(pa);
    // pixels and output channels of a tile
    constexpr int kTilePx = WIDE ? 128 : 256;
    constexpr int kTileM = WIDE ? 512 : 256;
    static_assert(TH * TW == kTilePx && TW % 8 == 0, "a tile's pixels, rows of 8-pixel vectors");
    // TH = 1: a flat tile, kTilePx consecutive output pixels in raster order
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
    // Eight A stages, a barrier every third step (k = 0, 3, 6 of a chunk):
    // a copy issued in step y overwrites A(y + LEAD - 8), which every wave
    // consumed before the last barrier (y - 2 or later) when LEAD <= 5, and
    // A(t), read in step t - 1, was issued in step t - LEAD, at least two
    // steps before the last barrier, which waited for it when LEAD >= 5.
    static_assert(LEAD == 5, "a barrier every third step needs a copy lead of 5 steps");
    constexpr int kAStages = 8;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    using L = WinLds<F8, WIDE>;
    // Sampling taps a wave blends: all 9, or on wide tiles 5 -- taps
    // 2s, 2s+1, 4+2s, 5+2s and (channels 4s..4s+3 of each 8) tap 8, for s =
    // wave / 4 -- as local taps 0..kLT-1.
    constexpr int kLT = WIDE ? 5 : kTaps;

    const uint32_t lds0 = lds_addr(smem);
    uint32_t *woff_tab = reinterpret_cast<uint32_t *>(smem + L::woff);

    // zero areas of both window buffers (read by lanes whose sample is not
    // in the window); no copy ever writes them
    for (int i = int(threadIdx.x); i < 2 * kWinZero / 8; i += kThreads) {
        const int b = i / (kWinZero / 8), o = i - b * (kWinZero / 8);
        *reinterpret_cast<uint2 *>(smem + L::win0 + b * L::buf + L::zero + o * 8) =
            make_uint2(0u, 0u);
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
        ti.m0 = int(bid % uint32_t(a->tiles_m)) * kTileM;
        bid /= uint32_t(a->tiles_m);
        ti.wo0 = int(bid % uint32_t(a->tiles_x)) * TW;
        bid /= uint32_t(a->tiles_x);
        ti.ho0 = int(bid % uint32_t(a->tiles_y)) * (kFlat ? kTilePx : TH);
        bid /= uint32_t(a->tiles_y);
        ti.img = int(bid % uint32_t(a->cnt));
        ti.g = int(bid / uint32_t(a->cnt));
        return ti;
    };
    int tile;
    // A partial-sum slot this workgroup published whose flag is still to be
    // set (see the publish below): wave-uniform, set by the tile that
    // published and cleared once the flag is out.
    bool flag_pending = false;
    {
        const Range r = range_of(a);
        if (r.u0 >= r.u1)
            return;
        tile = int((r.u1 - 1) / uint32_t(a->nch));   // the range's last tile comes first
    }
    // per-wave LDS word that holds the tile index across the main loop, and
    // the word that says whether this tile's hand-over wait gave up
    int *tile_park = reinterpret_cast<int *>(smem + L::park) +
                     __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
    int *gave_up_l = reinterpret_cast<int *>(smem + L::park) + 32;

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
        // wide tiles: waves w and w + 4 (one SIMD) share 32 pixels, and take
        // output channels 256*sub..+256 of the tile
        const int pair = WIDE ? (wave & 3) : wave;
        const int sub = WIDE ? (wave >> 2) : 0;
        // the wave's 32 pixels (tile pixels 32*pair ..+32; lane: 32*pair + lane%32)
        const int px_n = pair * 32 + (lane & 31);
        // global tap of local tap lt
        auto tap_of = [&](int lt) {
            if constexpr (WIDE)
                return lt < 4 ? (lt >> 1) * 4 + 2 * sub + (lt & 1) : 8;
            else
                return lt;
        };
        KArgs a = fresh_args(pa);
        const v4i rx = srd(a->xt, a->chunk_bytes);
        const uint32_t hw16 = uint32_t(a->H * a->W) * 16;   // bytes of one 8-channel block plane
        const uint32_t wrow = uint32_t(a->WC * 16);
        const uint32_t a_lane = uint32_t(half * (kAStage / 2) + (lane & 31) * 16);
        float zero;
        asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
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
        // every wave is done with the previous tile's LDS (window buffers
        // and copy table): the first of them is about to be overwritten
        lds_barrier();
        if (lane == 0)
            *tile_park = tile;

        // ---- the tile's offsets and masks, by DMA into window buffer 1
        // (idle until the main loop's first step), issued before the copies
        // so that they do not queue behind them: instruction j carries
        // channel j/kOmPer of the offset group's 2K offset and K mask channels
        // for tile pixels 128*(j%kOmPer) + 2*lane, +1 (an aligned 4-byte pair).
        constexpr int kOmPer = kTilePx / 128;
        const bool om_lds = a->om_lds != 0;
        if (om_lds) {
            const v4i ro = srd(a->off, a->off_bytes);
            const v4i rm = srd(a->msk, a->msk_bytes);
            // the fields the loop needs, read once: the DMA's memory clobber
            // would make the compiler reload each of them (a dependent
            // scalar load and wait) per instruction
            const int Wo = a->Wo, Ho = a->Ho;
            const uint32_t P = uint32_t(a->P);
            const uint32_t ob = uint32_t(img * a->offC + q * 2 * kTaps);
            const uint32_t mb = uint32_t(img * a->mskC + q * kTaps);
            for (int j = wave; j < kOmPlanes * kOmPer; j += kWaves) {
                const int plane = int(unsigned(j) / kOmPer);
                const int part = int(unsigned(j) % kOmPer);
                const int n = part * 128 + 2 * lane;
                int ho, wo;
                out_pixel(n, ho0, wo0, Wo, ho, wo);
                const bool ok = ho < Ho && wo < Wo;
                const bool is_off = plane < 2 * kTaps;
                const uint32_t chan = is_off ? ob + uint32_t(plane)
                                             : mb + uint32_t(plane - 2 * kTaps);
                const uint32_t voff = ok ? (chan * P + uint32_t(ho * Wo + wo)) * 2u : kOOB;
                dma4(lds0 + uint32_t(L::om + plane * (2 * kTilePx) + part * 256),
                     is_off ? ro : rm, voff, 0u);
            }
        }

        // ---- per-lane DMA source offsets of the window (kept in LDS, each
        // thread reading back only its own entries; wide tiles: in registers)
        // and of the A rows
        uint32_t wsrc[WIDE ? L::instr : 1];
        {
            // (the fields read once, before the table stores)
            const int WC = a->WC, WRC = a->WR * a->WC, H = a->H, W = a->W;
            const uint32_t img_base = uint32_t(img) * a->img_bytes;
            const float inv_wc = 1.0f / float(WC);
#pragma unroll
            for (int t = 0; t < L::instr; ++t) {
                const int S = (t * kWaves + wave) * 64 + lane;   // 16-byte slot of the buffer
                const int pl = S >= L::px ? 1 : 0;               // S < 2 * L::px
                const int px = S - pl * L::px;
                // px / WC through a float reciprocal: px < 1280 and WC <= 64, so
                // px/WC is at least 1/128 away from the next integer, far above
                // the float error
                const int r = int((float(px) + 0.5f) * inv_wc), c = px - r * WC;
                const int gr = r0 + r, gc = c0 + c;
                const bool ok = px < WRC && (unsigned)gr < (unsigned)H && (unsigned)gc < (unsigned)W;
                const uint32_t v =
                    ok ? img_base + uint32_t(pl) * hw16 + uint32_t(gr * W + gc) * 16 : kOOB;
                if constexpr (WIDE)
                    wsrc[t] = v;
                else
                    woff_tab[t * kThreads + tid] = v;
            }
        }
        // (F8, R = L::rows: entries 0..a8-1 for the four-tap slots, 16-byte
        // slot S = half S/2R, part S/R % 2, row S % R; entries a8..2a8-1 for
        // the tap-8 slot, 4-byte slot S = half S/2R, row S/2 % R, word S % 2)
        uint32_t aoff[F8 ? 2 * L::a8 : kAInstr];
        if constexpr (F8) {
#pragma unroll
            for (int t = 0; t < L::a8; ++t) {
                const int S = (t * kWaves + wave) * 64 + lane;
                const int pq = S / L::rows, row = S % L::rows;
                aoff[t] = (m0 + row < a->Mg) ? uint32_t(pq * a->Mg + m0 + row) * 16 : kOOB;
                const int h = S / (2 * L::rows), r2 = (S >> 1) % L::rows;
                aoff[L::a8 + t] = (m0 + r2 < a->Mg)
                                      ? uint32_t(h * a->Mg + m0 + r2) * 8 + uint32_t(S & 1) * 4
                                      : kOOB;
            }
        } else {
#pragma unroll
            for (int t = 0; t < kAInstr; ++t) {
                const int S = (t * kWaves + wave) * 64 + lane;
                const int pl = S >> 8, row = S & 255;
                aoff[t] = (m0 + row < a->Mg) ? uint32_t(pl * a->Mg + m0 + row) * 16 : kOOB;
            }
        }
        // the group's first 8-channel block plane, bytes
        const uint32_t ch_base = uint32_t(g * a->Cg / 8) * hw16;
        auto issue_window = [&](int chunk, int buf) {
            const uint32_t soff =
                __builtin_amdgcn_readfirstlane(ch_base + uint32_t(chunk * 2) * hw16);
            uint32_t wo[L::instr];                  // all table reads first: one LDS wait
#pragma unroll
            for (int t = 0; t < L::instr; ++t) {
                if constexpr (WIDE)
                    wo[t] = wsrc[t];
                else
                    wo[t] = woff_tab[t * kThreads + tid];
            }
#pragma unroll
            for (int t = 0; t < L::instr; ++t)
                dma16(lds0 + L::win0 + buf * L::buf + (t * kWaves + wave) * 1024 +
                          ((t * kWaves + wave) * 64 >= L::px ? kPlaneGap : 0),
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
                dma16(lds0 + kAOff + (step % kAStages) * kAStage + (t * kWaves + wave) * 1024, ra,
                      aoff[t], soff);
        };
        // F8: the weight of MFMA group j (0: taps 0-3, 1: taps 4-7, 2: tap 8)
        // of relative chunk rc into slot j; a chunk's block is 144*Mg bytes,
        // its regions 64*Mg bytes apart
        uint32_t a_chunk = 0, a_region = 0;
        if constexpr (F8) {
            a_chunk = uint32_t(a->Mg) * 144;
            a_region = uint32_t(a->Mg) * 64;
            asm volatile("" : "+s"(a_chunk), "+s"(a_region));
        }
        auto issue_a8 = [&](int rc, auto jc) {
            constexpr int j = decltype(jc)::value;
            const uint32_t soff = __builtin_amdgcn_readfirstlane(uint32_t(c_lo + rc) * a_chunk +
                                                                 uint32_t(j) * a_region);
            if constexpr (j < 2) {
#pragma unroll
                for (int t = 0; t < L::a8; ++t)
                    dma16(lds0 + j * L::quad + (t * kWaves + wave) * 1024, ra, aoff[t], soff);
            } else {
#pragma unroll
                for (int t = 0; t < L::a8; ++t)
                    dma4(lds0 + 2 * L::quad + (t * kWaves + wave) * 256, ra, aoff[L::a8 + t],
                         soff);
            }
        };

        // ---- prologue copies: window of the first chunk, A of steps 0 .. LEAD-1
        // (F8: of the first chunk's first group)
        issue_window(c_lo, 0);
        if constexpr (F8) {
            issue_a8(0, std::integral_constant<int, 0>{});
        } else {
#pragma unroll
            for (int s = 0; s < LEAD; ++s)
                if (s < steps)
                    issue_a(s);
        }

        // ---- sampling geometry of the lane's pixel, all (local) taps: the
        // byte offset of the top-left corner in a window buffer (16 bits, two
        // taps per register: local tap t in half t%2 of gpk[t/2]) and three
        // factors from which the four corner weights are formed per step (see
        // weights_of)
        uint32_t gpk[(kLT + 1) / 2] = {};
        float gw[kLT][3];
        uint32_t fbl = 0;                            // lane: local tap t needs the fallback
        {
            const int P = a->P;
            float oh[kLT], ow[kLT], mm[kLT];
            if (om_lds) {
                // this wave's offset and mask copies (issued before the window
                // and A copies, so older than the last L::instr + LEAD*kAInstr
                // of its copies) have landed, then every wave's
                constexpr int N = L::instr + (F8 ? L::a8 : LEAD * kAInstr);
                constexpr int kNoLgkm = 0x70 | 0xF00;
                static_assert(N < 64, "vmcnt range");
                __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | kNoLgkm);
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
                const char *om = smem + L::om + px_n * 2;
                constexpr int kOmPlane = 2 * kTilePx;
#pragma unroll
                for (int lt = 0; lt < kLT; ++lt) {
                    const int k = tap_of(lt);
                    oh[lt] = to_f32(*reinterpret_cast<const T *>(om + (2 * k) * kOmPlane));
                    ow[lt] = to_f32(*reinterpret_cast<const T *>(om + (2 * k + 1) * kOmPlane));
                    mm[lt] = to_f32(*reinterpret_cast<const T *>(om + (2 * kTaps + k) * kOmPlane));
                }
            } else {
                int ho, wo;
                out_pixel(px_n, ho0, wo0, a->Wo, ho, wo);
                const bool pv = ho < a->Ho && wo < a->Wo;
                const int pix = pv ? ho * a->Wo + wo : 0;
                const size_t ob = (size_t(img) * a->offC + size_t(q) * 2 * kTaps) * P + pix;
                const size_t mb = (size_t(img) * a->mskC + size_t(q) * kTaps) * P + pix;
                const T *off = static_cast<const T *>(a->off);
                const T *msk = static_cast<const T *>(a->msk);
#pragma unroll
                for (int lt = 0; lt < kLT; ++lt) {
                    const int k = tap_of(lt);
                    oh[lt] = to_f32(off[ob + size_t(2 * k) * P]);
                    ow[lt] = to_f32(off[ob + size_t(2 * k + 1) * P]);
                    mm[lt] = to_f32(msk[mb + size_t(k) * P]);
                }
            }
            if (flag_pending) {
                // the previous tile's published partial sums: everything
                // but this prologue's window and weight copies (the youngest
                // vector memory operations) is complete after this wait,
                // those stores included; then the flag
                constexpr int N = L::instr + (F8 ? L::a8 : LEAD * kAInstr);
                constexpr int kNoLgkmF = 0x70 | 0xF00;
                asm volatile("" ::: "memory");
                __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | kNoLgkmF);
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
                if (tid == 0) {
                    KArgs af = fresh_args(pa);
                    __hip_atomic_store(af->flags + cta, uint32_t(af->epoch), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
                flag_pending = false;
            }
            int ho, wo;
            out_pixel(px_n, ho0, wo0, a->Wo, ho, wo);
            const bool pv = ho < a->Ho && wo < a->Wo;
#pragma unroll
            for (int lt = 0; lt < kLT; ++lt) {
                const int k = tap_of(lt);
                const int i = k / 3, j = k % 3;
                const int ah = ho * a->sh - a->ph + i * a->dh;
                const int aw = wo * a->sw - a->pw + j * a->dw;
                const float lim = 33554432.0f;
                const bool fin = fabsf(oh[lt]) <= lim && fabsf(ow[lt]) <= lim;
                const float fh = fin ? floorf(oh[lt]) : 0.0f;
                const float fw = fin ? floorf(ow[lt]) : 0.0f;
                const float ly = fin ? oh[lt] - fh : 0.0f;
                const float lx = fin ? ow[lt] - fw : 0.0f;
                const int h0 = ah + int(fh), w0 = aw + int(fw);
                const bool any = pv && fin && h0 >= -1 && h0 < a->H && w0 >= -1 && w0 < a->W;
                const int lr = h0 - r0, lc = w0 - c0;
                const bool inw = (unsigned)lr <= unsigned(a->WR - 2) &&
                                 (unsigned)lc <= unsigned(a->WC - 2);
                const bool use = any && inw;
                const float m = use ? mm[lt] : 0.0f;
                gw[lt][0] = (1.0f - lx) * m;
                gw[lt][1] = lx * m;
                gw[lt][2] = ly;
                // (wide tiles, tap 8: the wave's 4 channels are bytes 8s..8s+7
                // of the 16-byte entry)
                const uint32_t sub8 = (WIDE && lt == 4) ? uint32_t(sub * 8) : 0u;
                const uint32_t wa =
                    use ? uint32_t(half * L::plane1 + (lr * a->WC + lc) * 16) + sub8
                        : uint32_t(L::zero);
                gpk[lt / 2] |= wa << (16 * (lt % 2));
                fbl |= uint32_t(any && !inw) << lt;
            }
        }
        // wave-level: which local tap has a lane that needs the fallback
        uint32_t fbw = 0;
#pragma unroll
        for (int b = 0; b < kLT; ++b)
            fbw |= uint32_t(__builtin_amdgcn_ballot_w64(((fbl >> b) & 1u) != 0u) != 0) << b;
        fbw = __builtin_amdgcn_readfirstlane(fbw);

        // Fallback: the lane's 8 channels of the sample of local tap lt in
        // chunk `chunk`, from global memory (rare).
        auto fallback = [&](int lt, int chunk, auto &bv) {
            if ((fbl >> lt) & 1u) {
                const int k = tap_of(lt);
                KArgs a = fresh_args(pa);
                const T *offp = static_cast<const T *>(a->off);
                const T *mskp = static_cast<const T *>(a->msk);
                int ho, wo;
                out_pixel(px_n, ho0, wo0, a->Wo, ho, wo);
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
                if constexpr (F8)
                    bv = blend_e4m3<T>(cv, w4, 0.0f);
                else
                    bv = blend<T>(cv[0], cv[1], cv[2], cv[3], w4, 0.0f);
            }
        };

        // Accumulators: zero, or -- for a tile whose first chunks the
        // previous workgroup of the run computed -- its partial sums, which
        // that workgroup published first thing (so the wait is short).  The
        // wait is bounded so that a broken invariant can never hang the GPU:
        // a workgroup that gives up sets the status word and writes NaN for
        // its tile (a NaN bias in the epilogue), so the failure shows in the
        // output and is reported to the host (never a silently wrong tensor).
        // The slot holds each lane's accumulator registers as they are: wave
        // w's 32 KB, 16-byte group j of every lane at w*32K + j*1K + lane*16.
        //
        // Ordering: the publisher's partial-sum stores and both flag accesses
        // are device-scope (SC1) accesses, which bypass the non-coherent
        // caches; every wave of the publisher waits for its stores to be
        // acknowledged (a vmcnt wait that leaves only younger operations in
        // flight, then a barrier) before the flag store, and the data loads
        // here are issued after the flag was seen (the barrier follows the
        // poll).  Empty asm statements with a memory clobber keep the
        // compiler from moving any of these accesses across the flag.
        float16v acc[8];
        {
            const bool resume = c_lo > 0;
            const uint32_t prev = range_of(a).prev;
            if (tid == 0 && !resume)
                *gave_up_l = 0;
            if (resume && tid == 0) {
                const uint32_t limit = a->spin_limit;
                uint32_t it = 0;
                for (; it < limit; ++it) {
                    if (__hip_atomic_load(a->flags + prev, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) == uint32_t(a->epoch))
                        break;
                    __builtin_amdgcn_s_sleep(2);
                }
                const bool gave = it >= limit;
                *gave_up_l = gave ? 1 : 0;
                if (gave)
                    __hip_atomic_store(a->status, kWindowGaveUp, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
            asm volatile("" ::: "memory");
            lds_barrier();
            asm volatile("" ::: "memory");
            const bool load = resume && *gave_up_l == 0;
            // (a tile started here reads through an empty buffer: zeros, with
            // no memory access and no branch)
            const __amdgpu_buffer_rsrc_t rs =
                srd_b(a->partial + (load ? size_t(prev) * 65536 : 0),
                      load ? uint32_t(65536 * 4) : 0u);
            const uint32_t lo = uint32_t(wave * 32768 + lane * 16);
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const auto v = __builtin_amdgcn_raw_buffer_load_b128(
                        rs, lo + uint32_t((i * 4 + q) * 1024), 0, kDevScope);
                    float4v f;
                    __builtin_memcpy(&f, &v, 16);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[i][4 * q + e] = f[e];
                }
        }

        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

        // The four corner weights of tap k with the mask folded in:
        // (1-ly)(1-lx)m, (1-ly)lx m, ly(1-lx)m, ly lx m from t0 = (1-lx)m,
        // t1 = lx m and ly (all 0 for a sample that reads nothing).
        // (The factors pass through an empty asm at every use, so that the
        // compiler cannot hoist the weights, loop-invariant per tap, out of
        // the main loop and hold all 36 of them in registers.)
        auto weights_of = [&](int k, float (&w)[4]) {
            float t0 = gw[k][0], t1 = gw[k][1], ly = gw[k][2];
            asm volatile("" : "+v"(t0), "+v"(t1), "+v"(ly));
            w[0] = fmaf(-ly, t0, t0);
            w[1] = fmaf(-ly, t1, t1);
            w[2] = ly * t0;
            w[3] = ly * t1;
        };
        // A fragment of block i of step `step` (plane = half, row = 32i + lane%32)
        auto read_a = [&](uint4 (&fa)[8], int step) {
            const uint32_t so = __builtin_amdgcn_readfirstlane(
                uint32_t(kAOff + (step % kAStages) * kAStage));
            const char *st = smem + (a_lane + so);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                fa[i] = *reinterpret_cast<const uint4 *>(st + i * 32 * 16);
        };
        // corners of local tap k from window buffer `buf` (wide tiles, tap 8:
        // the wave's 8 bytes of each, into .x and .y)
        auto read_corners = [&](uint4 (&cr)[4], int k, int buf) {
            const uint32_t bo =
                __builtin_amdgcn_readfirstlane(uint32_t(L::win0 + (buf ? L::buf : 0)));
            uint32_t pk = gpk[k / 2];
            asm volatile("" : "+v"(pk));                 // (not hoisted: see weights_of)
            const uint32_t wa = (k % 2) ? (pk >> 16) : (pk & 0xffffu);
            const char *p = smem + (wa + bo);
            const char *p2 = p + wrow;
            if (WIDE && k == 4) {
                const uint2 v0 = *reinterpret_cast<const uint2 *>(p);
                const uint2 v1 = *reinterpret_cast<const uint2 *>(p + 16);
                const uint2 v2 = *reinterpret_cast<const uint2 *>(p2);
                const uint2 v3 = *reinterpret_cast<const uint2 *>(p2 + 16);
                cr[0].x = v0.x; cr[0].y = v0.y;
                cr[1].x = v1.x; cr[1].y = v1.y;
                cr[2].x = v2.x; cr[2].y = v2.y;
                cr[3].x = v3.x; cr[3].y = v3.y;
            } else {
                cr[0] = *reinterpret_cast<const uint4 *>(p);
                cr[1] = *reinterpret_cast<const uint4 *>(p + 16);
                cr[2] = *reinterpret_cast<const uint4 *>(p2);
                cr[3] = *reinterpret_cast<const uint4 *>(p2 + 16);
            }
        };

        if constexpr (!F8) {
            uint4 fa[8];
            uint4 cr[4];
            // step 0's A fragments and corners
            read_a(fa, 0);
            read_corners(cr, 0, 0);

            // Waves w and w + 4 share a SIMD.  Each step is a blend half (this
            // step's B from the corners read in the previous step, then the next
            // step's corner reads) and an MFMA half (8 MFMAs and the next step's
            // A fragment reads).  (Tried and slower: no workgroup barrier, waves
            // kept within two steps of each other by arrival counters in LDS --
            // with 8 A stages and copies 5 steps ahead a copy then has only two
            // steps to land, and the waves waited on each other 30 % of the time.)  At a barrier, waves 0-3 wait before their blend
            // half and waves 4-7 before their MFMA half, so after it the two
            // waves of a SIMD run opposite halves (the barrier is released once
            // all eight waves have reached one of the two sites).
            const bool late = wave >= 4;

            // One step: relative step s = rc*9 + k of chunk c_lo + rc.  The tap
            // k is a compile-time index so the geometry stays in registers.
            auto step_body = [&](int rc, auto kc) {
                constexpr int k = decltype(kc)::value;
                const int s = rc * kTaps + k;
                const int chunk = c_lo + rc;
                const bool last_chunk = chunk + 1 >= c_hi;
                // One barrier every third step (k = 0, 3, 6): every wave's copies
                // issued up to two steps before it have landed (each wave waits
                // for its own, then the barrier), which covers every A stage and
                // window read until the next barrier.  Still in flight: the A
                // copy of the previous step, at k == 3 the window copy of the next
                // chunk (issued in step k == 1 after that step's A copy, waited
                // for at k == 6, first read in step k == 8), and -- for waves 4-7,
                // which wait after their blend half -- the copies of this step.
                // Every copy overwrites data last read at least two steps before
                // the last barrier (A of step s + LEAD - 8; the window of chunk - 1,
                // last read in step 9*chunk - 2), which every wave passed.  (No LDS
                // wait is needed for that: every read was consumed by the step
                // that used it.)
                constexpr int kNoLgkm = 0x70 | 0xF00;     // expcnt and lgkmcnt: no wait
                auto barrier = [&](int own) {
                    // own: copies of this step already issued by this wave
                    const bool a_prev = s >= 1 && s - 1 + LEAD < steps;   // copied in step s-1
                    if (k == 3 && !last_chunk) {
                        if (own) {
                            constexpr int N = 2 * kAInstr + L::instr;
                            __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | kNoLgkm);
                        } else {
                            constexpr int N = kAInstr + L::instr;
                            __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | kNoLgkm);
                        }
                    } else if (a_prev && own) {
                        constexpr int N = 2 * kAInstr;
                        __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | kNoLgkm);
                    } else if (a_prev || own) {
                        constexpr int N = kAInstr;
                        __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | kNoLgkm);
                    } else {
                        __builtin_amdgcn_s_waitcnt(kNoLgkm);
                    }
                    __builtin_amdgcn_s_barrier();
                };
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                if (k % 3 == 0 && !late)
                    barrier(0);
                __builtin_amdgcn_sched_barrier(0);
                asm volatile("" ::: "memory");
                const bool copy_a = s + LEAD < steps;
                if (copy_a)
                    issue_a(s + LEAD);
                if (k == 1 && !last_chunk)
                    issue_window(chunk + 1, (rc + 1) & 1);

                // blend half: B of step s (the samples are the MFMA's A operand:
                // rows are pixels), then the corners of step s+1.  Reads past the
                // last step hit valid (stale) LDS and are never used.
                constexpr int k1 = (k + 1) % kTaps;
                const int rc1 = (k + 1 >= kTaps) ? rc + 1 : rc;
                uint4 b;
                {
                    float w[4];
                    weights_of(k, w);
                    b = blend<T>(cr[0], cr[1], cr[2], cr[3], w, zero);
                }
                if (fbw & (1u << k))
                    fallback(k, chunk, b);
                read_corners(cr, k1, rc1 & 1);

                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                if (k % 3 == 0 && late)
                    barrier(copy_a ? 1 : 0);
                __builtin_amdgcn_sched_barrier(0);
                asm volatile("" ::: "memory");

                // MFMA half: the MFMAs of step s (B: the weights; columns are
                // output channels), each followed by the read of its A fragment
                // for step s+1
                const uint32_t so = __builtin_amdgcn_readfirstlane(
                    uint32_t(kAOff + ((s + 1) % kAStages) * kAStage));
                const char *st = smem + (a_lane + so);
                // (at a raised wave priority: the SIMD's other wave, in its blend
                // half, fills the issue slots the MFMAs leave)
                __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    acc[i] = Mma<T>::step(b, fa[i], acc[i]);
                    fa[i] = *reinterpret_cast<const uint4 *>(st + i * 32 * 16);
                    __builtin_amdgcn_sched_barrier(0);
                }
                __builtin_amdgcn_s_setprio(0);
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
        } else {
            // ---- E4M3 main loop.  A chunk's 9 taps are three MFMA groups
            // (j = 0: taps 0-3 and j = 1: taps 4-7, each one 64-deep FP8
            // instruction per 32x32 block on the lane's 8 channels of four
            // taps, 32 bytes; j = 2: tap 8, one 16-deep instruction on 8
            // bytes).  Group q = 3*rc + j of the segment reads weight slot j.
            // The loop is software-pipelined: phase p blends group p (its B
            // operand built tap by tap, each tap's corners read one tap ahead)
            // and, interleaved with the blend, runs the MFMAs of group p-1, so
            // that the matrix cores work while the VALU blends.  Barrier X_p
            // ends phase p: every wave's copy of A(p) has landed (each wave
            // waits for its own copies, then the barrier) and, for p = 3c+1,
            // the window of chunk c+1, whose first corners phase p+1 reads.
            // During phase p+1 each wave issues its share of A(p+2) into slot
            // (p+2) % 3, the slot of A(p-1), whose MFMAs ran in phase p, and,
            // for p = 3c+1, then the window of chunk c+2 into the buffer of
            // chunk c, last read in phase p -- spread through the phase, one
            // copy instruction after every 8/D of its MFMAs (D: the phase's
            // copy instructions), so that the texture unit works through
            // them while the waves compute instead of stalling every wave's
            // issue right after the barrier.  In flight at X_p besides what
            // it waits for: A(p+1) and the windows issued in phase p (p =
            // 3c+2) or in phase p-1 with A(p) (p = 3c+3).
            const int nseg = c_hi - c_lo;
            const int nq = 3 * nseg;
            const int hh = lane >> 5;
            // the lane's A fragment of block i (slot row 256*sub + 32i + lane%32,
            // R = L::rows): four-tap slot j part p at j*L::quad + q8_lane +
            // p*16R + i*512; tap-8 slot at s8_lane + i*256
            const int arow = sub * 256 + (lane & 31);
            const uint32_t q8_lane = uint32_t(hh * (32 * L::rows) + arow * 16);
            const uint32_t s8_lane = uint32_t(2 * L::quad + hh * (8 * L::rows) + arow * 8);
            constexpr int kNoLgkm = 0x70 | 0xF00;
            // (wide tiles: a barrier also waits for the wave's exchange store)
            constexpr int kBarLgkm = WIDE ? 0x70 : kNoLgkm;

            uint4 cr[4];
            read_corners(cr, 0, 0);
            // after the prologue's wait and barrier: window(1) (A(1) goes out
            // in phase 0)
            if (nseg > 1)
                issue_window(c_lo + 1, 1);

            // B operands: of the group being blended and of the one whose
            // MFMAs run meanwhile
            uint32_t bcur[8] = {}, bprev[8] = {};

            // A fragment of block i of group jm (compile time) from its slot
            auto frag64 = [&](int jm, int i) {
                const char *st = smem + (uint32_t(jm * L::quad) + q8_lane);
                const int4v lo = *reinterpret_cast<const int4v *>(st + i * 512);
                const int4v hi = *reinterpret_cast<const int4v *>(st + 16 * L::rows + i * 512);
                return int8v(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            };
            auto frag16 = [&](int i) {
                return *reinterpret_cast<const long *>(smem + s8_lane + i * 256);
            };

            // barrier X_p and the copies issued after it (p = 3*rc + j)
            auto barrier_issue = [&](int rc, auto jc) {
                constexpr int j = decltype(jc)::value;
                const int p = 3 * rc + j;
                const bool a_next = p + 1 < nq;
                // window issued after X_{p-1} (p = 3c+2: chunk c+1 < nseg-1)
                // or after X_{p-2}, with A(p) (p = 3c+3, c = rc-1: chunk rc+1)
                const bool w_younger = (j == 2 && rc + 2 < nseg) || (j == 0 && rc >= 1 &&
                                                                     rc + 1 < nseg);
                if (p == 0) {
                    // A(0) landed before the loop; window(1), A(1) may fly
                    constexpr int N = L::a8 + L::instr;
                    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | kBarLgkm);
                } else if (a_next && w_younger) {
                    constexpr int N = L::a8 + L::instr;
                    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | kBarLgkm);
                } else if (a_next) {
                    constexpr int N = L::a8;
                    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | kBarLgkm);
                } else if (w_younger) {
                    constexpr int N = L::instr;
                    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | kBarLgkm);
                } else {
                    __builtin_amdgcn_s_waitcnt(kBarLgkm);
                }
                __builtin_amdgcn_s_barrier();
            };

            // Phase p = 3*rc + j: blend group (rc, j) into bcur while the
            // MFMAs of group p-1 (type jm, operand bprev) run, if any.  Wide
            // tiles: each wave of a SIMD blends half of the group (local taps
            // 2j, 2j+1 -- its two of the four -- or its 4 channels of tap 8)
            // and stores its E4M3 bytes into the pair's exchange entry of
            // parity p % 2: [half s][lane][16 bytes] (tap 8: [half s][lane][4
            // bytes]); the MFMAs of group p, in phase p+1, read both halves
            // back -- the bytes of half s are exactly the operand's bytes
            // 16s..16s+15 (tap 8: 4s..4s+3) -- after barrier X_p, which waits
            // for the stores.  The entry is written again in phase p+2, after
            // barrier X_{p+1}, by when both reads have returned.
            auto phase = [&](int rc, auto jc, auto mfc) {
                constexpr int j = decltype(jc)::value;
                constexpr bool mfma = decltype(mfc)::value;
                constexpr int jm = (j + 2) % 3;            // the previous group's type
                constexpr int nt = j < 2 ? (WIDE ? 2 : 4) : 1;   // (local) taps
                constexpr int k0 = (WIDE ? 2 : 4) * j;     // first local tap
                constexpr int per = 8 / nt;                // MFMAs per tap
                const int chunk = c_lo + rc;
                const int p = 3 * rc + j;
                // phase 0 of the segment has no previous group: its MFMAs
                // multiply zero fragments (whatever the slot holds)
                const bool live = j != 0 || rc > 0;
                int8v bop64 = {};
                long bop16 = 0;
                if constexpr (WIDE) {
                    const char *xr =
                        smem + (uint32_t(L::xch + ((p + 1) & 1) * 8192) + uint32_t(pair * 2048));
                    if constexpr (jm < 2) {
                        const int4v lo = *reinterpret_cast<const int4v *>(xr + lane * 16);
                        const int4v hi = *reinterpret_cast<const int4v *>(xr + 1024 + lane * 16);
                        bop64 = int8v(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    } else {
                        const uint32_t d0 = *reinterpret_cast<const uint32_t *>(xr + lane * 4);
                        const uint32_t d1 =
                            *reinterpret_cast<const uint32_t *>(xr + 256 + lane * 4);
                        bop16 = live ? long(uint64_t(d0) | (uint64_t(d1) << 32)) : 0;
                    }
                } else {
                    bop64 = int8v{int(bprev[0]), int(bprev[1]), int(bprev[2]), int(bprev[3]),
                                  int(bprev[4]), int(bprev[5]), int(bprev[6]), int(bprev[7])};
                    bop16 = long(uint64_t(bprev[0]) | (uint64_t(bprev[1]) << 32));
                }
                // This phase's copies: A(p+1) (type ja of relative chunk rca)
                // and, for j = 2, then the window of chunk rc+2, as kD
                // instructions, instruction d after MFMA d*kStride.  A copy
                // past the segment's end is not skipped by a branch, which
                // would split the tap's block: its scalar offset is 2^31
                // instead, which takes a lane's offset past the buffer's
                // range (zeros) or, for a lane already at kOOB, wraps around
                // to an in-range read -- either way it fills a slot or
                // buffer that no wave reads again in this segment (and the
                // next tile's copies are issued after the main loop's final
                // full wait).
                constexpr int ja = (j + 1) % 3;
                const int rca = rc + (j + 1) / 3;
                constexpr int kD = L::a8 + (j == 2 ? L::instr : 0);
                constexpr int kStride = kD >= 8 ? 1 : 8 / kD;
                static_assert(kD <= 8, "one copy instruction per MFMA at most");
                const bool dma_a = p + 1 < nq;
                const bool dma_w = j == 2 && rc + 2 < nseg;
                const uint32_t soff_a = __builtin_amdgcn_readfirstlane(
                    dma_a ? uint32_t(c_lo + rca) * a_chunk + uint32_t(ja) * a_region : kOOB);
                const uint32_t soff_w = __builtin_amdgcn_readfirstlane(
                    dma_w ? ch_base + uint32_t((c_lo + rc + 2) * 2) * hw16 : kOOB);
                // window copy source offsets, each read one copy ahead (the
                // 256-channel kernels keep them in the LDS table: registers
                // for all of them would spill)
                auto woff_entry = [&](int t) {
                    if constexpr (WIDE)
                        return wsrc[t];
                    else
                        return woff_tab[t * kThreads + tid];
                };
                uint32_t wcur = 0;
                if constexpr (j == 2)
                    wcur = woff_entry(0);
                auto copy_after = [&](int i) {
                    if (i % kStride != 0 || i / kStride >= kD)
                        return;
                    const int d = i / kStride;
                    if (d < L::a8) {
                        if constexpr (ja < 2)
                            dma16(lds0 + ja * L::quad + (d * kWaves + wave) * 1024, ra, aoff[d],
                                  soff_a);
                        else
                            dma4(lds0 + 2 * L::quad + (d * kWaves + wave) * 256, ra,
                                 aoff[L::a8 + d], soff_a);
                    } else if constexpr (j == 2) {
                        const int t = d - L::a8;
                        const uint32_t wo = wcur;
                        if (t + 1 < L::instr)
                            wcur = woff_entry(t + 1);
                        dma16(lds0 + L::win0 + uint32_t(rc & 1) * L::buf + (t * kWaves + wave) * 1024 +
                                  ((t * kWaves + wave) * 64 >= L::px ? kPlaneGap : 0),
                              rx, wo, soff_w);
                    }
                };
                // fragments of MFMAs i and i+1 in flight (read two ahead)
                int8v f64[2];
                long f16[2];
                if constexpr (mfma) {
                    if constexpr (jm < 2) {
                        f64[0] = frag64(jm, 0);
                        f64[1] = frag64(jm, 1);
                    } else {
                        f16[0] = frag16(0);
                        f16[1] = frag16(1);
                    }
                }
                auto mma = [&](int i) {
                    if constexpr (jm < 2) {
                        const int8v f = f64[i & 1];
                        if (i + 2 < 8)
                            f64[i & 1] = frag64(jm, i + 2);
                        acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            bop64, f, acc[i], 0, 0, 0, 0, 0, 0);
                    } else {
                        const long f = live ? f16[i & 1] : 0;
                        if (i + 2 < 8)
                            f16[i & 1] = frag16(i + 2);
                        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(bop16, f, acc[i], 0,
                                                                            0, 0);
                    }
                };
                uint32_t own[4] = {};                      // wide: the wave's half
#pragma unroll
                for (int tt = 0; tt < nt; ++tt) {
                    const int k = k0 + tt;
                    const int k1 = (k + 1) % kLT;
                    const int buf1 = (k + 1 >= kLT) ? ((rc + 1) & 1) : (rc & 1);
                    uint4 cn[4];
                    read_corners(cn, k1, buf1);
                    float w[4];
                    weights_of(k, w);
                    // the tap's share of the previous group's MFMAs, spread
                    // through its blend FMAs (one basic block: the scheduler
                    // interleaves them as the group barriers ask)
#pragma unroll
                    for (int u = 0; u < per; ++u) {
                        if constexpr (mfma)
                            mma(tt * per + u);
                        copy_after(tt * per + u);
                    }
                    if (WIDE && k == 4) {
                        // wide tiles, tap 8: the wave's 4 channels
                        float bf[4];
                        blend_f32_4<T>(cr, w, zero, bf);
                        if constexpr (mfma) {
#pragma unroll
                            for (int u = 0; u < per; ++u) {
                                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                                __builtin_amdgcn_sched_group_barrier(0x002, 16 / per, 0);
                            }
                        }
                        const uint32_t b4 = e4m3_of4(bf);
                        uint2 b8 = make_uint2(b4, b4);
                        if (fbw & (1u << k))
                            fallback(k, chunk, b8);
                        own[0] = sub ? b8.y : b8.x;
                    } else {
                        float bf[8];
                        blend_f32<T>(cr, w, zero, bf);
                        if constexpr (mfma) {
#pragma unroll
                            for (int u = 0; u < per; ++u) {
                                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // MFMA
                                __builtin_amdgcn_sched_group_barrier(0x002, 32 / per, 0);   // VALU
                            }
                        }
                        uint2 b8 = e4m3_of(bf);
                        if (fbw & (1u << k))
                            fallback(k, chunk, b8);
                        if constexpr (WIDE) {
                            own[2 * tt] = b8.x;
                            own[2 * tt + 1] = b8.y;
                        } else {
                            bcur[2 * tt] = b8.x;
                            bcur[2 * tt + 1] = b8.y;
                        }
                    }
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        cr[c] = cn[c];
                    __builtin_amdgcn_sched_barrier(0);
                }
                if constexpr (WIDE) {
                    char *xw = smem + (uint32_t(L::xch + (p & 1) * 8192) + uint32_t(pair * 2048));
                    if constexpr (j < 2)
                        *reinterpret_cast<uint4 *>(xw + sub * 1024 + lane * 16) =
                            make_uint4(own[0], own[1], own[2], own[3]);
                    else
                        *reinterpret_cast<uint32_t *>(xw + sub * 256 + lane * 4) = own[0];
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        bprev[e] = bcur[e];
                }
            };
            // the last group's MFMAs (type 2), after the last phase's barrier
            auto tail = [&]() {
                long bop16;
                if constexpr (WIDE) {
                    const char *xr = smem + (uint32_t(L::xch + ((nq - 1) & 1) * 8192) +
                                             uint32_t(pair * 2048));
                    const uint32_t d0 = *reinterpret_cast<const uint32_t *>(xr + lane * 4);
                    const uint32_t d1 = *reinterpret_cast<const uint32_t *>(xr + 256 + lane * 4);
                    bop16 = long(uint64_t(d0) | (uint64_t(d1) << 32));
                } else {
                    bop16 = long(uint64_t(bprev[0]) | (uint64_t(bprev[1]) << 32));
                }
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(bop16, frag16(i), acc[i],
                                                                        0, 0, 0);
            };

            using yes = std::true_type;
            auto chunk_body = [&](int rc) {
                phase(rc, std::integral_constant<int, 0>{}, yes{});
                asm volatile("" ::: "memory");
                barrier_issue(rc, std::integral_constant<int, 0>{});
                asm volatile("" ::: "memory");
                phase(rc, std::integral_constant<int, 1>{}, yes{});
                asm volatile("" ::: "memory");
                barrier_issue(rc, std::integral_constant<int, 1>{});
                asm volatile("" ::: "memory");
                phase(rc, std::integral_constant<int, 2>{}, yes{});
                asm volatile("" ::: "memory");
                barrier_issue(rc, std::integral_constant<int, 2>{});
                asm volatile("" ::: "memory");
            };
            for (int rc = 0; rc < nseg; ++rc)
                chunk_body(rc);
            tail();
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
            const uint32_t lo = uint32_t((tid >> 6) * 32768 + (tid & 63) * 16);
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4v f = {acc[i][4 * q], acc[i][4 * q + 1], acc[i][4 * q + 2],
                                       acc[i][4 * q + 3]};
                    u32x4 u;
                    __builtin_memcpy(&u, &f, 16);
                    __builtin_amdgcn_raw_buffer_store_b128(u, rs, lo + uint32_t((i * 4 + q) * 1024),
                                                           0, kDevScope);
                }
            // The flag goes out once these device-scope stores are complete
            // (acknowledged where every XCD sees them).  Rather than draining
            // the counter here, the next tile's prologue sets it after its
            // own copies are issued: its counter wait then covers these
            // older stores.  The workgroup that finishes the tile reads the
            // flag only at the end of its range, so the later flag costs
            // nothing, and it still precedes any hand-over wait of this
            // workgroup (no chain of waits between neighbours).
            asm volatile("" ::: "memory");
            flag_pending = true;
        } else {
            // ---- the tile's last chunks: + bias in fp32, one rounding,
            // stores straight from the accumulators.  Register r of block i
            // holds output channel m0 + 32i + lane%32 at tile pixel
            // 32*wave + 8(r/4) + 4(lane/32) + r%4 (wide tiles: channel
            // m0 + 256*(wave/4) + 32i + lane%32 at pixel 32*(wave%4) + ...).  For each half h of the
            // wave's 32 pixels, one lane swap (v_permlane32_swap: lanes
            // 32..63 of the first register with lanes 0..31 of the second)
            // gives lanes < 32 pixels 16h..16h+7 and lanes >= 32 pixels
            // 16h+8..16h+15 of their channel: one 16-byte store each.  No load
            // is issued between the stores (on this GPU a load's wait also
            // waits for every older store): the bias comes first.
            const int Mg = a->Mg, P = a->P, Ho = a->Ho, Wo = a->Wo;
            const int wv = tid >> 6, ln = tid & 63;
            const int wsub = WIDE ? (wv >> 2) : 0, wpair = WIDE ? (wv & 3) : wv;
            float bv[8];
            float sv[8];                             // F8: the rows' 2^-e
            {
                const T *bias = static_cast<const T *>(a->bias);
                // the hand-over wait of this tile gave up: NaN for all of it
                const bool poison = te.c_lo > 0 && *gave_up_l != 0;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int m = te.m0 + 256 * wsub + 32 * i + (ln & 31);
                    bv[i] = (bias && m < Mg) ? to_f32(bias[size_t(te.g) * Mg + m]) : 0.0f;
                    if (poison)
                        bv[i] = __builtin_nanf("");
                    if constexpr (F8)
                        sv[i] = m < Mg ? a->wscale[size_t(te.g) * Mg + m] : 0.0f;
                }
            }
            // output planes of the tile's image and group, as a buffer (a
            // lane with nothing to store gets an out-of-range offset)
            const __amdgpu_buffer_rsrc_t ro =
                srd_b(static_cast<const T *>(a->out) +
                          (size_t(te.img) * a->Co + size_t(te.g) * a->Mg) * a->P,
                      uint32_t(size_t(Mg) * P * sizeof(T)));
            const bool vec = a->vec_out != 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int m = te.m0 + 256 * wsub + 32 * i + (ln & 31);
                const bool mok = m < Mg;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float16v &c = acc[i];
                    const float bb = bv[i];
                    // (F8: 2^-e * sum + bias, one rounding: the product is exact)
                    auto o = [&](int r) {
                        if constexpr (F8)
                            return fmaf(c[8 * h + r], sv[i], bb);
                        else
                            return c[8 * h + r] + bb;
                    };
                    const uint32_t v0 = pack2<T>(o(0), o(1));
                    const uint32_t v1 = pack2<T>(o(2), o(3));
                    const uint32_t v2 = pack2<T>(o(4), o(5));
                    const uint32_t v3 = pack2<T>(o(6), o(7));
                    const auto w0 = __builtin_amdgcn_permlane32_swap(v0, v2, false, false);
                    const auto w1 = __builtin_amdgcn_permlane32_swap(v1, v3, false, false);
                    const u32x4 ov = {uint32_t(w0[0]), uint32_t(w1[0]), uint32_t(w0[1]),
                                      uint32_t(w1[1])};
                    const int n = wpair * 32 + 16 * h + 8 * (ln >> 5);
                    int ho, wo;
                    out_pixel(n, te.ho0, te.wo0, Wo, ho, wo);
                    const bool ok = mok && ho < Ho && wo < Wo;
                    const uint32_t base =
                        ok ? (uint32_t(m) * uint32_t(P) + uint32_t(ho * Wo + wo)) *
                                 uint32_t(sizeof(T))
                           : kOOB;
                    if (vec) {
                        // (with vec, 8-pixel runs stay inside a row or, for
                        // flat tiles, inside the plane)
                        __builtin_amdgcn_raw_buffer_store_b128(ov, ro, base, 0, 0);
                    } else {
                        const uint32_t ow[4] = {ov[0], ov[1], ov[2], ov[3]};
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const bool in = kFlat ? ho * Wo + wo + e < Ho * Wo : wo + e < Wo;
                            __builtin_amdgcn_raw_buffer_store_b16(
                                uint16_t(ow[e >> 1] >> (16 * (e & 1))), ro,
                                in ? base + uint32_t(e) * uint32_t(sizeof(T)) : kOOB, 0, 0);
                        }
                    }
                }
            }
        }
        if (tile <= int(rg.u0 / uint32_t(a->nch)))
            break;                                   // that was the range's first tile
        --tile;
    }
    if (flag_pending) {
        // the range held only the published tile: drain, then the flag
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (threadIdx.x == 0) {
            KArgs af = fresh_args(pa);
            __hip_atomic_store(af->flags + cta, uint32_t(af->epoch), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
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

template <typename T, int TH, int TW, int LEAD, bool F8, bool WIDE>
hipError_t window_cfg(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                      const float *wscale, const void *xt, const void *offset, const void *mask,
                      const void *bias, void *out, const WindowScratch &ws, hipStream_t s)
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
    constexpr int tile_px = TH * TW, tile_m = WIDE ? 512 : 256;
    a.WR = int(window_extent(flat ? window_flat_rows(p.Wo, tile_px) : TH, p.sh, p.kh, p.dh,
                             plan.win_margin));
    a.WC = int(window_extent(flat ? p.Wo : TW, p.sw, p.kw, p.dw, plan.win_margin));
    a.tiles_y = int(flat ? (p.P + tile_px - 1) / tile_px : (p.Ho + TH - 1) / TH);
    a.tiles_x = int(flat ? 1 : (p.Wo + TW - 1) / TW);
    a.tiles_m = int((p.Mg + tile_m - 1) / tile_m);
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
    // offsets and masks reach LDS by 4-byte DMA when every tile pixel pair
    // (even pixel, same row or, flat, same plane) is a 4-byte aligned pair
    const uint64_t off_bytes = uint64_t(cnt) * uint64_t(a.offC) * uint64_t(p.P) * sizeof(T);
    const uint64_t msk_bytes = uint64_t(cnt) * uint64_t(a.mskC) * uint64_t(p.P) * sizeof(T);
    if (off_bytes >= (uint64_t(1) << 31) || msk_bytes >= (uint64_t(1) << 31))
        return hipErrorInvalidValue;
    a.off_bytes = uint32_t(off_bytes);
    a.msk_bytes = uint32_t(msk_bytes);
    a.om_lds = p.P % 2 == 0 && (flat || p.Wo % 2 == 0) &&
               reinterpret_cast<uintptr_t>(offset) % 4 == 0 &&
               reinterpret_cast<uintptr_t>(mask) % 4 == 0;
    a.spin_limit = plan.win_spin_limit;
    // one group's weight (F8: its E4M3 chunk blocks)
    a.a_bytes = F8 ? uint32_t(size_t(p.Cg / kCC) * size_t(p.Mg) * kWindowFp8ChunkBytesPerRow)
                   : uint32_t(size_t(p.Mg) * p.Kg * sizeof(T));
    if (F8 && !wscale)
        return hipErrorInvalidValue;
    if (a.WR * a.WC > WinLds<F8, WIDE>::px || a.WC * 16 + 32 > kWinZero)
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
        {tiles, uint64_t(std::max(1, device_cu_count())), uint64_t(std::max(1, ws.slots))});
    if (plan.win_max_ctas > 0)
        blocks = std::min<uint64_t>(blocks, uint64_t(plan.win_max_ctas));
    if (ws.epoch <= 0 || (blocks < tiles && (!ws.partial || !ws.flags)))
        return hipErrorInvalidValue;
    if (!split_cached(int64_t(tiles), int64_t(a.nch), int64_t(blocks), plan.win_seg_cost_x4,
                      a.bounds))
        return hipErrorInvalidValue;
    auto kern = window_kernel<T, TH, TW, LEAD, F8, WIDE>;
    constexpr int lds = WinLds<F8, WIDE>::total;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (attr != hipSuccess)
        return attr;
    a.A = wpack; a.xt = xt; a.off = offset; a.msk = mask; a.bias = bias; a.out = out;
    a.wscale = wscale;
    a.partial = ws.partial; a.flags = ws.flags; a.status = ws.flags + ws.slots;
    hipLaunchKernelGGL(kern, dim3(uint32_t(blocks)), dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

template <typename T, int TH, int TW>
hipError_t window_lead(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                       const float *wscale, const void *xt, const void *offset, const void *mask,
                       const void *bias, void *out, const WindowScratch &ws, hipStream_t s)
{
    if (plan.win_lead != 5)
        return hipErrorInvalidValue;
    if constexpr (TH * TW == 128) {
        if (plan.path != Path::WindowFp8 || !plan.win_wide)
            return hipErrorInvalidValue;
        return window_cfg<T, TH, TW, 5, true, true>(p, plan, cnt, wpack, wscale, xt, offset, mask,
                                                    bias, out, ws, s);
    } else {
        if (plan.win_wide)
            return hipErrorInvalidValue;
        if (plan.path == Path::WindowFp8)
            return window_cfg<T, TH, TW, 5, true, false>(p, plan, cnt, wpack, wscale, xt, offset,
                                                         mask, bias, out, ws, s);
        return window_cfg<T, TH, TW, 5, false, false>(p, plan, cnt, wpack, wscale, xt, offset,
                                                      mask, bias, out, ws, s);
    }
}

template <typename T>
hipError_t window_t(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                    const float *wscale, const void *xt, const void *offset, const void *mask,
                    const void *bias, void *out, const WindowScratch &ws, hipStream_t s)
{
    switch (plan.win_tile) {
    case WindowTile::H16_W16:
        return window_lead<T, 16, 16>(p, plan, cnt, wpack, wscale, xt, offset, mask, bias, out,
                                      ws, s);
    case WindowTile::H8_W32:
        return window_lead<T, 8, 32>(p, plan, cnt, wpack, wscale, xt, offset, mask, bias, out,
                                     ws, s);
    case WindowTile::H32_W8:
        return window_lead<T, 32, 8>(p, plan, cnt, wpack, wscale, xt, offset, mask, bias, out,
                                     ws, s);
    case WindowTile::FLAT:
        return window_lead<T, 1, 256>(p, plan, cnt, wpack, wscale, xt, offset, mask, bias, out,
                                      ws, s);
    case WindowTile::H8_W16:
        return window_lead<T, 8, 16>(p, plan, cnt, wpack, wscale, xt, offset, mask, bias, out,
                                     ws, s);
    case WindowTile::H16_W8:
        return window_lead<T, 16, 8>(p, plan, cnt, wpack, wscale, xt, offset, mask, bias, out,
                                     ws, s);
    case WindowTile::FLAT128:
        return window_lead<T, 1, 128>(p, plan, cnt, wpack, wscale, xt, offset, mask, bias, out,
                                      ws, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_window(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                         const float *wscale, const void *xt, const void *offset,
                         const void *mask, const void *bias, void *out, const WindowScratch &ws,
                         hipStream_t stream)
{
    switch (p.dtype) {
    case MDCN_F16:
        return window_t<half_t>(p, plan, cnt, wpack, wscale, xt, offset, mask, bias, out, ws,
                                stream);
    case MDCN_BF16:
        return window_t<bf16_t>(p, plan, cnt, wpack, wscale, xt, offset, mask, bias, out, ws,
                                stream);
    case MDCN_F32:
        break;
    }
    return hipErrorInvalidValue;
}

// Compute units of the current device (cached per device).
int device_cu_count()
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

}  // namespace mdcn
