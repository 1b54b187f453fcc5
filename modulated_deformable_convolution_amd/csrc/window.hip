// window.hip -- the deformable gather fused into the MFMA GEMM, with the
// input window of each output tile staged in LDS.
//   out[n][g*Mg + m][ho][wo] = bias[g*Mg + m]
//       + sum_{k, c'} A[g][m][k*Cg + c'] * mask * bilinear0(x[n][g*Cg + c'], sample(k, ho, wo))
// [plugin guide §五 steps 1-3, without a columns buffer between step 1 and 2].
//
// A workgroup (4 waves, one per SIMD) computes 256 output channels x one
// TH x TW tile of output pixels (256 pixels) of one image and group.  The
// contraction runs chunk-major: for each chunk of 16 input channels, the
// rectangle of input pixels that the tile's samples can reach -- the anchors
// of all taps plus a margin of `margin` pixels on every side for the offsets
// -- is copied into LDS once (the "window", channels-last, two planes of 8
// channels), and the 9 taps of the chunk are then 9 K-steps that read their
// bilinear corners from it.  A sample with a corner on the image that falls
// outside the window is rare with the margin sized for the offsets; its lane
// reads zeros from the window and its value is computed from global memory
// instead (the fallback), so the result does not depend on the margin.
//
// Every wave owns 64 pixels (two slabs of 32) and all 256 output channels:
// it makes the B fragments of its own pixels in registers (lane l of a slab
// owns pixel l%32 and channels 8*(l/32)..+8 of the chunk, which is exactly
// the MFMA B-fragment layout), so B never goes through LDS, and reads the A
// fragments (packed weight rows) from LDS stages filled by DMA three steps
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
//   window buffer b (b = 0, 1): [plane 0: kWinPx x 16][plane 1: kWinPx x 16][zeros: kWinZero]
//   window copy table:          [instruction t][thread]: source byte offset of the
//                               thread's 16 bytes of window copy instruction t
//   A stage s (s = 0..LEAD):    [plane 0: 256 rows x 16][plane 1: 256 rows x 16]
// Plane p of an entry holds channels 8p..8p+7 of the chunk.
constexpr int kWinPlane = kWindowPixels * 16;
constexpr int kWinZero = kWindowZeroBytes;
constexpr int kWinBuf = 2 * kWinPlane + kWinZero;
constexpr int kAStage = 256 * 2 * 16;
constexpr int kWinInstr = 2 * kWindowPixels / 64 / 4;   // window DMA instructions per wave
constexpr int kWoffOff = 2 * kWinBuf;
constexpr int kAOff = kWoffOff + kWinInstr * 256 * 4;
// A stages: the copy of step s+LEAD is issued in step s, into one of LEAD+1
// stages.
constexpr int lds_total(int lead) { return kAOff + (lead + 1) * kAStage; }
constexpr int kAInstr = kAStage / 1024 / 4;             // A DMA instructions per wave
constexpr int kEpRow = 256 + 4;                          // epilogue slice row, floats
static_assert(lds_total(kWindowMaxLead) <= int(kLdsBytes), "LDS budget");
static_assert(32 * kEpRow * 4 <= lds_total(2), "epilogue slice must fit");
static_assert((2 * kWindowPixels) % 256 == 0, "window DMA covers whole wave instructions");

struct WinArgs {
    int Mg, Kp, Co, P, Ho, Wo;
    int C, H, W, Cg, nch;          // nch: chunks of 16 channels per group
    int sh, sw, ph, pw, dh, dw;
    int margin, WR, WC;            // window rows / columns
    int tiles_x, tiles_y, tiles_m, cnt;
    int offC, mskC, Cdg;           // offset / mask channels per image; C / deformable_group
    int has_bias, vec_out;
    uint32_t img_bytes, chunk_bytes, a_bytes;
};

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
void window_kernel(const T *__restrict__ A, const T *__restrict__ xt, const T *__restrict__ off,
                   const T *__restrict__ msk, const T *__restrict__ bias, T *__restrict__ out,
                   WinArgs a)
{
    static_assert(TH * TW == 256 && TW % 8 == 0, "a tile is 256 pixels, rows of 8-pixel vectors");
    static_assert(LEAD >= 2 && LEAD + 1 <= 9, "copies lead by 2..8 steps");
    constexpr int kAStages = LEAD + 1;
    constexpr int E = int(sizeof(T));
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    // ---- workgroup -> (group, image, tile row, tile column, channel tile)
    uint32_t bid = xcd_swizzle(blockIdx.x, gridDim.x);
    const int mt = int(bid % uint32_t(a.tiles_m));
    bid /= uint32_t(a.tiles_m);
    const int tx = int(bid % uint32_t(a.tiles_x));
    bid /= uint32_t(a.tiles_x);
    const int ty = int(bid % uint32_t(a.tiles_y));
    bid /= uint32_t(a.tiles_y);
    const int img = int(bid % uint32_t(a.cnt));
    const int g = __builtin_amdgcn_readfirstlane(int(bid / uint32_t(a.cnt)));
    const int m0 = mt * 256;
    const int ho0 = ty * TH, wo0 = tx * TW;
    const int r0 = ho0 * a.sh - a.ph - a.margin;     // window origin (input coordinates)
    const int c0 = wo0 * a.sw - a.pw - a.margin;
    const int q = (g * a.Cg) / a.Cdg;                // the group's offset group

    const int tid = int(threadIdx.x);
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;                      // plane: channels 8*half..+8 of a chunk

    const uint32_t lds0 = lds_addr(smem);
    const v4i rx = srd(xt, a.chunk_bytes);
    const v4i ra = srd(reinterpret_cast<const char *>(A) + size_t(g) * a.a_bytes, a.a_bytes);
    const uint32_t hw16 = uint32_t(a.H * a.W) * 16;   // bytes of one 8-channel block plane

    // ---- per-lane DMA source offsets of the window (per tile, kept in LDS)
    // and of the A rows
    uint32_t *woff_tab = reinterpret_cast<uint32_t *>(smem + kWoffOff);
#pragma unroll
    for (int t = 0; t < kWinInstr; ++t) {
        const int S = (t * 4 + wave) * 64 + lane;          // 16-byte slot of the buffer
        const int pl = S / kWindowPixels;
        const int px = S - pl * kWindowPixels;
        const int r = px / a.WC, c = px - (px / a.WC) * a.WC;
        const int gr = r0 + r, gc = c0 + c;
        const bool ok = px < a.WR * a.WC && (unsigned)gr < (unsigned)a.H &&
                        (unsigned)gc < (unsigned)a.W;
        const uint32_t o = ok ? uint32_t(img) * a.img_bytes + uint32_t(pl) * hw16 +
                                    uint32_t(gr * a.W + gc) * 16
                              : kOOB;
        woff_tab[t * 256 + tid] = o;
    }
    uint32_t aoff[kAInstr];
#pragma unroll
    for (int t = 0; t < kAInstr; ++t) {
        const int S = (t * 4 + wave) * 64 + lane;
        const int pl = S >> 8, row = S & 255;
        aoff[t] = (m0 + row < a.Mg) ? uint32_t(pl * a.Mg + m0 + row) * 16 : kOOB;
    }
    // the group's first 8-channel block plane, bytes
    const uint32_t ch_base = uint32_t(g * a.Cg / 8) * hw16;
    // (the table is read back only after the barrier that follows its writes)
    auto issue_window = [&](int chunk, int buf) {
        const uint32_t soff = __builtin_amdgcn_readfirstlane(ch_base + uint32_t(chunk * 2) * hw16);
        uint32_t wo[kWinInstr];                 // all table reads first: one LDS wait
#pragma unroll
        for (int t = 0; t < kWinInstr; ++t)
            wo[t] = woff_tab[t * 256 + tid];
#pragma unroll
        for (int t = 0; t < kWinInstr; ++t)
            dma16(lds0 + buf * kWinBuf + (t * 4 + wave) * 1024, rx, wo[t], soff);
    };
    const int steps = a.nch * kTaps;
    auto issue_a = [&](int step) {
        const uint32_t soff = __builtin_amdgcn_readfirstlane(uint32_t(step * 2 * a.Mg) * 16);
#pragma unroll
        for (int t = 0; t < kAInstr; ++t)
            dma16(lds0 + kAOff + (step % kAStages) * kAStage + (t * 4 + wave) * 1024, ra, aoff[t],
                  soff);
    };

    // ---- prologue copies: window of chunk 0, A of steps 0 .. LEAD-1
    issue_window(0, 0);
#pragma unroll
    for (int s = 0; s < LEAD; ++s)
        if (s < steps)
            issue_a(s);

    // ---- sampling geometry of the lane's two pixels, all taps
    uint32_t gaddr[2][kTaps];
    float gw[2][kTaps][4];
    uint32_t fbl = 0;                                // lane: (slab, tap) needs the fallback
    {
        const int P = a.P;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int n = (wave * 2 + s) * 32 + (lane & 31);
            const int ho = ho0 + n / TW, wo = wo0 + n % TW;
            const bool pv = ho < a.Ho && wo < a.Wo;
            const int pix = pv ? ho * a.Wo + wo : 0;
            const size_t ob = (size_t(img) * a.offC + size_t(q) * 2 * kTaps) * P + pix;
            const size_t mb = (size_t(img) * a.mskC + size_t(q) * kTaps) * P + pix;
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
                const int ah = ho * a.sh - a.ph + i * a.dh;
                const int aw = wo * a.sw - a.pw + j * a.dw;
                const float lim = 33554432.0f;
                const bool fin = fabsf(oh[k]) <= lim && fabsf(ow[k]) <= lim;
                const float fh = fin ? floorf(oh[k]) : 0.0f;
                const float fw = fin ? floorf(ow[k]) : 0.0f;
                const float ly = fin ? oh[k] - fh : 0.0f;
                const float lx = fin ? ow[k] - fw : 0.0f;
                const int h0 = ah + int(fh), w0 = aw + int(fw);
                const bool any = pv && fin && h0 >= -1 && h0 < a.H && w0 >= -1 && w0 < a.W;
                const int lr = h0 - r0, lc = w0 - c0;
                const bool inw = (unsigned)lr <= unsigned(a.WR - 2) &&
                                 (unsigned)lc <= unsigned(a.WC - 2);
                const bool use = any && inw;
                const float hy = 1.0f - ly, hx = 1.0f - lx, m = mm[k];
                gw[s][k][0] = use ? hy * hx * m : 0.0f;
                gw[s][k][1] = use ? hy * lx * m : 0.0f;
                gw[s][k][2] = use ? ly * hx * m : 0.0f;
                gw[s][k][3] = use ? ly * lx * m : 0.0f;
                gaddr[s][k] = use ? uint32_t(half * kWinPlane + (lr * a.WC + lc) * 16)
                                  : uint32_t(2 * kWinPlane);
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
            const int n = (wave * 2 + s) * 32 + (lane & 31);
            const int ho = ho0 + n / TW, wo = wo0 + n % TW;
            const int pix = ho * a.Wo + wo;
            const size_t ob = (size_t(img) * a.offC + size_t(q) * 2 * kTaps + 2 * k) * a.P + pix;
            const float oh = to_f32(off[ob]), ow = to_f32(off[ob + a.P]);
            const float m = to_f32(msk[(size_t(img) * a.mskC + size_t(q) * kTaps + k) * a.P + pix]);
            const int i = k / 3, j = k % 3;
            const Taps tp = make_taps(ho * a.sh - a.ph + i * a.dh, wo * a.sw - a.pw + j * a.dw,
                                      oh, ow, m, a.H, a.W);
            const uint32_t cb = ch_base + uint32_t(chunk * 2 + half) * hw16;
            uint4 cv[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t o = tp.valid[t]
                                       ? uint32_t(img) * a.img_bytes + uint32_t(tp.idx[t]) * 16 +
                                             cb
                                       : kOOB;
                const auto r = __builtin_amdgcn_raw_buffer_load_b128(
                    __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(xt), (short)0,
                                                      int(a.chunk_bytes), 0x00020000),
                    o, 0, 0);
                __builtin_memcpy(&cv[t], &r, 16);
            }
            const float w4[4] = {tp.wt[0], tp.wt[1], tp.wt[2], tp.wt[3]};
            bv = blend<T>(cv[0], cv[1], cv[2], cv[3], w4, 0.0f);
        }
    };

    // zero areas of both window buffers (read by lanes whose sample is not
    // in the window)
    for (int i = tid; i < 2 * kWinZero / 8; i += 256) {
        const int b = i / (kWinZero / 8), o = i - b * (kWinZero / 8);
        *reinterpret_cast<uint2 *>(smem + b * kWinBuf + 2 * kWinPlane + o * 8) = make_uint2(0u, 0u);
    }

    float16v acc[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][s][r] = 0.0f;

    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // A fragment of block i of step `step` (plane = half, row = 32i + lane%32)
    const uint32_t a_lane = uint32_t(half * (kAStage / 2) + (lane & 31) * 16);
    auto read_a = [&](uint4 (&fa)[8], int step) {
        const uint32_t so = __builtin_amdgcn_readfirstlane(
            uint32_t(kAOff + (step % kAStages) * kAStage));
        const char *st = smem + (a_lane + so);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            fa[i] = *reinterpret_cast<const uint4 *>(st + i * 32 * 16);
    };
    const uint32_t wrow = uint32_t(a.WC * 16);
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

    float zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
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
        fallback(0, 0, 0, b[0]);
        fallback(1, 0, 0, b[1]);
    }
    if (steps > 1) {
        read_corners(cr[0], 0, 1 % kTaps, 0);
        read_corners(cr[1], 1, 1 % kTaps, 0);
    }

    // One step: s = chunk*9 + k.  K (tap) is a compile-time index so the
    // geometry stays in registers.
    auto step_body = [&](int chunk, auto kc) {
        constexpr int k = decltype(kc)::value;
        const int s = chunk * kTaps + k;
        const bool last_chunk = chunk + 1 >= a.nch;
        // A of step s+1 (and, with it, every older copy) has landed; the
        // previous step's LDS reads are complete.  A(s+1) was issued in step
        // s+1-LEAD; issued after it, and allowed to be in flight: the A
        // copies of the LEAD-2 steps between, and the window copy of the
        // next chunk when a step k == 0 lies in [s+1-LEAD, s-1].  In the last
        // chunk no window is issued and the A copies stop at the last step.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        if (last_chunk) {
            constexpr int NA = kAInstr * ((LEAD - 2) < (7 - k) ? (LEAD - 2) : (7 - k > 0 ? 7 - k : 0));
            __builtin_amdgcn_s_waitcnt((NA & 15) | ((NA >> 4) << 14) | 0x70);
        } else if (k >= 1 && k <= LEAD - 1) {
            constexpr int N = kAInstr * (LEAD - 2) + kWinInstr;
            __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70);
        } else {
            constexpr int N = kAInstr * (LEAD - 2);
            __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70);
        }
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        if (s + LEAD < steps)
            issue_a(s + LEAD);
        if (k == 0 && !last_chunk)
            issue_window(chunk + 1, (chunk + 1) & 1);

        // MFMAs of step s, interleaved group by group (the wave issues in
        // order and is the only one on its SIMD) with the reads of step
        // s+1's A fragments (block i as soon as its two MFMAs have issued),
        // the blend of step s+1's B (one element pair per group) and the
        // corner reads of step s+2 (a slab's, once its blend is done).
        // Reads past the last step hit valid (stale) LDS and are never used.
        constexpr int k1 = (k + 1) % kTaps, k2 = (k + 2) % kTaps;
        const int ch1 = (k + 1 >= kTaps) ? chunk + 1 : chunk;
        const int ch2 = (k + 2 >= kTaps) ? chunk + 1 : chunk;
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
                read_corners(cr[sl], sl, k2, ch2 & 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        b[0] = make_uint4(bn[0][0], bn[0][1], bn[0][2], bn[0][3]);
        b[1] = make_uint4(bn[1][0], bn[1][1], bn[1][2], bn[1][3]);
        if (s + 1 < steps && (fbw & ((1u << k1) | (1u << (kTaps + k1))))) {
            fallback(0, k1, ch1, b[0]);
            fallback(1, k1, ch1, b[1]);
        }
    };

    for (int chunk = 0; chunk < a.nch; ++chunk) {
        step_body(chunk, std::integral_constant<int, 0>{});
        step_body(chunk, std::integral_constant<int, 1>{});
        step_body(chunk, std::integral_constant<int, 2>{});
        step_body(chunk, std::integral_constant<int, 3>{});
        step_body(chunk, std::integral_constant<int, 4>{});
        step_body(chunk, std::integral_constant<int, 5>{});
        step_body(chunk, std::integral_constant<int, 6>{});
        step_body(chunk, std::integral_constant<int, 7>{});
        step_body(chunk, std::integral_constant<int, 8>{});
    }

    // ---- epilogue: per block of 32 output channels, through LDS, + bias,
    // one rounding, 16-byte stores of 8 pixels along a tile row.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    float *slice = reinterpret_cast<float *>(smem);
    const bool vec = a.vec_out != 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                slice[(8 * (r >> 2) + 4 * half + (r & 3)) * kEpRow + (wave * 2 + s) * 32 +
                      (lane & 31)] = acc[i][s][r];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int v = tid + 256 * j;
            const int row = v >> 5, n = (v & 31) * 8;
            const int m = m0 + i * 32 + row;
            const int ho = ho0 + n / TW, wo = wo0 + n % TW;
            if (m < a.Mg && ho < a.Ho) {
                const float bv = a.has_bias ? to_f32(bias[size_t(g) * a.Mg + m]) : 0.0f;
                T *dst = out + (size_t(img) * a.Co + size_t(g) * a.Mg + m) * a.P +
                         size_t(ho) * a.Wo + wo;
                const float *sp = slice + row * kEpRow + n;
                if (vec && wo + 8 <= a.Wo) {
                    Vec16<T> o;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        o.e[e] = from_f32<T>(sp[e] + bv);
                    store16(dst, o);
                } else {
                    for (int e = 0; e < 8 && wo + e < a.Wo; ++e)
                        dst[e] = from_f32<T>(sp[e] + bv);
                }
            }
        }
        __syncthreads();
    }
}

template <typename T, int TH, int TW, int LEAD>
hipError_t window_cfg(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                      const void *xt, const void *offset, const void *mask, const void *bias,
                      void *out, hipStream_t s)
{
    WinArgs a;
    a.Mg = int(p.Mg); a.Kp = int(plan.Kp); a.Co = int(p.Co); a.P = int(p.P);
    a.Ho = int(p.Ho); a.Wo = int(p.Wo);
    a.C = int(p.C); a.H = int(p.H); a.W = int(p.W); a.Cg = int(p.Cg);
    a.nch = int(p.Cg / kCC);
    a.sh = int(p.sh); a.sw = int(p.sw); a.ph = int(p.ph); a.pw = int(p.pw);
    a.dh = int(p.dh); a.dw = int(p.dw);
    a.margin = int(plan.win_margin);
    a.WR = int(window_extent(TH, p.sh, p.kh, p.dh, plan.win_margin));
    a.WC = int(window_extent(TW, p.sw, p.kw, p.dw, plan.win_margin));
    a.tiles_y = int((p.Ho + TH - 1) / TH);
    a.tiles_x = int((p.Wo + TW - 1) / TW);
    a.tiles_m = int((p.Mg + 255) / 256);
    a.cnt = int(cnt);
    a.offC = int(2 * p.DG * p.K);
    a.mskC = int(p.DG * p.K);
    a.Cdg = int(p.Cdg);
    a.has_bias = bias != nullptr;
    a.vec_out = (p.Wo % 8 == 0) && reinterpret_cast<uintptr_t>(out) % 16 == 0;
    a.img_bytes = uint32_t(size_t(p.H) * p.W * p.C * sizeof(T));
    a.chunk_bytes = uint32_t(size_t(cnt) * a.img_bytes);
    a.a_bytes = uint32_t(size_t(p.Mg) * p.Kg * sizeof(T));     // one group's weight
    if (a.WR * a.WC > kWindowPixels || a.WC * 16 + 32 > kWinZero)
        return hipErrorInvalidValue;
    const uint64_t blocks = uint64_t(p.G) * cnt * a.tiles_y * a.tiles_x * a.tiles_m;
    if (blocks == 0)
        return hipSuccess;
    if (blocks > 0x7fffffffull)
        return hipErrorInvalidValue;
    auto kern = window_kernel<T, TH, TW, LEAD>;
    constexpr int lds = lds_total(LEAD);
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (attr != hipSuccess)
        return attr;
    hipLaunchKernelGGL(kern, dim3(uint32_t(blocks)), dim3(256), lds, s,
                       static_cast<const T *>(wpack), static_cast<const T *>(xt),
                       static_cast<const T *>(offset), static_cast<const T *>(mask),
                       static_cast<const T *>(bias), static_cast<T *>(out), a);
    return hipGetLastError();
}

template <typename T, int TH, int TW>
hipError_t window_lead(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                       const void *xt, const void *offset, const void *mask, const void *bias,
                       void *out, hipStream_t s)
{
    switch (plan.win_lead) {
    case 3:
        return window_cfg<T, TH, TW, 3>(p, plan, cnt, wpack, xt, offset, mask, bias, out, s);
    case 5:
        return window_cfg<T, TH, TW, 5>(p, plan, cnt, wpack, xt, offset, mask, bias, out, s);
    case 7:
        return window_cfg<T, TH, TW, 7>(p, plan, cnt, wpack, xt, offset, mask, bias, out, s);
    }
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t window_t(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                    const void *xt, const void *offset, const void *mask, const void *bias,
                    void *out, hipStream_t s)
{
    switch (plan.win_tile) {
    case WindowTile::H16_W16:
        return window_lead<T, 16, 16>(p, plan, cnt, wpack, xt, offset, mask, bias, out, s);
    case WindowTile::H8_W32:
        return window_lead<T, 8, 32>(p, plan, cnt, wpack, xt, offset, mask, bias, out, s);
    case WindowTile::H32_W8:
        return window_lead<T, 32, 8>(p, plan, cnt, wpack, xt, offset, mask, bias, out, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_window(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                         const void *xt, const void *offset, const void *mask, const void *bias,
                         void *out, hipStream_t stream)
{
    switch (p.dtype) {
    case MDCN_F16:
        return window_t<half_t>(p, plan, cnt, wpack, xt, offset, mask, bias, out, stream);
    case MDCN_BF16:
        return window_t<bf16_t>(p, plan, cnt, wpack, xt, offset, mask, bias, out, stream);
    case MDCN_F32:
        break;
    }
    return hipErrorInvalidValue;
}

}  // namespace mdcn
