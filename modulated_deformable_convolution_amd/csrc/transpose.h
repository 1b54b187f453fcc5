// transpose.h -- x from [C][HW] planes to channels-last through lane swaps:
// 16-byte chunks of EV = 16/sizeof(T) elements, an EV x EV block per group
// of EV lanes.  Used by the layout kernels and by the one-launch fused
// kernel (which moves x itself before its GEMM).
#pragma once

#include "device_common.h"

namespace mdcn {

// The same transpose without LDS, one wave per unit of eight 16-byte
// chunks a lane.  A chunk holds EV = 16/sizeof(T) elements; the EV lanes
// whose lane numbers differ only in bits {0, 4, 5} (EV = 8) or {4, 5}
// (EV = 4) hold the rows of an EV x EV tile (row i = those bits in that
// order), and exchanging each of those lane bits with one bit of the
// position inside the chunk (bit 0 with the 16-bit half, by a quad swap and
// a byte permute; bits 4 and 5 with the dword index, by the row and
// half-wave swaps) leaves lane j of the group with column j.  Loads read
// channel rows (x is [C][HW] per image), stores write pixel rows.
template <int EV>
__device__ __forceinline__ uint4 transpose_lanes(uint4 v, int lane)
{
    uint32_t d[4] = {v.x, v.y, v.z, v.w};
    if constexpr (EV == 8) {
        // lane bit 0 <-> 16-bit half: an even lane keeps its low halves and
        // takes its partner's low halves as high halves, an odd lane the
        // reverse
        const uint32_t sel = (lane & 1) ? 0x03020706u : 0x05040100u;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t q = uint32_t(__builtin_amdgcn_update_dpp(
                0, int(d[k]), 0xB1 /* quad_perm 1,0,3,2 */, 0xF, 0xF, false));
            d[k] = __builtin_amdgcn_perm(q, d[k], sel);
        }
    }
    // lane bit 4 <-> dword bit 0 (odd rows of 16 lanes of the first operand
    // swapped with even rows of the second)
#pragma unroll
    for (int k = 0; k < 4; k += 2) {
        const auto r = __builtin_amdgcn_permlane16_swap(d[k], d[k + 1], false, false);
        d[k] = r[0];
        d[k + 1] = r[1];
    }
    // lane bit 5 <-> dword bit 1 (upper half-wave of the first operand
    // swapped with the lower half-wave of the second)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const auto r = __builtin_amdgcn_permlane32_swap(d[k], d[k + 2], false, false);
        d[k] = r[0];
        d[k + 2] = r[1];
    }
    return make_uint4(d[0], d[1], d[2], d[3]);
}

// 8-channel blocks (16-bit elements): unit u (one wave) moves one block x
// 512 pixels.  Chunk t of lane group g holds the block's 8 channel rows at
// pixels 512*pc + 8*(8*t + g) .. +7, so a load instruction reads 8 whole
// 128-byte lines of x and, after the transpose, a store instruction writes
// 1 KiB of contiguous block plane.  Units are ordered (image, block, pixel
// chunk).  Requires C and HW to be multiples of 8 and 16-byte aligned x
// and xt.
template <typename T>
__device__ __forceinline__ void transpose_blocks_wave(const T *__restrict__ x,
                                                      T *__restrict__ xt, int C, int HW,
                                                      uint32_t u)
{
    static_assert(sizeof(T) == 2, "8-channel blocks of 16 bytes take 16-bit elements");
    constexpr int R = 8;                        // chunks per lane
    const int lane = int(threadIdx.x) & 63;
    const int i = (lane & 1) | ((lane >> 3) & 6);   // row (load) / column (store) in the group
    const int g = (lane >> 1) & 7;                  // lane group
    const uint32_t npc = uint32_t(HW + 511) / 512u, cbs = uint32_t(C) / 8u;
    const uint32_t pc = u % npc, r = u / npc;
    const uint32_t cb = r % cbs, n = r / cbs;
    const T *src = x + (size_t(n) * C + 8 * cb + i) * size_t(HW);
    T *dst = xt + (size_t(n) * cbs + cb) * size_t(HW) * 8;
    uint4 v[R];
#pragma unroll
    for (int t = 0; t < R; ++t) {
        const int po = int(pc) * 512 + (t * 8 + g) * 8;
        v[t] = make_uint4(0u, 0u, 0u, 0u);
        if (po < HW)
            v[t] = *reinterpret_cast<const uint4 *>(src + po);
    }
#pragma unroll
    for (int t = 0; t < R; ++t) {
        const int po = int(pc) * 512 + (t * 8 + g) * 8;
        const uint4 w = transpose_lanes<8>(v[t], lane);
        if (po < HW)
            *reinterpret_cast<uint4 *>(dst + size_t(po + i) * 8) = w;
    }
}

// NHWC: 256 threads (4 waves) per tile of 64 channels x 64 pixels, tiles
// ordered (image, pixel chunk, channel chunk).  Each wave loads Q/4 chunk
// rows (EV channels x 64 pixels: EV whole lines of x per instruction),
// transposes them across lanes, and puts each pixel's 16-byte chunk into
// LDS (row = pixel, Q = 64/EV chunks of 16 bytes, XOR-swizzled so that
// neither side conflicts); after a barrier each wave stores 64/Q pixels x
// 64 channels per instruction (contiguous 16*Q bytes per pixel).  lds holds
// 64*Q chunks.  Requires C and HW to be multiples of EV and 16-byte aligned
// x and xt.  t is the thread's index among the 256.
template <typename T>
struct NhwcTile {
    static constexpr int EV = 16 / int(sizeof(T));
    static constexpr int Q = 64 / EV;           // chunks per pixel row of the tile
    static constexpr int PW = Q / 4;            // chunk rows per wave
    uint32_t n;
    int p0, c0;
    uint4 v[PW];

    __device__ __forceinline__ static int swz(int pl)
    {
        return ((pl / EV) ^ (EV == 8 ? pl : 0)) & (Q - 1);
    }
    __device__ __forceinline__ static int row_of(int lane)
    {
        return EV == 8 ? ((lane & 1) | ((lane >> 3) & 6)) : ((lane >> 4) & 3);
    }
    __device__ __forceinline__ static int group_of(int lane)
    {
        return EV == 8 ? ((lane >> 1) & 7) : (lane & 15);
    }
    // the tile's loads
    __device__ __forceinline__ void load(const T *__restrict__ x, int C, int HW, uint32_t tile, int t)
    {
        const int lane = t & 63, wave = t >> 6;
        const uint32_t ncc = uint32_t(C + 63) / 64u, npc = uint32_t(HW + 63) / 64u;
        const uint32_t cc = tile % ncc, r = tile / ncc;
        const uint32_t pc = r % npc;
        n = r / npc;
        p0 = int(pc) * 64;
        c0 = int(cc) * 64;
        const int po = p0 + EV * group_of(lane);    // first pixel of the lane group
#pragma unroll
        for (int k = 0; k < PW; ++k) {
            const int c = c0 + EV * (wave * PW + k);
            v[k] = make_uint4(0u, 0u, 0u, 0u);
            if (po < HW && c < C)
                v[k] = *reinterpret_cast<const uint4 *>(
                    x + (size_t(n) * C + c + row_of(lane)) * size_t(HW) + po);
        }
    }
    // the transposed chunks into LDS (a barrier must follow before take)
    __device__ __forceinline__ void put(uint4 *lds, int t) const
    {
        const int lane = t & 63, wave = t >> 6;
        const int pl = EV * group_of(lane) + row_of(lane);   // the lane's pixel after the transpose
#pragma unroll
        for (int k = 0; k < PW; ++k) {
            const int o = wave * PW + k;
            lds[pl * Q + (o ^ swz(pl))] = transpose_lanes<EV>(v[k], lane);
        }
    }
    // the pixel rows from LDS to xt; store(chunk, element offset) writes one
    // 16-byte chunk
    template <typename Store>
    __device__ __forceinline__ void take(const uint4 *lds, int C, int HW, int t, Store store) const
    {
        const int lane = t & 63, wave = t >> 6;
#pragma unroll
        for (int k = 0; k < PW; ++k) {
            const int pl = (wave * PW + k) * (64 / Q) + lane / Q;
            const int o = lane % Q;
            const int p = p0 + pl, c = c0 + EV * o;
            if (p < HW && c < C)
                store(lds[pl * Q + (o ^ swz(pl))], (size_t(n) * HW + p) * size_t(C) + c);
        }
    }
};

// The same tile order and interface for any C and HW, one element at a
// time: 16 elements a thread, LDS as 64 channel rows of 65 elements (the odd
// pitch keeps both sides free of bank conflicts); take's store gets one
// element and its offset.
template <typename T>
struct NhwcTileScalar {
    static constexpr int kLdsBytes = 64 * 65 * int(sizeof(T));
    uint32_t n;
    int p0, c0;
    T v[16];

    __device__ __forceinline__ void load(const T *__restrict__ x, int C, int HW, uint32_t tile, int t)
    {
        const uint32_t ncc = uint32_t(C + 63) / 64u, npc = uint32_t(HW + 63) / 64u;
        const uint32_t cc = tile % ncc, r = tile / ncc;
        const uint32_t pc = r % npc;
        n = r / npc;
        p0 = int(pc) * 64;
        c0 = int(cc) * 64;
        const int p = p0 + (t & 63);
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int c = c0 + (t >> 6) + 4 * k;
            v[k] = (p < HW && c < C) ? x[(size_t(n) * C + c) * size_t(HW) + p] : T(0);
        }
    }
    __device__ __forceinline__ void put(T *lds, int t) const
    {
#pragma unroll
        for (int k = 0; k < 16; ++k)
            lds[((t >> 6) + 4 * k) * 65 + (t & 63)] = v[k];
    }
    template <typename Store>
    __device__ __forceinline__ void take(const T *lds, int C, int HW, int t, Store store) const
    {
        const int c = c0 + (t & 63);
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int pl = (t >> 6) + 4 * k;
            const int p = p0 + pl;
            if (p < HW && c < C)
                store(lds[(t & 63) * 65 + pl], (size_t(n) * HW + p) * size_t(C) + c);
        }
    }
};

// NHWC tiles of cnt images.
__host__ __device__ __forceinline__ uint32_t nhwc_tiles(int C, int HW, int cnt)
{
    return uint32_t(cnt) * uint32_t((HW + 63) / 64) * uint32_t((C + 63) / 64);
}

}  // namespace mdcn
