// mfma_common.h -- pieces shared by the GEMM and the fused gather-GEMM:
// the per-dtype MFMA step on 16-byte fragments (and the E4M3 step on pairs
// of them), the swizzled 128-byte-row
// LDS tile layout, one pipeline step of MFMAs over such a tile, and the
// LDS-staged epilogue (bias in fp32, one rounding, 16-byte stores).
//
// Tile layout in LDS: row r of a tile is 128 bytes (64 f16/bf16 or 32 f32 of
// K); its 16-byte chunk c sits at r*128 + ((c ^ ((r/2) % 8)) * 16).  A 32x32
// MFMA fragment (32 consecutive rows, one chunk) then spreads each group of
// 16 lanes over 16 distinct 16-byte bank groups.
//
// Accumulator register r of lane l in a 32x32 tile holds row
// 8*(r/4) + 4*(l/32) + r%4 and column l%32.  Lane l feeds row l%32 of A and
// of B with chunk (2*kg + l/32) of k-group kg; A and B use the same lane -> k
// mapping, so the order in which the hardware walks k inside one instruction
// does not matter.
#pragma once

#include "device_common.h"

namespace mdcn {

template <typename T> struct Mma;

template <> struct Mma<half_t> {
    static __device__ __forceinline__ float16v step(const uint4 &a, const uint4 &b, float16v c)
    {
        half8 av, bv;
        __builtin_memcpy(&av, &a, 16);
        __builtin_memcpy(&bv, &b, 16);
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, c, 0, 0, 0);
    }
};

template <> struct Mma<bf16_t> {
    static __device__ __forceinline__ float16v step(const uint4 &a, const uint4 &b, float16v c)
    {
        bf16x8 av, bv;
        __builtin_memcpy(&av, &a, 16);
        __builtin_memcpy(&bv, &b, 16);
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c, 0, 0, 0);
    }
};

template <> struct Mma<float> {
    static __device__ __forceinline__ float16v step(const uint4 &a, const uint4 &b, float16v c)
    {
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
        return c;
    }
};

typedef int int8v __attribute__((ext_vector_type(8)));

// (v_mfma_f32_32x32x64_f8f6f4 through the scaled builtin with zero scale
// operands, which is the unscaled instruction; A and B bytes pair up by
// (lane, byte), so any lane -> k mapping that A and B share is valid.)

typedef __attribute__((address_space(3))) void lds_void;

// Raw buffer resource over `bytes` bytes at `base` (loads past the end read 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, int(bytes),
                                             0x00020000);
}

__device__ __forceinline__ int swz_chunk(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// fences global memory, which makes every wave wait for all of its
// outstanding global loads first; this one waits for the wave's LDS
// operations alone, so prefetched global loads stay in flight across it.
// Data that a DMA writes into LDS must be waited for (vmcnt) by the caller.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The A and B fragments of one 128-byte K step for the wave's FM x FN block
// of 32x32 tiles: 4 k-groups of 16-byte fragments, A rows from `sA` and B
// rows from `sB`.  Reading them all into registers before the next step's
// operand DMA is issued matters: an LDS read issued after an LDS-writing DMA
// is made to wait for that DMA.
template <int FM, int FN>
struct StepFrags {
    uint4 a[4][FM], b[4][FN];
};

template <int FM, int FN>
__device__ __forceinline__ void load_step_frags(StepFrags<FM, FN> &f, const char *sA,
                                                const char *sB, int lane)
{
    const char *pa = sA + (lane & 31) * 128;
    const char *pb = sB + (lane & 31) * 128;
    const int sw = (lane >> 1) & 7;   // (row / 2) % 8 of every fragment row of this lane
    const int half = lane >> 5;
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
        const int q = kg * 2 + half;
#pragma unroll
        for (int i = 0; i < FM; ++i)
            f.a[kg][i] = *reinterpret_cast<const uint4 *>(pa + i * 32 * 128 + (q ^ sw) * 16);
#pragma unroll
        for (int j = 0; j < FN; ++j)
            f.b[kg][j] = *reinterpret_cast<const uint4 *>(pb + j * 32 * 128 + (q ^ sw) * 16);
    }
}

// The A and B fragments of k-group kg alone (see load_step_frags).
template <int FM, int FN>
__device__ __forceinline__ void load_kgroup_frags(uint4 (&fa)[FM], uint4 (&fb)[FN], const char *sA,
                                                  const char *sB, int lane, int kg)
{
    const char *pa = sA + (lane & 31) * 128;
    const char *pb = sB + (lane & 31) * 128;
    const int q = kg * 2 + (lane >> 5);
    const int sw = (lane >> 1) & 7;
#pragma unroll
    for (int i = 0; i < FM; ++i)
        fa[i] = *reinterpret_cast<const uint4 *>(pa + i * 32 * 128 + (q ^ sw) * 16);
#pragma unroll
    for (int j = 0; j < FN; ++j)
        fb[j] = *reinterpret_cast<const uint4 *>(pb + j * 32 * 128 + (q ^ sw) * 16);
}

// The MFMAs of one k-group from its fragments.
template <typename T, int FM, int FN>
__device__ __forceinline__ void mfma_frags(float16v (&acc)[FM][FN], const uint4 (&fa)[FM],
                                           const uint4 (&fb)[FN])
{
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = Mma<T>::step(fa[i], fb[j], acc[i][j]);
}

// The MFMAs of k-group kg of a step.
template <typename T, int FM, int FN>
__device__ __forceinline__ void mfma_kgroup(float16v (&acc)[FM][FN], const StepFrags<FM, FN> &f,
                                            int kg)
{
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = Mma<T>::step(f.a[kg][i], f.b[kg][j], acc[i][j]);
}

template <typename T, int FM, int FN>
__device__ __forceinline__ void mfma_step_frags(float16v (&acc)[FM][FN],
                                                const StepFrags<FM, FN> &f)
{
#pragma unroll
    for (int kg = 0; kg < 4; ++kg)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = Mma<T>::step(f.a[kg][i], f.b[kg][j], acc[i][j]);
}

// fp32 operands on the bf16 matrix cores (the "split" GEMM of the backward):
// each fp32 value a is hi + mid + lo up to 2^-25 |a|, three bf16 values
// (hi = bf16(a), mid = bf16(a - hi), lo = bf16(a - hi - mid), each rounded to
// nearest even; the differences are exact in fp32), and a product a*b is
// taken as the six terms hi*hi + mid*hi + hi*mid + mid*mid + hi*lo + lo*hi
// (the dropped mid*lo + lo*mid + lo*lo are below 2^-23 |ab|).  A 16-byte
// fragment pair (4 fp32 k per lane) is three v_mfma_f32_32x32x16_bf16 on
// 8-bf16 operands whose two halves pair up by (lane, position):
// [hi | mid] x [hi | hi], [hi | mid] x [mid | mid], [hi | lo] x [lo | hi].
// The products of bf16 values are exact and the sums are fp32.  (A value
// beyond the largest bf16, about 3.39e38, or an infinity gives a NaN.)
struct f32x3_t {
    float v;
};

struct Split3 {
    uint2 hi, mid, lo;                    // 4 bf16 each, k order
};

__device__ __forceinline__ uint32_t bf16_pair_rne(float a, float b)
{
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const b2 r = __builtin_convertvector((f2){a, b}, b2);
    uint32_t o;
    __builtin_memcpy(&o, &r, 4);
    return o;
}

__device__ __forceinline__ Split3 split3(const uint4 &a)
{
    const float v[4] = {__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z),
                        __uint_as_float(a.w)};
    uint32_t h[2], m[2], l[2];
    float r[4], t[4];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        h[q] = bf16_pair_rne(v[2 * q], v[2 * q + 1]);
        r[2 * q] = v[2 * q] - __uint_as_float(h[q] << 16);
        r[2 * q + 1] = v[2 * q + 1] - __uint_as_float(h[q] & 0xffff0000u);
        m[q] = bf16_pair_rne(r[2 * q], r[2 * q + 1]);
        t[2 * q] = r[2 * q] - __uint_as_float(m[q] << 16);
        t[2 * q + 1] = r[2 * q + 1] - __uint_as_float(m[q] & 0xffff0000u);
        l[q] = bf16_pair_rne(t[2 * q], t[2 * q + 1]);
    }
    Split3 o;
    o.hi = make_uint2(h[0], h[1]);
    o.mid = make_uint2(m[0], m[1]);
    o.lo = make_uint2(l[0], l[1]);
    return o;
}

__device__ __forceinline__ float16v mfma_bf16_halves(const uint2 &a0, const uint2 &a1,
                                                     const uint2 &b0, const uint2 &b1,
                                                     float16v c)
{
    const uint4 av = make_uint4(a0.x, a0.y, a1.x, a1.y);
    const uint4 bv = make_uint4(b0.x, b0.y, b1.x, b1.y);
    return Mma<bf16_t>::step(av, bv, c);
}

// The MFMAs of one 128-byte fp32 K step on the bf16 matrix cores (see
// f32x3_t), one k-group at a time: B's parts first, then each A fragment's
// parts right before its MFMAs, so that few split registers are live.
template <int FM, int FN>
__device__ __forceinline__ void mfma_step_frags_x3(float16v (&acc)[FM][FN],
                                                   const StepFrags<FM, FN> &f)
{
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
        Split3 sb[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j)
            sb[j] = split3(f.b[kg][j]);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const Split3 sa = split3(f.a[kg][i]);
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                acc[i][j] = mfma_bf16_halves(sa.hi, sa.mid, sb[j].hi, sb[j].hi, acc[i][j]);
                acc[i][j] = mfma_bf16_halves(sa.hi, sa.mid, sb[j].mid, sb[j].mid, acc[i][j]);
                acc[i][j] = mfma_bf16_halves(sa.hi, sa.lo, sb[j].lo, sb[j].hi, acc[i][j]);
            }
        }
    }
}

// One 128-byte K step of E4M3 operands: 128 k per row, two MFMAs of 64 k
// per 32x32 tile.  Lane l of MFMA kp reads 16-byte chunks 4*kp + l/32 and
// 4*kp + 2 + l/32 of its row (the same chunks for A and B) straight into the
// two halves of one 8-register operand.
typedef int int4v __attribute__((ext_vector_type(4)));

template <int FM, int FN>
struct StepFragsE4m3 {
    int8v a[2][FM], b[2][FN];
};

__device__ __forceinline__ int8v load_pair(const char *row, int c0, int c1, int sw)
{
    const int4v lo = *reinterpret_cast<const int4v *>(row + (c0 ^ sw) * 16);
    const int4v hi = *reinterpret_cast<const int4v *>(row + (c1 ^ sw) * 16);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int FM, int FN>
__device__ __forceinline__ void load_step_frags_e4m3(StepFragsE4m3<FM, FN> &f, const char *sA,
                                                     const char *sB, int lane)
{
    const char *pa = sA + (lane & 31) * 128;
    const char *pb = sB + (lane & 31) * 128;
    const int sw = (lane >> 1) & 7;
    const int half = lane >> 5;
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
            f.a[kp][i] = load_pair(pa + i * 32 * 128, 4 * kp + half, 4 * kp + 2 + half, sw);
#pragma unroll
        for (int j = 0; j < FN; ++j)
            f.b[kp][j] = load_pair(pb + j * 32 * 128, 4 * kp + half, 4 * kp + 2 + half, sw);
    }
}

template <int FM, int FN>
__device__ __forceinline__ void mfma_step_frags_e4m3(float16v (&acc)[FM][FN],
                                                     const StepFragsE4m3<FM, FN> &f)
{
#pragma unroll
    for (int kp = 0; kp < 2; ++kp)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    f.a[kp][i], f.b[kp][j], acc[i][j], 0, 0, 0, 0, 0, 0);
}

struct EpilogueArgs {
    int g, m0, n0;            // group, first weight row and first column of the tile
    int Mg, Ncols, P, Co;
    int has_bias, vec_out;    // vec_out: P and `out` allow 16-byte stores
    const float *rscale;      // SCALED epilogues: factor of each output channel's sums
};

// Writes the wave's block of accumulators (rows wm*WTM.., columns wn*WTN..
// of the tile) to out[n][g*Mg + m][pix] for column n*P + pix, adding bias in
// fp32 (SCALED: the sums times rscale[g*Mg + m] first).  Staged through the
// wave's own slice of `smem`, which the caller must no longer need (a
// barrier before the call).
template <typename T, int WTM, int WTN, bool SCALED = false>
__device__ __forceinline__ void epilogue_store(float16v (&acc)[WTM / 32][WTN / 32], char *smem,
                                               const T *__restrict__ bias, T *__restrict__ out,
                                               const EpilogueArgs &e, int wm, int wn, int wave,
                                               int lane)
{
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int EV = 16 / sizeof(T);                 // output elements per store
    constexpr int SROW = WTN + 4;                      // slice row, floats (padded)
    float *slice = reinterpret_cast<float *>(smem) + wave * 32 * SROW;
    const bool vec_out = e.vec_out != 0;               // vectors never straddle two images
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                slice[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * SROW + j * 32 + (lane & 31)] =
                    acc[i][j][r];
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
        const int mb = e.m0 + wm * WTM + i * 32;       // first output row of the block
        const int nb = e.n0 + wn * WTN;                // first column of the wave's tile
        if (vec_out) {
#pragma unroll
            for (int it = 0; it < 32 * WTN / EV / 64; ++it) {
                const int idx = it * 64 + lane;
                const int rl = idx / (WTN / EV);
                const int cl = (idx % (WTN / EV)) * EV;
                const int m = mb + rl, n = nb + cl;
                if (m < e.Mg && n < e.Ncols) {
                    const float bv = e.has_bias ? to_f32(bias[size_t(e.g) * e.Mg + m]) : 0.0f;
                    const float rs = SCALED ? e.rscale[size_t(e.g) * e.Mg + m] : 1.0f;
                    const int img = n / e.P;
                    const int pix = n - img * e.P;
                    const float *sp = slice + rl * SROW + cl;
                    Vec16<T> o;
#pragma unroll
                    for (int t = 0; t < EV; ++t)
                        o.e[t] = from_f32<T>(SCALED ? fmaf(sp[t], rs, bv) : sp[t] + bv);
                    store16(out + (size_t(img) * e.Co + size_t(e.g) * e.Mg + m) * e.P + pix, o);
                }
            }
        } else {
            for (int idx = lane; idx < 32 * WTN; idx += 64) {
                const int rl = idx / WTN, cl = idx % WTN;
                const int m = mb + rl, n = nb + cl;
                if (m < e.Mg && n < e.Ncols) {
                    const float bv = e.has_bias ? to_f32(bias[size_t(e.g) * e.Mg + m]) : 0.0f;
                    const float rs = SCALED ? e.rscale[size_t(e.g) * e.Mg + m] : 1.0f;
                    const int img = n / e.P;
                    const int pix = n - img * e.P;
                    const float v = slice[rl * SROW + cl];
                    out[(size_t(img) * e.Co + size_t(e.g) * e.Mg + m) * e.P + pix] =
                        from_f32<T>(SCALED ? fmaf(v, rs, bv) : v + bv);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
    }
}

}  // namespace mdcn
