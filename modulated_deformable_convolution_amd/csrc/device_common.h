// device_common.h -- element types and small device helpers shared by the
// HIP kernels of this library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace mdcn {

typedef _Float16 half_t;
typedef __bf16 bf16_t;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));

// Conversions.  Narrowing conversions round to nearest even.
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(half_t v) { return (float)v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ half_t from_f32<half_t>(float v) { return (half_t)v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return (bf16_t)v; }

// OCP FP8 E4M3 numbers (sign, 4 exponent bits with bias 7, 3 mantissa bits;
// largest finite value 448; S.1111.111 is NaN), one byte each.  gfx950's
// v_cvt_pk_fp8_f32 writes this format and rounds to nearest even; it turns
// magnitudes above 464 into NaN, so values are saturated to +-448 first
// (NaN stays NaN: the comparison is false for it).
typedef uint8_t e4m3_t;

__device__ __forceinline__ float sat_e4m3(float v)
{
    return fabsf(v) > 448.0f ? copysignf(448.0f, v) : v;
}

// Four values -> four E4M3 bytes (a in the lowest byte).
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(a), sat_e4m3(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(c), sat_e4m3(d), w, true);
    return uint32_t(w);
}

// The same without the saturation, for values already within +-448 (or NaN).
__device__ __forceinline__ uint32_t pack4_e4m3_unsat(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return uint32_t(w);
}

__device__ __forceinline__ e4m3_t to_e4m3(float v)
{
    return e4m3_t(__builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(v), 0.0f, 0, false) & 0xff);
}

// 16 bytes of T: 4 floats or 8 halves / bf16s.
template <typename T> struct Vec16 {
    static constexpr int N = 16 / sizeof(T);
    union {
        uint4 raw;
        T e[N];
    };
};

template <typename T>
__device__ __forceinline__ Vec16<T> load16(const T *p)
{
    Vec16<T> v;
    v.raw = *reinterpret_cast<const uint4 *>(p);
    return v;
}

template <typename T>
__device__ __forceinline__ void store16(T *p, const Vec16<T> &v)
{
    *reinterpret_cast<uint4 *>(p) = v.raw;
}

// Sampling geometry of one (offset group, tap, output pixel): the four
// bilinear corners as element offsets of (row * W + col) within the image,
// and their weights with the modulation mask folded in.  A corner that is
// off the image gets weight 0 and offset 0 (a safe address), so reading it
// and adding 0 * value is replaced by skipping it (see `valid`).
struct Taps {
    int idx[4];
    float wt[4];
    bool valid[4];
};

// h = anchor_h + off_h, w = anchor_w + off_w (anchor_* are exact integers).
// The integer parts are anchor + floor(offset) and the fractions are
// offset - floor(offset), so no rounding of the sum enters the weights.
// Corners off the image read 0 (zero-padded bilinear interpolation); an
// offset that is not finite, or so large that the sample is certainly off
// the image, leaves every corner invalid.
__device__ __forceinline__ Taps make_taps(int anchor_h, int anchor_w, float off_h, float off_w,
                                          float m, int H, int W)
{
    Taps t;
    const float lim = 33554432.0f;  // 2^25: beyond it the sample is off any valid image
    bool ok = (fabsf(off_h) <= lim) && (fabsf(off_w) <= lim);
    float fh = ok ? floorf(off_h) : 0.0f;
    float fw = ok ? floorf(off_w) : 0.0f;
    float ly = ok ? off_h - fh : 0.0f;
    float lx = ok ? off_w - fw : 0.0f;
    int h0 = anchor_h + (int)fh;
    int w0 = anchor_w + (int)fw;
    bool r0 = ok && (unsigned)h0 < (unsigned)H;
    bool r1 = ok && (unsigned)(h0 + 1) < (unsigned)H;
    bool c0 = (unsigned)w0 < (unsigned)W;
    bool c1 = (unsigned)(w0 + 1) < (unsigned)W;
    float hy = 1.0f - ly, hx = 1.0f - lx;
    t.valid[0] = r0 && c0;
    t.valid[1] = r0 && c1;
    t.valid[2] = r1 && c0;
    t.valid[3] = r1 && c1;
    t.wt[0] = t.valid[0] ? hy * hx * m : 0.0f;
    t.wt[1] = t.valid[1] ? hy * lx * m : 0.0f;
    t.wt[2] = t.valid[2] ? ly * hx * m : 0.0f;
    t.wt[3] = t.valid[3] ? ly * lx * m : 0.0f;
    t.idx[0] = t.valid[0] ? h0 * W + w0 : 0;
    t.idx[1] = t.valid[1] ? h0 * W + w0 + 1 : 0;
    t.idx[2] = t.valid[2] ? (h0 + 1) * W + w0 : 0;
    t.idx[3] = t.valid[3] ? (h0 + 1) * W + w0 + 1 : 0;
    return t;
}

// Workgroup index remapped so that consecutive logical tiles land on the same
// XCD (the hardware deals workgroups round-robin over the 8 XCDs, each with
// its own L2).  Identity when the grid is not a multiple of 8.
__device__ __forceinline__ uint32_t xcd_swizzle(uint32_t bid, uint32_t nblocks)
{
    if (nblocks % 8u != 0u)
        return bid;
    return (bid % 8u) * (nblocks / 8u) + bid / 8u;
}

}  // namespace mdcn
