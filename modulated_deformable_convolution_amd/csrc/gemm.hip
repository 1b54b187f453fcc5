// gemm.hip -- grouped GEMM of the packed weight with the deformable columns on
// CDNA4 matrix cores, bias add and output cast fused into the epilogue
// [plugin guide §五 step 2: one GEMM per group with m = Co/group,
// n = Ho*Wo, k = C/group*kh*kw; §五 step 3: bias broadcast per output channel].
//
//   out[n][g*Mg + m][pix] = sum_kk A[g][m][kk] * B[g][n*P + pix][kk] + bias[g*Mg + m]
//
// Both operands are K-contiguous ("NT"), the per-lane layout of the MFMA
// fragments: lane l of a 32x32 MFMA holds 16 contiguous bytes of row (l % 32)
// of A and of B.  A and B use the same lane -> k mapping, so the order in which
// the hardware walks k inside one instruction does not matter.  The images of
// one chunk are concatenated along n (columns n*P + pix).
//
// Data movement: each pipeline step moves STEP (= 128) bytes of K of every
// tile row -- one cache line -- straight from global memory into LDS with
// buffer_load_dwordx4 ... lds (no register staging).  Such a wave instruction
// writes 1 KB of LDS contiguously (lane i at +16*i) and here fetches 8 whole
// rows: 8 lanes per row, so every request is a full, coalesced line.  In LDS
// a row is 128 bytes with its 16-byte chunk index XORed with (row / 2) % 8;
// the MFMA fragment read of 32 consecutive rows at one chunk then spreads
// each group of 16 lanes over 16 distinct 16-byte bank groups of a 256-byte
// LDS line.  Rows past the
// matrix edge are clamped to a valid row; they only feed accumulator rows or
// columns that the epilogue never stores.  Two LDS stages: the loads of step
// s+1 are in flight while the MFMAs of step s run (more stages cost
// occupancy, which matters more here).
//
//   f16 / bf16: one v_mfma_f32_32x32x16_{f16,bf16} per 16-byte fragment pair;
//   f32:        four v_mfma_f32_32x32x2_f32 per 16-byte fragment pair.
#include "device_common.h"
#include "launch.h"

namespace mdcn {

namespace {

struct GemmArgs {
    int Mg, Ncols, Kp, P, Co;
    int tiles_m, tiles_n;
    int has_bias;
    int vec_out;        // 16-byte output stores allowed (P and `out` aligned to them)
};

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

typedef __attribute__((address_space(3))) void lds_void;

// Raw buffer resource over `bytes` bytes at `base` (loads past the end read 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, int(bytes),
                                             0x00020000);
}

// One pipeline step's operand loads of one wave: IPW instructions of 8 tile
// rows each (A rows first, then B rows).  Lane i of an instruction fetches
// chunk (i%8) ^ ((row/2)%8) of row r0 + i/8, which lands in LDS slot r0*8 + i.
template <int BM, int BN, int NW, int STEP>
__device__ __forceinline__ void issue_step(char *stage_base, __amdgpu_buffer_rsrc_t ra,
                                           __amdgpu_buffer_rsrc_t rb, const uint32_t *voff,
                                           int wave, int step)
{
    constexpr int IPW = (BM + BN) / 8 / NW;
    const int soff = step * STEP;
#pragma unroll
    for (int t = 0; t < IPW; ++t) {
        const int row0 = (wave * IPW + t) * 8;             // wave-uniform
        if (row0 < BM)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(stage_base + row0 * STEP),
                                                     16, voff[t], soff, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(stage_base + row0 * STEP),
                                                     16, voff[t], soff, 0, 0);
    }
}

template <typename T, int BM, int BN, int WAVES_M, int WAVES_N, int STEP>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64) void gemm_bias_kernel(
    const T *__restrict__ A, const T *__restrict__ B, const T *__restrict__ bias,
    T *__restrict__ out, GemmArgs a)
{
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int NCH = STEP / 16;                       // 16-byte chunks per row per step
    constexpr int STAGE_BYTES = (BM + BN) * STEP;
    constexpr int IPW = (BM + BN) / 8 / NW;              // load instructions per wave per step
    static_assert(STEP == 128, "a tile row holds one 128-byte line per step");
    static_assert(BM % 32 == 0 && BN % 32 == 0 && (BM + BN) / 8 % NW == 0,
                  "tile rows must split evenly into 8-row load instructions per wave");
    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE_BYTES];

    uint32_t bid = xcd_swizzle(blockIdx.x, gridDim.x);
    const int mt = int(bid % uint32_t(a.tiles_m));
    bid /= uint32_t(a.tiles_m);
    const int nt = int(bid % uint32_t(a.tiles_n));
    const int g = int(bid / uint32_t(a.tiles_n));
    const int m0 = mt * BM, n0 = nt * BN;

    const int lane = int(threadIdx.x) & 63;
    // wave index as a scalar: LDS destinations of the loads must be wave-uniform
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);

    const uint32_t row_bytes = uint32_t(a.Kp) * uint32_t(sizeof(T));
    const char *Ag = reinterpret_cast<const char *>(A) + size_t(g) * a.Mg * row_bytes;
    const char *Bg = reinterpret_cast<const char *>(B) + size_t(g) * a.Ncols * row_bytes;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ag, uint32_t(a.Mg) * row_bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bg, uint32_t(a.Ncols) * row_bytes);

    // Global byte offset of what this lane fetches in each of its wave's load
    // instructions (rows past the edge clamped); the same for every step.
    uint32_t voff[IPW];
#pragma unroll
    for (int t = 0; t < IPW; ++t) {
        const int row = (wave * IPW + t) * 8 + (lane >> 3);     // tile row (A rows first)
        const int chunk = (lane & 7) ^ ((row >> 1) & 7);
        if (row < BM)
            voff[t] = uint32_t(min(m0 + row, a.Mg - 1)) * row_bytes + chunk * 16;
        else
            voff[t] = uint32_t(min(n0 + row - BM, a.Ncols - 1)) * row_bytes + chunk * 16;
    }

    const int wm = wave % WAVES_M, wn = wave / WAVES_M;
    float16v acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.0f;

    const int steps = int(row_bytes / STEP);
    issue_step<BM, BN, NW, STEP>(smem, ra, rb, voff, wave, 0);
    for (int st = 0; st < steps; ++st) {
        const int stage = st & 1;
        __builtin_amdgcn_s_waitcnt(0);   // this thread's loads of step st have landed
        __syncthreads();                 // ... and everyone's; stage^1 is free again
        if (st + 1 < steps)
            issue_step<BM, BN, NW, STEP>(smem + (stage ^ 1) * STAGE_BYTES, ra, rb, voff, wave,
                                         st + 1);
        const char *sA = smem + stage * STAGE_BYTES + (wm * WTM + (lane & 31)) * STEP;
        const char *sB = smem + stage * STAGE_BYTES + (BM + wn * WTN + (lane & 31)) * STEP;
        const int sw = (lane >> 1) & 7;   // (row / 2) % 8 of every fragment row of this lane
        const int half = lane >> 5;
#pragma unroll
        for (int kg = 0; kg < NCH / 2; ++kg) {
            const int q = kg * 2 + half;
            uint4 af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const uint4 *>(sA + i * 32 * STEP + (q ^ sw) * 16);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[j] = *reinterpret_cast<const uint4 *>(sB + j * 32 * STEP + (q ^ sw) * 16);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = Mma<T>::step(af[i], bf[j], acc[i][j]);
        }
    }

    // Epilogue, through LDS so that each lane stores 16 contiguous bytes of
    // an output row.  Per 32-row block of the wave's tile: the fp32
    // accumulators go to the wave's own LDS slice (row-major), then come back
    // as vectors along the pixel axis; bias is added in fp32 and the sum
    // rounded once.  Accumulator register r of lane l in a 32x32 tile holds
    // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
    constexpr int EV = 16 / sizeof(T);                 // output elements per store
    constexpr int SROW = WTN + 4;                      // slice row, floats (padded)
    static_assert(NW * 32 * SROW * 4 <= 2 * STAGE_BYTES, "epilogue slices must fit in LDS");
    __syncthreads();                                   // operand stages no longer needed
    float *slice = reinterpret_cast<float *>(smem) + wave * 32 * SROW;
    const bool vec_out = a.vec_out != 0;               // vectors never straddle two images
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
        const int mb = m0 + wm * WTM + i * 32;         // first output row of the block
        const int nb = n0 + wn * WTN;                  // first column of the wave's tile
        if (vec_out) {
#pragma unroll
            for (int it = 0; it < 32 * WTN / EV / 64; ++it) {
                const int e = it * 64 + lane;
                const int rl = e / (WTN / EV);
                const int cl = (e % (WTN / EV)) * EV;
                const int m = mb + rl, n = nb + cl;
                if (m < a.Mg && n < a.Ncols) {
                    const float bv = a.has_bias ? to_f32(bias[size_t(g) * a.Mg + m]) : 0.0f;
                    const int img = n / a.P;
                    const int pix = n - img * a.P;
                    const float *sp = slice + rl * SROW + cl;
                    Vec16<T> o;
#pragma unroll
                    for (int t = 0; t < EV; ++t)
                        o.e[t] = from_f32<T>(sp[t] + bv);
                    store16(out + (size_t(img) * a.Co + size_t(g) * a.Mg + m) * a.P + pix, o);
                }
            }
        } else {
            for (int e = lane; e < 32 * WTN; e += 64) {
                const int rl = e / WTN, cl = e % WTN;
                const int m = mb + rl, n = nb + cl;
                if (m < a.Mg && n < a.Ncols) {
                    const float bv = a.has_bias ? to_f32(bias[size_t(g) * a.Mg + m]) : 0.0f;
                    const int img = n / a.P;
                    const int pix = n - img * a.P;
                    out[(size_t(img) * a.Co + size_t(g) * a.Mg + m) * a.P + pix] =
                        from_f32<T>(slice[rl * SROW + cl] + bv);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
    }
}

template <typename T, int BM, int BN, int WM, int WN>
hipError_t gemm_cfg(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                    const void *col, const void *bias, void *out, hipStream_t s)
{
    constexpr int STEP = 128;
    GemmArgs a;
    a.Mg = int(p.Mg);
    a.Ncols = int(cnt * p.P);
    a.Kp = int(plan.Kp);
    a.P = int(p.P);
    a.Co = int(p.Co);
    a.tiles_m = int((p.Mg + BM - 1) / BM);
    a.tiles_n = int((a.Ncols + BN - 1) / BN);
    a.has_bias = bias != nullptr;
    a.vec_out = (p.P % (16 / int(sizeof(T))) == 0) && reinterpret_cast<uintptr_t>(out) % 16 == 0;
    const uint64_t blocks = uint64_t(p.G) * a.tiles_m * a.tiles_n;
    hipLaunchKernelGGL((gemm_bias_kernel<T, BM, BN, WM, WN, STEP>), dim3(uint32_t(blocks)),
                       dim3(WM * WN * 64), 0, s, static_cast<const T *>(wpack),
                       static_cast<const T *>(col), static_cast<const T *>(bias),
                       static_cast<T *>(out), a);
    return hipGetLastError();
}

template <typename T>
hipError_t gemm_t(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                  const void *col, const void *bias, void *out, hipStream_t s)
{
    switch (plan.gemm_tile) {
    case GemmTile::M256_N256_W2x4:
        return gemm_cfg<T, 256, 256, 2, 4>(p, plan, cnt, wpack, col, bias, out, s);
    case GemmTile::M256_N128_W4x2:
        return gemm_cfg<T, 256, 128, 4, 2>(p, plan, cnt, wpack, col, bias, out, s);
    case GemmTile::M128_N256_W2x4:
        return gemm_cfg<T, 128, 256, 2, 4>(p, plan, cnt, wpack, col, bias, out, s);
    case GemmTile::M128_N128_W2x2:
        return gemm_cfg<T, 128, 128, 2, 2>(p, plan, cnt, wpack, col, bias, out, s);
    case GemmTile::M128_N64_W2x2:
        return gemm_cfg<T, 128, 64, 2, 2>(p, plan, cnt, wpack, col, bias, out, s);
    case GemmTile::M64_N128_W2x2:
        return gemm_cfg<T, 64, 128, 2, 2>(p, plan, cnt, wpack, col, bias, out, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                       const void *col, const void *bias, void *out, hipStream_t stream)
{
    switch (p.dtype) {
    case MDCN_F32: return gemm_t<float>(p, plan, cnt, wpack, col, bias, out, stream);
    case MDCN_F16: return gemm_t<half_t>(p, plan, cnt, wpack, col, bias, out, stream);
    case MDCN_BF16: return gemm_t<bf16_t>(p, plan, cnt, wpack, col, bias, out, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mdcn
