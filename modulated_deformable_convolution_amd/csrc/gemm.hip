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
// occupancy, which matters more here).  Each step's fragments are read into
// registers before the next step's DMA is issued, so the DMA overlaps the
// MFMAs instead of delaying the reads.
//
//   f16 / bf16: one v_mfma_f32_32x32x16_{f16,bf16} per 16-byte fragment pair;
//   f32:        four v_mfma_f32_32x32x2_f32 per 16-byte fragment pair;
//   f32, split (the backward's GEMMs): each fp32 operand as three bf16
//               parts, three v_mfma_f32_32x32x16_bf16 per fragment pair
//               (f32x3_t in mfma_common.h);
//   FP8 path:   E4M3 operands (the quantized weight and columns), one
//               v_mfma_f32_32x32x64_f8f6f4 per two 16-byte fragment pairs,
//               and the epilogue multiplies each output channel's sums by its
//               weight row's scale 2^-e before the bias.
#include <type_traits>

#include "launch.h"
#include "mfma_common.h"

namespace mdcn {

namespace {

struct GemmArgs {
    int Mg, Ncols, Kp, P, Co;
    int tiles_m, tiles_n;
    int has_bias;
    int vec_out;        // 16-byte output stores allowed (P and `out` aligned to them)
    uint32_t kb;        // bytes of K per row (a multiple of STEP)
    uint32_t sa, sb;    // bytes between consecutive rows of A, of B
    uint64_t ga, gb;    // bytes between the groups' blocks of A, of B
};

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

// OP: the operand element type, T (or E4M3 bytes for the FP8 path, whose
// rscale holds each weight row's scale); T: bias and output.
template <typename T, typename OP, int BM, int BN, int WAVES_M, int WAVES_N, int STEP>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64) void gemm_bias_kernel(
    const OP *__restrict__ A, const OP *__restrict__ B, const T *__restrict__ bias,
    const float *__restrict__ rscale, T *__restrict__ out, GemmArgs a)
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

    const char *Ag = reinterpret_cast<const char *>(A) + size_t(g) * a.ga;
    const char *Bg = reinterpret_cast<const char *>(B) + size_t(g) * a.gb;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ag, uint32_t(a.Mg - 1) * a.sa + a.kb);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bg, uint32_t(a.Ncols - 1) * a.sb + a.kb);

    // Global byte offset of what this lane fetches in each of its wave's load
    // instructions (rows past the edge clamped); the same for every step.
    uint32_t voff[IPW];
#pragma unroll
    for (int t = 0; t < IPW; ++t) {
        const int row = (wave * IPW + t) * 8 + (lane >> 3);     // tile row (A rows first)
        const int chunk = (lane & 7) ^ ((row >> 1) & 7);
        if (row < BM)
            voff[t] = uint32_t(min(m0 + row, a.Mg - 1)) * a.sa + chunk * 16;
        else
            voff[t] = uint32_t(min(n0 + row - BM, a.Ncols - 1)) * a.sb + chunk * 16;
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

    const int steps = int(a.kb / STEP);
    issue_step<BM, BN, NW, STEP>(smem, ra, rb, voff, wave, 0);
    for (int st = 0; st < steps; ++st) {
        const int stage = st & 1;
        __builtin_amdgcn_s_waitcnt(0);   // this thread's loads of step st have landed
        __syncthreads();                 // ... and everyone's; stage^1 is free again
        // all of step st's fragments, before the DMA
        const char *sa = smem + stage * STAGE_BYTES + wm * WTM * STEP;
        const char *sb = smem + stage * STAGE_BYTES + (BM + wn * WTN) * STEP;
        if constexpr (sizeof(OP) == 1) {
            StepFragsE4m3<FM, FN> f;
            load_step_frags_e4m3<FM, FN>(f, sa, sb, lane);
            if (st + 1 < steps)
                issue_step<BM, BN, NW, STEP>(smem + (stage ^ 1) * STAGE_BYTES, ra, rb, voff,
                                             wave, st + 1);
            mfma_step_frags_e4m3<FM, FN>(acc, f);
        } else {
            StepFrags<FM, FN> f;
            load_step_frags<FM, FN>(f, sa, sb, lane);
            if (st + 1 < steps)
                issue_step<BM, BN, NW, STEP>(smem + (stage ^ 1) * STAGE_BYTES, ra, rb, voff,
                                             wave, st + 1);
            if constexpr (std::is_same<OP, f32x3_t>::value)
                mfma_step_frags_x3<FM, FN>(acc, f);
            else
                mfma_step_frags<T, FM, FN>(acc, f);
        }
    }

    // Epilogue through LDS: bias in fp32, one rounding, 16-byte stores.
    static_assert(NW * 32 * (WTN + 4) * 4 <= 2 * STAGE_BYTES, "epilogue slices must fit in LDS");
    __syncthreads();                                   // operand stages no longer needed
    const EpilogueArgs e{g, m0, n0, a.Mg, a.Ncols, a.P, a.Co, a.has_bias, a.vec_out, rscale};
    epilogue_store<T, WTM, WTN, (sizeof(OP) == 1)>(acc, smem, bias, out, e, wm, wn, wave, lane);
}

template <typename T, typename OP, int BM, int BN, int WM, int WN>
hipError_t gemm_cfg(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                    const void *col, const void *bias, const float *rscale, void *out,
                    const GemmStrides *st, hipStream_t s)
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
    // rows of Kp elements, one block of rows per group, unless given
    const uint32_t row_bytes = uint32_t(plan.Kp) * uint32_t(sizeof(OP));
    a.kb = st ? st->kb : row_bytes;
    a.sa = st ? st->sa : row_bytes;
    a.sb = st ? st->sb : row_bytes;
    a.ga = st ? st->ga : uint64_t(a.Mg) * row_bytes;
    a.gb = st ? st->gb : uint64_t(a.Ncols) * row_bytes;
    if (a.kb % STEP != 0 || a.kb == 0)
        return hipErrorInvalidValue;
    const uint64_t blocks = uint64_t(p.G) * a.tiles_m * a.tiles_n;
    hipLaunchKernelGGL((gemm_bias_kernel<T, OP, BM, BN, WM, WN, STEP>), dim3(uint32_t(blocks)),
                       dim3(WM * WN * 64), 0, s, static_cast<const OP *>(wpack),
                       static_cast<const OP *>(col), static_cast<const T *>(bias), rscale,
                       static_cast<T *>(out), a);
    return hipGetLastError();
}

template <typename T, typename OP>
hipError_t gemm_t(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                  const void *col, const void *bias, const float *rs, void *out, hipStream_t s,
                  const GemmStrides *st = nullptr)
{
    switch (plan.gemm_tile) {
    case GemmTile::M256_N256_W2x4:
        return gemm_cfg<T, OP, 256, 256, 2, 4>(p, plan, cnt, wpack, col, bias, rs, out, st, s);
    case GemmTile::M256_N128_W4x2:
        return gemm_cfg<T, OP, 256, 128, 4, 2>(p, plan, cnt, wpack, col, bias, rs, out, st, s);
    case GemmTile::M128_N256_W2x4:
        return gemm_cfg<T, OP, 128, 256, 2, 4>(p, plan, cnt, wpack, col, bias, rs, out, st, s);
    case GemmTile::M128_N128_W2x2:
        return gemm_cfg<T, OP, 128, 128, 2, 2>(p, plan, cnt, wpack, col, bias, rs, out, st, s);
    case GemmTile::M128_N64_W2x2:
        return gemm_cfg<T, OP, 128, 64, 2, 2>(p, plan, cnt, wpack, col, bias, rs, out, st, s);
    case GemmTile::M64_N128_W2x2:
        return gemm_cfg<T, OP, 64, 128, 2, 2>(p, plan, cnt, wpack, col, bias, rs, out, st, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_strided(const Problem &p, const Plan &plan, const void *a, const void *b,
                               void *out, const GemmStrides &st, hipStream_t stream)
{
    if (p.dtype != MDCN_F32)
        return hipErrorInvalidValue;
    return gemm_t<float, f32x3_t>(p, plan, 1, a, b, nullptr, nullptr, out, stream, &st);
}

hipError_t launch_gemm_f32_split(const Problem &p, const Plan &plan, const void *a,
                                 const void *b, void *out, hipStream_t stream)
{
    if (p.dtype != MDCN_F32)
        return hipErrorInvalidValue;
    return gemm_t<float, f32x3_t>(p, plan, 1, a, b, nullptr, nullptr, out, stream);
}

hipError_t launch_gemm(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                       const void *col, const void *bias, const float *wscale, void *out,
                       hipStream_t stream)
{
    if (plan.path == Path::GatherGemmFp8) {
        switch (p.dtype) {
        case MDCN_F32:
            return gemm_t<float, e4m3_t>(p, plan, cnt, wpack, col, bias, wscale, out, stream);
        case MDCN_F16:
            return gemm_t<half_t, e4m3_t>(p, plan, cnt, wpack, col, bias, wscale, out, stream);
        case MDCN_BF16:
            return gemm_t<bf16_t, e4m3_t>(p, plan, cnt, wpack, col, bias, wscale, out, stream);
        }
        return hipErrorInvalidValue;
    }
    switch (p.dtype) {
    case MDCN_F32: return gemm_t<float, float>(p, plan, cnt, wpack, col, bias, nullptr, out, stream);
    case MDCN_F16:
        return gemm_t<half_t, half_t>(p, plan, cnt, wpack, col, bias, nullptr, out, stream);
    case MDCN_BF16:
        return gemm_t<bf16_t, bf16_t>(p, plan, cnt, wpack, col, bias, nullptr, out, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mdcn
