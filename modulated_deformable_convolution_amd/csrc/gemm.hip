// gemm.hip -- grouped GEMM of the packed weight with the deformable columns on
// CDNA4 matrix cores, bias add and output cast fused into the epilogue
// [plugin guide §五 step 2: one GEMM per group with m = Co/group,
// n = Ho*Wo, k = C/group*kh*kw; §五 step 3: bias broadcast per output channel].
//
//   out[n][g*Mg + m][pix] = sum_kk A[g][m][kk] * B[g][n*P + pix][kk] + bias[g*Mg + m]
//
// Both operands are K-contiguous ("NT"), which is the per-lane layout of the
// MFMA fragments: lane l of a 32x32 MFMA holds 16 contiguous bytes of row
// (l % 32) of A and of B.  A and B use the same lane -> k mapping, so the
// order in which the hardware walks k inside one instruction does not matter.
// The images of one chunk are concatenated along n (columns n*P + pix), so
// ragged per-image pixel counts never leave a tile half empty.
//
// Tiling: BM x BN per workgroup, WAVES_M x WAVES_N waves of 64 lanes, each
// wave owning a (BM/WAVES_M) x (BN/WAVES_N) block of 32x32 accumulator tiles
// (fp32).  K advances 64 bytes per step through double-buffered LDS (rows
// padded to 80 bytes, which makes the 16-byte fragment reads of 8
// consecutive lanes hit 8 disjoint groups of 4 banks).
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

constexpr int kRowBytes = 80;   // LDS bytes per tile row: 64 of data + 16 of padding
constexpr int kStepBytes = 64;  // bytes of K per row per pipeline step

template <typename T, int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64) void gemm_bias_kernel(
    const T *__restrict__ A, const T *__restrict__ B, const T *__restrict__ bias,
    T *__restrict__ out, GemmArgs a)
{
    constexpr int NT = WAVES_M * WAVES_N * 64;
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int CHUNKS = (BM + BN) * (kStepBytes / 16);   // 16-byte pieces per step
    static_assert(CHUNKS % NT == 0, "tile rows must split evenly over the threads");
    constexpr int PER_T = CHUNKS / NT;
    __shared__ __attribute__((aligned(16))) char smem[2][(BM + BN) * kRowBytes];

    uint32_t bid = xcd_swizzle(blockIdx.x, gridDim.x);
    const int mt = int(bid % uint32_t(a.tiles_m));
    bid /= uint32_t(a.tiles_m);
    const int nt = int(bid % uint32_t(a.tiles_n));
    const int g = int(bid / uint32_t(a.tiles_n));
    const int m0 = mt * BM, n0 = nt * BN;

    const size_t row_bytes = size_t(a.Kp) * sizeof(T);
    const char *Ag = reinterpret_cast<const char *>(A) + size_t(g) * a.Mg * row_bytes;
    const char *Bg = reinterpret_cast<const char *>(B) + size_t(g) * a.Ncols * row_bytes;

    // Global source of each of this thread's 16-byte pieces.  Rows past the
    // matrix edge are clamped to a valid row and their data replaced by 0.
    const char *src[PER_T];
    bool live[PER_T];
    int lds_off[PER_T];
#pragma unroll
    for (int s = 0; s < PER_T; ++s) {
        const int cid = int(threadIdx.x) + s * NT;
        const int r = cid / (kStepBytes / 16);
        const int part = cid % (kStepBytes / 16);
        if (r < BM) {
            const int m = m0 + r;
            live[s] = m < a.Mg;
            src[s] = Ag + size_t(live[s] ? m : a.Mg - 1) * row_bytes + part * 16;
        } else {
            const int n = n0 + (r - BM);
            live[s] = n < a.Ncols;
            src[s] = Bg + size_t(live[s] ? n : a.Ncols - 1) * row_bytes + part * 16;
        }
        lds_off[s] = r * kRowBytes + part * 16;
    }

    uint4 stage[PER_T];
    auto fetch = [&](int step) {
#pragma unroll
        for (int s = 0; s < PER_T; ++s) {
            uint4 v = *reinterpret_cast<const uint4 *>(src[s] + size_t(step) * kStepBytes);
            stage[s] = live[s] ? v : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto deposit = [&](int buf) {
#pragma unroll
        for (int s = 0; s < PER_T; ++s)
            *reinterpret_cast<uint4 *>(&smem[buf][lds_off[s]]) = stage[s];
    };

    const int lane = int(threadIdx.x) & 63;
    const int wave = int(threadIdx.x) >> 6;
    const int wm = wave % WAVES_M, wn = wave / WAVES_M;
    const int frag_row = lane & 31;
    const int frag_half = (lane >> 5) * 16;

    float16v acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.0f;

    const int steps = int(row_bytes / kStepBytes);
    fetch(0);
    deposit(0);
    __syncthreads();
    for (int st = 0; st < steps; ++st) {
        const int buf = st & 1;
        if (st + 1 < steps)
            fetch(st + 1);
        const char *sA = &smem[buf][(wm * WTM) * kRowBytes];
        const char *sB = &smem[buf][(BM + wn * WTN) * kRowBytes];
#pragma unroll
        for (int kg = 0; kg < kStepBytes / 32; ++kg) {
            uint4 af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const uint4 *>(
                    sA + (i * 32 + frag_row) * kRowBytes + kg * 32 + frag_half);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[j] = *reinterpret_cast<const uint4 *>(
                    sB + (j * 32 + frag_row) * kRowBytes + kg * 32 + frag_half);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = Mma<T>::step(af[i], bf[j], acc[i][j]);
        }
        if (st + 1 < steps)
            deposit(buf ^ 1);
        __syncthreads();
    }

    // Epilogue.  Accumulator register r of lane l in a 32x32 tile holds
    // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int n = n0 + wn * WTN + j * 32 + (lane & 31);
        if (n >= a.Ncols)
            continue;
        const int img = n / a.P;
        const int pix = n - img * a.P;
        T *obase = out + (size_t(img) * a.Co + size_t(g) * a.Mg) * a.P + pix;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (m < a.Mg) {
                    float v = acc[i][j][r];
                    if (a.has_bias)
                        v += to_f32(bias[size_t(g) * a.Mg + m]);
                    obase[size_t(m) * a.P] = from_f32<T>(v);
                }
            }
        }
    }
}

template <typename T>
hipError_t gemm_t(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                  const void *col, const void *bias, void *out, hipStream_t s)
{
    constexpr int BM = 128, BN = 128, WM = 2, WN = 2;
    GemmArgs a;
    a.Mg = int(p.Mg);
    a.Ncols = int(cnt * p.P);
    a.Kp = int(plan.Kp);
    a.P = int(p.P);
    a.Co = int(p.Co);
    a.tiles_m = int((p.Mg + BM - 1) / BM);
    a.tiles_n = int((a.Ncols + BN - 1) / BN);
    a.has_bias = bias != nullptr;
    const uint64_t blocks = uint64_t(p.G) * a.tiles_m * a.tiles_n;
    hipLaunchKernelGGL((gemm_bias_kernel<T, BM, BN, WM, WN>), dim3(uint32_t(blocks)),
                       dim3(WM * WN * 64), 0, s, static_cast<const T *>(wpack),
                       static_cast<const T *>(col), static_cast<const T *>(bias),
                       static_cast<T *>(out), a);
    return hipGetLastError();
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
