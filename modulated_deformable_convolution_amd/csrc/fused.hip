// fused.hip -- the deformable gather fused into the grouped MFMA GEMM
// (implicit GEMM): the B operand of each K step is produced in LDS from the
// bilinear samples instead of being read from a column buffer.
//   out[n][g*Mg + m][pix] = bias[g*Mg + m]
//       + sum_{k, c'} A[g][m][k*Cg + c'] * mask * bilinear0(x[n][g*Cg + c'], sample(k, pix))
// [plugin guide §五 steps 1-3: the same three stages, without the columns
// buffer between step 1 and step 2].
//
// Tiling and A (packed weight) movement are those of gemm.hip: BM x BN tile,
// 128-byte K steps (64 f16/bf16 or 32 f32 channels of one tap, which requires
// C/group to be a multiple of that), two LDS stages, swizzled 128-byte rows.
// B rows are output pixels (columns n*P + pix of the chunk).
//
// The workgroup's waves specialise.  Consumer waves move A by DMA and run the
// MFMAs: at each step they read the staged fragments into registers, issue
// the DMA of the next step's A rows into the other stage, then multiply, so
// the DMA flies under the MFMAs.  Producer waves make the B rows: each
// producer thread owns one B row and CPT of its eight 16-byte chunks, keeps
// that pixel's bilinear geometry for the current (tap, offset group) in
// registers -- four corner byte offsets into the NHWC chunk and four fp32
// weights with the mask folded in -- and recomputes it only when the tap or
// offset group changes, from offset and mask values it loaded one step
// earlier.  Its corner loads (buffer loads; a corner off the image gets an
// out-of-range offset and reads 0) are issued three steps ahead of the
// consumers, between the chunks of the blend, conversion and LDS write of the
// step one ahead, so each load has two steps to land.  One consumer and one producer
// wave share each SIMD, so MFMA and VALU work overlap; one barrier per step
// separates the two LDS stages.
#include "launch.h"
#include "mfma_common.h"

namespace mdcn {

namespace {

constexpr uint32_t kOffImage = 0x80000000u;   // a byte offset past any chunk

struct FusedArgs {
    int Mg, Ncols, Kp, P, Co;
    int tiles_m, tiles_n;
    int has_bias, vec_out;
    int Cg, Cdg, C, H, W, Wo, kw, K;
    int sh, sw, ph, pw, dh, dw;
    int offC, mskC;
    uint32_t img_bytes;          // bytes of one NHWC image
    uint32_t chunk_bytes;        // bytes of the chunk's NHWC images (< 2^31)
    int steps;                   // K steps: Kg / (128 / sizeof(T))
};

// Buffer resource over `bytes` bytes at `base`, built from scalar copies so
// that it provably lives in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t scalar_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t v = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
    void *p = reinterpret_cast<void *>((uint64_t(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, int(n), 0x00020000);
}

// One K step of the wave's A rows (IPWA instructions of 8 rows) into a stage.
template <int IPWA>
__device__ __forceinline__ void issue_a_rows(char *stage_base, __amdgpu_buffer_rsrc_t ra,
                                             const uint32_t *voff_a, int wave, int step)
{
#pragma unroll
    for (int t = 0; t < IPWA; ++t)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (lds_void *)(stage_base + (wave * IPWA + t) * 8 * 128), 16, voff_a[t],
            step * 128, 0, 0);
}

// Instruction t of issue_a_rows alone.
__device__ __forceinline__ void issue_a_row(char *stage_base, __amdgpu_buffer_rsrc_t ra,
                                            const uint32_t *voff_a, int wave, int step, int ipwa,
                                            int t)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(stage_base + (wave * ipwa + t) * 8 * 128),
                                             16, voff_a[t], step * 128, 0, 0);
}

template <typename T>
__device__ __forceinline__ void fma_chunk(float *acc, const uint4 &raw, float w)
{
    Vec16<T> v;
    v.raw = raw;
#pragma unroll
    for (int e = 0; e < Vec16<T>::N; ++e)
        acc[e] = fmaf(w, to_f32(v.e[e]), acc[e]);
}

template <typename T, int BM, int BN, int CWM, int CWN, int PW>
__global__ __launch_bounds__((CWM * CWN + PW) * 64) void fused_kernel(
    const T *__restrict__ A, const T *__restrict__ xt, const T *__restrict__ off,
    const T *__restrict__ msk, const T *__restrict__ bias, T *__restrict__ out, FusedArgs a)
{
    constexpr int STEP = 128;
    constexpr int NC = CWM * CWN;                // consumer (MFMA) waves
    constexpr int NP = PW * 64;                  // producer threads
    constexpr int WTM = BM / CWM, WTN = BN / CWN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int STAGE_BYTES = (BM + BN) * STEP;
    constexpr int EV = 16 / int(sizeof(T));      // elements per 16-byte chunk
    constexpr int SE = STEP / int(sizeof(T));    // K elements per step
    constexpr int IPWA = BM / 8 / NC;            // A load instructions per consumer wave
    constexpr int CPT = BN * 8 / NP;             // B chunks per producer thread per step
    constexpr int TPR = 8 / CPT;                 // producer threads per B row
    static_assert(BM % 32 == 0 && BN % 32 == 0 && (BM / 8) % NC == 0,
                  "A rows must split evenly into 8-row load instructions per consumer wave");
    static_assert((BN * 8) % NP == 0 && CPT >= 1 && CPT <= 8 && 8 % CPT == 0,
                  "B chunks must split evenly over the producer threads");
    static_assert(NC * 32 * (WTN + 4) * 4 <= 2 * STAGE_BYTES, "epilogue slices must fit in LDS");
    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE_BYTES];

    uint32_t bid = xcd_swizzle(blockIdx.x, gridDim.x);
    const int mt = int(bid % uint32_t(a.tiles_m));
    bid /= uint32_t(a.tiles_m);
    const int nt = int(bid % uint32_t(a.tiles_n));
    const int g = __builtin_amdgcn_readfirstlane(int(bid / uint32_t(a.tiles_n)));
    const int m0 = mt * BM, n0 = nt * BN;

    const int tid = int(threadIdx.x);
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    if (wave < NC) {
        // ---------------- consumer: A by DMA, MFMAs over the staged tiles
        const uint32_t row_bytes = uint32_t(a.Kp) * uint32_t(sizeof(T));
        const char *Ag = reinterpret_cast<const char *>(A) + size_t(g) * a.Mg * row_bytes;
        const __amdgpu_buffer_rsrc_t ra = scalar_rsrc(Ag, uint32_t(a.Mg) * row_bytes);
        uint32_t voff_a[IPWA];
#pragma unroll
        for (int t = 0; t < IPWA; ++t) {
            const int row = (wave * IPWA + t) * 8 + (lane >> 3);
            voff_a[t] = uint32_t(min(m0 + row, a.Mg - 1)) * row_bytes +
                        swz_chunk(row, lane & 7) * 16;
        }
        const int wm = wave % CWM, wn = wave / CWM;
        float16v acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[i][j][r] = 0.0f;
        issue_a_rows<IPWA>(smem, ra, voff_a, wave, 0);
        for (int st = 0; st < a.steps; ++st) {
            const int stage = st & 1;
            __builtin_amdgcn_s_waitcnt(0);   // this wave's A rows of step st have landed
            lds_barrier();                   // ... and all of step st's A and B
            StepFrags<FM, FN> f;             // read before the DMA into the other stage
            load_step_frags<FM, FN>(f, smem + stage * STAGE_BYTES + wm * WTM * STEP,
                                    smem + stage * STAGE_BYTES + (BM + wn * WTN) * STEP, lane);
            // The next step's A DMA is spread over the four k-groups of MFMAs
            // so that a busy texture unit never holds up the whole step.
            const bool more = st + 1 < a.steps;
#pragma unroll
            for (int kg = 0; kg < 4; ++kg) {
                mfma_kgroup<T, FM, FN>(acc, f, kg);
#pragma unroll
                for (int t = 0; t < IPWA; ++t)
                    if (more && (t * 4) / IPWA == kg)
                        issue_a_row(smem + (stage ^ 1) * STAGE_BYTES, ra, voff_a, wave, st + 1,
                                    IPWA, t);
            }
        }
        __syncthreads();                     // operand stages no longer needed
        const EpilogueArgs e{g, m0, n0, a.Mg, a.Ncols, a.P, a.Co, a.has_bias, a.vec_out};
        epilogue_store<T, WTM, WTN>(acc, smem, bias, out, e, wm, wn, wave, lane);
        return;
    }

    // ---------------- producer: B from the bilinear gather
    const int ptid = tid - NC * 64;
    // This thread's B row (output column) and chunk range.
    const int brow = ptid / TPR;
    const int bh = ptid % TPR;
    const int ncol = min(n0 + brow, a.Ncols - 1);        // rows past the edge: any valid column
    const int img = ncol / a.P;
    const int pix = ncol - img * a.P;
    const int ho = pix / a.Wo;
    const int anc_h = ho * a.sh - a.ph, anc_w = (pix - ho * a.Wo) * a.sw - a.pw;
    const uint32_t elem_c = uint32_t(a.C) * uint32_t(sizeof(T));
    // Per corner: byte offset of this thread's first chunk at that corner
    // (image base + pixel + the thread's channel slot), or kOffImage for a
    // corner off the image; the step's channel base is added as the uniform
    // buffer offset, the chunk index as the immediate offset.  kOffImage plus
    // either stays past the end of the range, so such a load reads 0.
    const uint32_t lane_base = uint32_t(img) * a.img_bytes + uint32_t(bh * CPT * 16);
    const __amdgpu_buffer_rsrc_t rx = scalar_rsrc(xt, a.chunk_bytes);
    char *b_lds = smem + BM * STEP + brow * STEP;

    uint32_t goff[4];
    float gwt[4];
    int gk = -1, gq = -1;                 // (tap, offset group) of goff/gwt
    T pf_oh, pf_ow, pf_m;                 // offset and mask of the next geo_for's step

    // (tap, offset group) of this thread's chunks at K step `step`: the step
    // covers channels cbase .. cbase+SE-1 of tap k (SE divides C/group).
    auto step_tap = [&](int step, int &k, int &q, int &cbase) {
        const int kk0 = step * SE;
        k = kk0 / a.Cg;
        cbase = g * a.Cg + (kk0 - k * a.Cg);                     // uniform first channel
        q = (cbase + bh * CPT * EV) / a.Cdg;
    };
    auto fetch_geo = [&](int k, int q) {
        const size_t ob = (size_t(img) * a.offC + size_t(q) * 2 * a.K + 2 * k) * a.P + pix;
        pf_oh = off[ob];
        pf_ow = off[ob + a.P];
        pf_m = msk[(size_t(img) * a.mskC + size_t(q) * a.K + k) * a.P + pix];
    };
    // A register set: the corner chunks of one step and the four bilinear
    // weights they are blended with (the weights of later steps may differ).
    struct BSet {
        uint4 v[CPT][4];
        float w[4];
    };
    // Geometry of step `step`: recomputes the corner offsets and weights
    // (goff, gwt) if the (tap, offset group) changed, and starts loading the
    // offset and mask of the step after (the last step reloads its own; a
    // load behind no branch lets the compiler's later wait for it count
    // exactly, leaving the corner loads in flight).  Returns the step's
    // uniform channel byte offset.
    auto geo_for = [&](int step) -> int {
        int k, q, cbase;
        step_tap(step, k, q, cbase);
        // pf_* hold this step's offset and mask.  They are converted and
        // pinned here, outside the branch: with their only use inside it the
        // compiler moves the loads into the branch, right in front of the
        // use, where waiting for them also waits for every corner load.
        float oh = to_f32(pf_oh), ow = to_f32(pf_ow), m = to_f32(pf_m);
        asm volatile("" : "+v"(oh), "+v"(ow), "+v"(m));
        if (k != gk || q != gq) {
            const int i = k / a.kw, j = k - (k / a.kw) * a.kw;
            const Taps tp = make_taps(anc_h + i * a.dh, anc_w + j * a.dw, oh, ow, m, a.H, a.W);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                goff[s] = tp.valid[s] ? lane_base + uint32_t(tp.idx[s]) * elem_c : kOffImage;
                gwt[s] = tp.wt[s];
            }
            gk = k;
            gq = q;
        }
        int k1, q1, c1;
        step_tap(min(step + 1, a.steps - 1), k1, q1, c1);
        fetch_geo(k1, q1);
        return __builtin_amdgcn_readfirstlane(cbase * int(sizeof(T)));
    };
    // The four corner loads of chunk jc (geometry from the last geo_for).
    auto issue_chunk = [&](int jc, int soff, BSet &b) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const auto r = __builtin_amdgcn_raw_buffer_load_b128(rx, goff[s] + jc * 16, soff, 0);
            __builtin_memcpy(&b.v[jc][s], &r, 16);
        }
    };
    auto keep_weights = [&](BSet &b) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            b.w[s] = gwt[s];
    };
    // Blend, convert and store chunk jc of a step into LDS stage `stage`.
    auto blend_chunk = [&](int jc, const BSet &b, int stage) {
        float accv[EV];
#pragma unroll
        for (int e = 0; e < EV; ++e)
            accv[e] = 0.0f;
#pragma unroll
        for (int s = 0; s < 4; ++s)
            fma_chunk<T>(accv, b.v[jc][s], b.w[s]);
        Vec16<T> o;
#pragma unroll
        for (int e = 0; e < EV; ++e)
            o.e[e] = from_f32<T>(accv[e]);
        *reinterpret_cast<uint4 *>(b_lds + stage * STAGE_BYTES +
                                   swz_chunk(brow, bh * CPT + jc) * 16) = o.raw;
    };
    // Blend one step from set b into `stage` and, chunk by chunk, refill b
    // with the corners of step `next` (when `more`): the loads go out between
    // the chunks of the blend, so the texture unit is fed while the VALU
    // works, and each load has two steps to land.
    auto blend_and_refill = [&](BSet &b, int stage, int next, bool more) {
        const int soff = more ? geo_for(next) : 0;
#pragma unroll
        for (int jc = 0; jc < CPT; ++jc) {
            blend_chunk(jc, b, stage);
            if (more)
                issue_chunk(jc, soff, b);
            __builtin_amdgcn_sched_barrier(0);   // keep the chunks interleaved
        }
        if (more)
            keep_weights(b);
    };

    // Two register sets: s0 holds the even steps, s1 the odd ones.  Step
    // st+1's B is finished while the consumers run step st, and its set is
    // refilled with step st+3.  Only this wave's LDS writes must be complete
    // at the barrier; the loads of later steps stay in flight, so the wait is
    // explicit (a fence here would wait for every load): s_waitcnt
    // lgkmcnt(0), in the gfx9 encoding (vmcnt in bits 3:0 and 15:14 at its
    // maximum, expcnt 6:4 at its maximum, lgkmcnt 11:8 zero).
    constexpr int WAIT_LDS = 0xC07F;
    BSet s0, s1;
    {
        int k0, q0, c0;
        step_tap(0, k0, q0, c0);
        fetch_geo(k0, q0);
    }
    auto load_b = [&](int step, BSet &b) {
        const int soff = geo_for(step);
        keep_weights(b);
#pragma unroll
        for (int jc = 0; jc < CPT; ++jc)
            issue_chunk(jc, soff, b);
    };
    // Steps 0, 1 and 2 (the last step again when there are fewer: no load
    // behind a branch here either).
    load_b(0, s0);
    load_b(min(1, a.steps - 1), s1);
    blend_and_refill(s0, 0, min(2, a.steps - 1), true);
    auto body = [&](int st, BSet &b, bool more) {
        const int stage = st & 1;
        // The compiler barrier and scheduling fences keep the B stores before
        // the barrier and step st+1's B arithmetic after it, so the consumers
        // are released as soon as step st's operands are in LDS.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(WAIT_LDS);
        __builtin_amdgcn_s_barrier();    // step st's A and B are in LDS
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        if (st + 1 < a.steps)
            blend_and_refill(b, stage ^ 1, st + 3, more);
    };
    // Main loop: every body loads (st + 4 < steps); then at most four steps,
    // loading while st + 3 < steps.
    int st = 0;
    for (; st + 4 < a.steps; st += 2) {
        body(st, s1, true);
        body(st + 1, s0, true);
    }
    if (st < a.steps)
        body(st, s1, st + 3 < a.steps);
    if (st + 1 < a.steps)
        body(st + 1, s0, st + 4 < a.steps);
    if (st + 2 < a.steps)
        body(st + 2, s1, false);
    if (st + 3 < a.steps)
        body(st + 3, s0, false);
    __syncthreads();                     // matches the consumers' barrier before the epilogue
}

template <typename T, int BM, int BN, int CWM, int CWN, int PW>
hipError_t fused_cfg(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                     const void *xt, const void *offset, const void *mask, const void *bias,
                     void *out, hipStream_t s)
{
    FusedArgs a;
    a.Mg = int(p.Mg);
    a.Ncols = int(cnt * p.P);
    a.Kp = int(plan.Kp);
    a.P = int(p.P);
    a.Co = int(p.Co);
    a.tiles_m = int((p.Mg + BM - 1) / BM);
    a.tiles_n = int((a.Ncols + BN - 1) / BN);
    a.has_bias = bias != nullptr;
    a.vec_out = (p.P % (16 / int(sizeof(T))) == 0) && reinterpret_cast<uintptr_t>(out) % 16 == 0;
    a.Cg = int(p.Cg); a.Cdg = int(p.Cdg); a.C = int(p.C);
    a.H = int(p.H); a.W = int(p.W); a.Wo = int(p.Wo); a.kw = int(p.kw); a.K = int(p.K);
    a.sh = int(p.sh); a.sw = int(p.sw); a.ph = int(p.ph); a.pw = int(p.pw);
    a.dh = int(p.dh); a.dw = int(p.dw);
    a.offC = int(2 * p.DG * p.K); a.mskC = int(p.DG * p.K);
    a.img_bytes = uint32_t(size_t(p.H) * p.W * p.C * sizeof(T));
    a.chunk_bytes = uint32_t(size_t(cnt) * a.img_bytes);
    a.steps = int(p.Kg * int64_t(sizeof(T)) / 128);
    const uint64_t blocks = uint64_t(p.G) * a.tiles_m * a.tiles_n;
    hipLaunchKernelGGL((fused_kernel<T, BM, BN, CWM, CWN, PW>), dim3(uint32_t(blocks)),
                       dim3((CWM * CWN + PW) * 64), 0, s, static_cast<const T *>(wpack),
                       static_cast<const T *>(xt), static_cast<const T *>(offset),
                       static_cast<const T *>(mask), static_cast<const T *>(bias),
                       static_cast<T *>(out), a);
    return hipGetLastError();
}

template <typename T>
hipError_t fused_t(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                   const void *xt, const void *offset, const void *mask, const void *bias,
                   void *out, hipStream_t s)
{
    switch (plan.fused_tile) {
    case FusedTile::M256_N128:
        return fused_cfg<T, 256, 128, 2, 2, 4>(p, plan, cnt, wpack, xt, offset, mask, bias, out, s);
    case FusedTile::M128_N128:
        return fused_cfg<T, 128, 128, 2, 2, 4>(p, plan, cnt, wpack, xt, offset, mask, bias, out, s);
    case FusedTile::M256_N64:
        return fused_cfg<T, 256, 64, 2, 2, 2>(p, plan, cnt, wpack, xt, offset, mask, bias, out, s);
    case FusedTile::M128_N64:
        return fused_cfg<T, 128, 64, 2, 2, 2>(p, plan, cnt, wpack, xt, offset, mask, bias, out, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fused(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                        const void *xt, const void *offset, const void *mask, const void *bias,
                        void *out, hipStream_t stream)
{
    switch (p.dtype) {
    case MDCN_F32:
        return fused_t<float>(p, plan, cnt, wpack, xt, offset, mask, bias, out, stream);
    case MDCN_F16:
        return fused_t<half_t>(p, plan, cnt, wpack, xt, offset, mask, bias, out, stream);
    case MDCN_BF16:
        return fused_t<bf16_t>(p, plan, cnt, wpack, xt, offset, mask, bias, out, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mdcn
