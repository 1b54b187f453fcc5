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
// A 16-byte chunk must lie in one offset group (C/deformable_group a multiple
// of 8 f16/bf16 or 4 f32 channels).
// B rows are output pixels (columns n*P + pix of the chunk).
//
// The workgroup's waves specialise.  Consumer waves only read the staged
// fragments and run the MFMAs (an in-order wave that issues memory operations
// stalls whenever the texture unit's queue is full, which would stop its
// MFMAs).  Producer waves move A by DMA and make the B rows.
//
// Gather cost is set by how many cache lines one load instruction touches,
// not by its bytes, so a producer load reads whole lines: eight lanes read
// the 128 bytes (the step's channels) of one pixel's corner, and a thread
// handles CPT rows (pixels) for one 16-byte chunk.  The bilinear geometry of
// every (offset group, tap, row) of the tile -- four corner byte offsets into
// the NHWC chunk and four fp32 weights with the mask folded in -- is built
// once per tile into an LDS table by the whole workgroup; a producer re-reads
// its rows' entries when the tap or offset group changes.  Corner loads
// (buffer loads; a corner off the image gets an out-of-range offset and
// reads 0) are issued three steps ahead of the consumers, between the rounds
// of the blend, conversion and LDS write of the step one ahead, so each load
// has two steps to land.  One consumer and one producer wave share each SIMD,
// so MFMA and VALU work overlap; one barrier per step separates the two LDS
// stages.
#include <atomic>
#include <cstdlib>
#include <map>
#include <mutex>

#include "launch.h"
#include "mfma_common.h"
#include "transpose.h"

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
    int DG;                      // deformable groups
    int nq;                      // offset groups of the geometry table (per group)
    uint32_t img_bytes;          // bytes of one NHWC image
    uint32_t chunk_bytes;        // bytes of the chunk's NHWC images (< 2^31)
    int steps;                   // K steps: Kg / (128 / sizeof(T))
};

// The one-launch forward: the workgroups first move x to NHWC and repack
// the weight themselves (each its share), then wait for one another at a
// bounded grid barrier before the GEMM.  Each workgroup announces that its
// share is stored by writing this launch's ticket (a value no other launch
// uses) into its own flag of a slot; it proceeds once every flag of the
// launch holds the ticket.  A workgroup that gives up waiting (some
// workgroup of the grid did not get a CU in time) moves all of x and the
// whole weight itself -- the same values the others store -- so the result
// never depends on the wait.
constexpr int kOneSlots = 64;                // flag slots (by workspace address)
constexpr int kOneMaxBlocks = 512;           // workgroups of a one-launch grid
constexpr uint32_t kOneSpinLimit = 1u << 15; // polls of the flags before giving up
__device__ uint64_t g_one_flags[kOneSlots * kOneMaxBlocks];

struct OneArgs {
    const void *x;               // the chunk's x, [cnt][C][H][W]
    const void *w;               // weight [Co][Cg][kh][kw]
    void *xt;                    // NHWC copy the GEMM reads (written here)
    void *wp;                    // packed weight the GEMM reads (written here)
    uint64_t *flags;             // the slot's kOneMaxBlocks flags
    uint64_t ticket;             // this launch's flag value
    uint32_t spin_limit;         // polls before a workgroup moves everything itself
    int vec;                     // x moves in 16-byte chunks (C, HW multiples of 16/elem)
    int HW, cnt;                 // pixels of an image, images of the chunk
    int total, Kg;               // packed weight elements (Co x Kp), Cg x K
};

// Cache policy of the set-up's stores and of the flags: device scope (SC1 on
// gfx950): written through to where every XCD sees them.
constexpr int kDevScopeAux = 16;
// LDS of one group of 256 threads in the set-up (the larger of the two tile
// transposes, 16-byte aligned)
constexpr int kOneLdsBytes = 64 * 65 * 4 + 64;

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

// A 16-byte LDS store the compiler does not track.  The compiler orders
// every LDS access after an LDS-writing DMA behind that DMA's completion;
// the producer's B stores never overlap the A rows its DMA fills, so they
// are written here, and the explicit lgkmcnt(0) before each barrier covers
// them.  (An untracked LDS operation can only make the compiler's own
// lgkmcnt waits wait longer, never shorter: LDS operations complete in order.)
__device__ __forceinline__ void lds_store16(char *p, uint4 v)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const uint32_t addr = uint32_t(reinterpret_cast<uintptr_t>((lds_void *)p));
    const u32x4 d = {v.x, v.y, v.z, v.w};
    asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(d) : "memory");
}

// x / d for 0 <= x, d < 2^16 through the fp32 reciprocal rd ~ 1/d: the
// product is within one of the quotient, and one correction each way makes
// it exact.
__device__ __forceinline__ int div_small(int x, int d, float rd)
{
    int q = int(float(x) * rd);
    q -= int(q * d > x);
    q += int((q + 1) * d <= x);
    return q;
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

// The tile's geometry table: for every (offset group qf+qq, tap k, B row r)
// entry e = (qq*K + k)*BN + r, 32 bytes: the byte offsets into the NHWC chunk
// of the four bilinear corners of row r's sample (kOffImage for a corner off
// the image) and their weights with the mask folded in.  Built once per
// tile by the whole workgroup; rows past the last column repeat a valid one.
template <typename T, int BN, int NT>
__device__ __forceinline__ void build_geo_table(char *tab, const FusedArgs &a,
                                                const T *__restrict__ off,
                                                const T *__restrict__ msk, int qf, int n0,
                                                int tid)
{
    const int E = a.nq * a.K * BN;
    const uint32_t elem_c = uint32_t(a.C) * uint32_t(sizeof(T));
#pragma unroll 2
    for (int e = tid; e < E; e += NT) {
        const int r = e % BN;
        const int kq = e / BN;
        const int k = kq % a.K;
        const int q = min(qf + kq / a.K, a.DG - 1);
        const int ncol = min(n0 + r, a.Ncols - 1);
        const int img = ncol / a.P;
        const int pix = ncol - img * a.P;
        const int ho = pix / a.Wo, wo = pix - ho * a.Wo;
        const int i = k / a.kw, j = k - (k / a.kw) * a.kw;
        const size_t ob = (size_t(img) * a.offC + size_t(q) * 2 * a.K + 2 * k) * a.P + pix;
        const float oh = to_f32(off[ob]);
        const float ow = to_f32(off[ob + a.P]);
        const float m = to_f32(msk[(size_t(img) * a.mskC + size_t(q) * a.K + k) * a.P + pix]);
        const Taps tp = make_taps(ho * a.sh - a.ph + i * a.dh, wo * a.sw - a.pw + j * a.dw, oh,
                                  ow, m, a.H, a.W);
        const uint32_t base = uint32_t(img) * a.img_bytes;
        uint32_t o[4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
            o[s] = tp.valid[s] ? base + uint32_t(tp.idx[s]) * elem_c : kOffImage;
        *reinterpret_cast<uint4 *>(tab + size_t(e) * 32) = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<float4 *>(tab + size_t(e) * 32 + 16) =
            make_float4(tp.wt[0], tp.wt[1], tp.wt[2], tp.wt[3]);
    }
}

// The one-launch set-up: NHWC tiles of x (256 threads a tile, one LDS
// buffer of kOneLdsBytes per group of 256 threads at the start of the
// stages) and packed weight elements ([Co][Kp], tap-major k*Cg + c', zero
// past Kg), stored with device scope.  A workgroup's share is a contiguous
// range of each, by its index in the grid.
struct OneRange {
    uint32_t lo, hi;             // NHWC tiles
    uint32_t plo, phi;           // packed weight elements
};

__device__ __forceinline__ OneRange one_range(const FusedArgs &a, const OneArgs &o, bool all)
{
    const uint64_t G = gridDim.x, b = blockIdx.x;
    const uint32_t TT = nhwc_tiles(a.C, o.HW, o.cnt), tot = uint32_t(o.total);
    if (all)
        return {0u, TT, 0u, tot};
    return {uint32_t(b * TT / G), uint32_t((b + 1) * TT / G), uint32_t(b * tot / G),
            uint32_t((b + 1) * tot / G)};
}

template <typename T>
__device__ __forceinline__ T one_weight(const FusedArgs &a, const OneArgs &o, uint32_t e)
{
    const int kk = int(e % uint32_t(a.Kp));
    const int co = int(e / uint32_t(a.Kp));
    if (kk >= o.Kg)
        return T(0);
    const int k = kk / a.Cg;
    const int cl = kk - k * a.Cg;
    return static_cast<const T *>(o.w)[(size_t(co) * a.Cg + cl) * a.K + k];
}

template <typename T>
__device__ __forceinline__ void store_dev(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, T v)
{
    if constexpr (sizeof(T) == 2)
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, v), r, byte_off, 0,
                                              kDevScopeAux);
    else
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, byte_off, 0,
                                              kDevScopeAux);
}

// Tiles [from, rg.hi) and weight elements [pfrom, rg.phi) (this thread's
// share of them), one round of NT/256 tiles at a time.  Every thread of the
// workgroup calls it (it has barriers).  The barriers order LDS only: the
// device-scope stores stay in flight until the wait before the grid barrier
// (a full __syncthreads would wait for each round's stores to be written
// through, about a microsecond and a half each).
template <typename T, int NT>
__device__ __forceinline__ void one_setup_rest(char *smem, const FusedArgs &a, const OneArgs &o,
                                               int tid, uint32_t from, uint32_t hi,
                                               uint32_t pfrom, uint32_t phi)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    constexpr int NQ = NT / 256;
    static_assert(NT % 256 == 0, "whole groups of 256 threads");
    const int q = tid >> 8, t = tid & 255;
    uint4 *lds = reinterpret_cast<uint4 *>(smem + q * kOneLdsBytes);
    const T *x = static_cast<const T *>(o.x);
    const __amdgpu_buffer_rsrc_t rxt = scalar_rsrc(o.xt, a.chunk_bytes);
    for (uint32_t base = from; base < hi; base += NQ) {
        const uint32_t tile = base + uint32_t(q);
        const bool ok = tile < hi;
        if (o.vec) {
            NhwcTile<T> tl;
            if (ok) {
                tl.load(x, a.C, o.HW, tile, t);
                tl.put(lds, t);
            }
            lds_barrier();
            if (ok)
                tl.take(lds, a.C, o.HW, t, [&](const uint4 &v, size_t off) {
                    const u32x4 d = {v.x, v.y, v.z, v.w};
                    __builtin_amdgcn_raw_buffer_store_b128(d, rxt, uint32_t(off * sizeof(T)), 0,
                                                           kDevScopeAux);
                });
        } else {
            NhwcTileScalar<T> tl;
            if (ok) {
                tl.load(x, a.C, o.HW, tile, t);
                tl.put(reinterpret_cast<T *>(lds), t);
            }
            lds_barrier();
            if (ok)
                tl.take(reinterpret_cast<const T *>(lds), a.C, o.HW, t,
                        [&](const T &v, size_t off) {
                            store_dev(rxt, uint32_t(off * sizeof(T)), v);
                        });
        }
        lds_barrier();
    }
    const __amdgpu_buffer_rsrc_t rwp = scalar_rsrc(o.wp, uint32_t(o.total) * uint32_t(sizeof(T)));
    for (uint32_t e = pfrom + uint32_t(tid); e < phi; e += NT)
        store_dev(rwp, e * uint32_t(sizeof(T)), one_weight<T>(a, o, e));
}

// The first loads of the workgroup's share, issued before the geometry table
// is built so that their latency overlaps it (16-byte tiles only): the
// first R rounds of tiles and P weight elements a thread.
template <typename T, int NT>
struct OnePre {
    static constexpr int R = 2, P = 2;
    NhwcTile<T> tl[R];
    T wv[P];
};

template <typename T, int NT>
__device__ __forceinline__ void one_setup_begin(OnePre<T, NT> &pre, const FusedArgs &a,
                                                const OneArgs &o, int tid)
{
    if (!o.vec)
        return;
    constexpr int NQ = NT / 256;
    const OneRange rg = one_range(a, o, false);
    const int q = tid >> 8, t = tid & 255;
#pragma unroll
    for (int r = 0; r < OnePre<T, NT>::R; ++r) {
        const uint32_t tile = rg.lo + uint32_t(r * NQ + q);
        if (tile < rg.hi)
            pre.tl[r].load(static_cast<const T *>(o.x), a.C, o.HW, tile, t);
    }
#pragma unroll
    for (int j = 0; j < OnePre<T, NT>::P; ++j) {
        const uint32_t e = rg.plo + uint32_t(tid + j * NT);
        pre.wv[j] = e < rg.phi ? one_weight<T>(a, o, e) : T(0);
    }
}

// The rest of the workgroup's share: the preloaded rounds transposed and
// stored, then whatever they did not cover.
template <typename T, int NT>
__device__ __forceinline__ void one_setup_end(const OnePre<T, NT> &pre, char *smem,
                                              const FusedArgs &a, const OneArgs &o, int tid)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    constexpr int NQ = NT / 256;
    const OneRange rg = one_range(a, o, false);
    if (!o.vec) {
        one_setup_rest<T, NT>(smem, a, o, tid, rg.lo, rg.hi, rg.plo, rg.phi);
        return;
    }
    const int q = tid >> 8, t = tid & 255;
    uint4 *lds = reinterpret_cast<uint4 *>(smem + q * kOneLdsBytes);
    const __amdgpu_buffer_rsrc_t rxt = scalar_rsrc(o.xt, a.chunk_bytes);
    // The preloaded values landed while the table was built.  Waiting for
    // them here, explicitly, lets the compiler drop its own waits on them
    // below, which would otherwise also wait for the stores issued in
    // between (loads and stores share one counter).
    __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0)
#pragma unroll
    for (int r = 0; r < OnePre<T, NT>::R; ++r) {
        const uint32_t base = rg.lo + uint32_t(r * NQ);
        if (base >= rg.hi)
            break;
        const bool ok = base + uint32_t(q) < rg.hi;
        if (ok)
            pre.tl[r].put(lds, t);
        lds_barrier();
        if (ok)
            pre.tl[r].take(lds, a.C, o.HW, t, [&](const uint4 &v, size_t off) {
                const u32x4 d = {v.x, v.y, v.z, v.w};
                __builtin_amdgcn_raw_buffer_store_b128(d, rxt, uint32_t(off * sizeof(T)), 0,
                                                       kDevScopeAux);
            });
        lds_barrier();
    }
    const __amdgpu_buffer_rsrc_t rwp = scalar_rsrc(o.wp, uint32_t(o.total) * uint32_t(sizeof(T)));
#pragma unroll
    for (int j = 0; j < OnePre<T, NT>::P; ++j) {
        const uint32_t e = rg.plo + uint32_t(tid + j * NT);
        if (e < rg.phi)
            store_dev(rwp, e * uint32_t(sizeof(T)), pre.wv[j]);
    }
    one_setup_rest<T, NT>(smem, a, o, tid, rg.lo + uint32_t(OnePre<T, NT>::R * NQ), rg.hi,
                          rg.plo + uint32_t(OnePre<T, NT>::P * NT), rg.phi);
}

template <typename T, int BM, int BN, int CWM, int CWN, int PW, bool ONE>
__global__ __launch_bounds__((CWM * CWN + PW) * 64) void fused_kernel(
    const T *A, const T *xt, const T *__restrict__ off, const T *__restrict__ msk,
    const T *__restrict__ bias, T *__restrict__ out, FusedArgs a, OneArgs o)
{
    constexpr int STEP = 128;
    constexpr int NC = CWM * CWN;                // consumer (MFMA) waves
    constexpr int NP = PW * 64;                  // producer threads
    constexpr int NT = NC * 64 + NP;
    constexpr int WTM = BM / CWM, WTN = BN / CWN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int STAGE_BYTES = (BM + BN) * STEP;
    constexpr int EV = 16 / int(sizeof(T));      // elements per 16-byte chunk
    constexpr int SE = STEP / int(sizeof(T));    // K elements per step
    constexpr int IPWA = BM / 8 / PW;            // A load instructions per producer wave
    constexpr int ROWS = NP / 8;                 // B rows per producer round
    constexpr int CPT = BN / ROWS;               // rounds: B rows per producer thread
    static_assert(BM % 32 == 0 && BN % 32 == 0 && (BM / 8) % PW == 0,
                  "A rows must split evenly into 8-row load instructions per producer wave");
    static_assert(NP % 8 == 0 && BN % ROWS == 0 && CPT >= 1 && CPT <= 8,
                  "B rows must split evenly over the producer rounds");
    static_assert(NC * 32 * (WTN + 4) * 4 <= 2 * STAGE_BYTES, "epilogue slices must fit in LDS");
    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE_BYTES];
    extern __shared__ __attribute__((aligned(16))) char tab[];   // geometry table

    uint32_t bid = xcd_swizzle(blockIdx.x, gridDim.x);
    const int mt = int(bid % uint32_t(a.tiles_m));
    bid /= uint32_t(a.tiles_m);
    const int nt = int(bid % uint32_t(a.tiles_n));
    const int g = __builtin_amdgcn_readfirstlane(int(bid / uint32_t(a.tiles_n)));
    const int m0 = mt * BM, n0 = nt * BN;
    const int qf = (g * a.Cg) / a.Cdg;           // first offset group of group g

    const int tid = int(threadIdx.x);
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    OnePre<T, NT> pre;
    if constexpr (ONE) {
        static_assert(NT / 256 * kOneLdsBytes <= 2 * STAGE_BYTES, "set-up buffers in the stages");
        one_setup_begin<T, NT>(pre, a, o, tid);
    }
    build_geo_table<T, BN, NT>(tab, a, off, msk, qf, n0, tid);
    if constexpr (ONE) {
        one_setup_end<T, NT>(pre, smem, a, o, tid);
        // grid barrier: every wave's device-scope stores are complete before
        // the workgroup's flag is written; wave 0 polls the grid's flags
        __shared__ uint32_t one_late;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (wave == 0) {
            const uint32_t G = gridDim.x;
            if (lane == 0)
                __hip_atomic_store(o.flags + blockIdx.x, o.ticket, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            bool done = false;
            for (uint32_t it = 0; it < o.spin_limit && !done; ++it) {
                bool mine = true;
                for (uint32_t j = uint32_t(lane); j < G; j += 64)
                    mine = mine && __hip_atomic_load(o.flags + j, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT) == o.ticket;
                done = __all(mine);
                if (!done)
                    __builtin_amdgcn_s_sleep(1);
            }
            if (lane == 0)
                one_late = done ? 0u : 1u;
        }
        __syncthreads();
        if (one_late) {
            const OneRange all = one_range(a, o, true);
            one_setup_rest<T, NT>(smem, a, o, tid, all.lo, all.hi, all.plo, all.phi);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        // The NHWC copy and the packed weight are read through the caches
        // from here on.  No cache can hold a stale line of them: the caches
        // start the kernel without one, nothing reads them before this
        // point, and the loads below are issued after every workgroup's
        // device-scope stores are complete.  (An agent-scope acquire here
        // would invalidate the whole L2 of the XCD once per workgroup, under
        // the feet of the workgroups already in their GEMM.)
    }
    __syncthreads();

    if (wave < NC) {
        // ---------------- consumer: MFMAs over the staged tiles
        const int wm = wave % CWM, wn = wave / CWM;
        float16v acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[i][j][r] = 0.0f;
        for (int st = 0; st < a.steps; ++st) {
            const int stage = st & 1;
            lds_barrier();                   // step st's A and B are in LDS
            const char *sA = smem + stage * STAGE_BYTES + wm * WTM * STEP;
            const char *sB = smem + stage * STAGE_BYTES + (BM + wn * WTN) * STEP;
            // fragments one k-group ahead of the MFMAs (two register sets)
            uint4 fa[2][FM], fb[2][FN];
            load_kgroup_frags<FM, FN>(fa[0], fb[0], sA, sB, lane, 0);
#pragma unroll
            for (int kg = 0; kg < 4; ++kg) {
                if (kg < 3)
                    load_kgroup_frags<FM, FN>(fa[(kg + 1) & 1], fb[(kg + 1) & 1], sA, sB, lane,
                                              kg + 1);
                mfma_frags<T, FM, FN>(acc, fa[kg & 1], fb[kg & 1]);
            }
        }
        __syncthreads();                     // operand stages no longer needed
        const EpilogueArgs e{g, m0, n0, a.Mg, a.Ncols, a.P, a.Co, a.has_bias, a.vec_out};
        epilogue_store<T, WTM, WTN>(acc, smem, bias, out, e, wm, wn, wave, lane);
        return;
    }

    // ---------------- producer: B from the bilinear gather
    // Lane c of each group of eight owns 16-byte chunk c of every B row the
    // group handles, rows r0 + ROWS*i for i < CPT: the eight lanes of a
    // corner load read one whole 128-byte line (the step's channels of one
    // pixel), so each load instruction touches eight lines.
    const int ptid = tid - NC * 64;
    const int pw = wave - NC;
    const int c = ptid & 7;
    const int r0 = ptid >> 3;
    // The packed weight's rows of the tile (A), moved by DMA: IPWA
    // instructions of 8 rows per producer wave and step.
    const uint32_t row_bytes = uint32_t(a.Kp) * uint32_t(sizeof(T));
    const char *Ag = reinterpret_cast<const char *>(A) + size_t(g) * a.Mg * row_bytes;
    const __amdgpu_buffer_rsrc_t ra = scalar_rsrc(Ag, uint32_t(a.Mg) * row_bytes);
    uint32_t voff_a[IPWA];
#pragma unroll
    for (int t = 0; t < IPWA; ++t) {
        const int row = (pw * IPWA + t) * 8 + (lane >> 3);
        voff_a[t] = uint32_t(min(m0 + row, a.Mg - 1)) * row_bytes + swz_chunk(row, lane & 7) * 16;
    }
    const __amdgpu_buffer_rsrc_t rx = scalar_rsrc(xt, a.chunk_bytes);
    char *b_lds = smem + BM * STEP;

    // Geometry of the (tap, offset group) last read from the table, the
    // lane's chunk offset included.  kOffImage plus the chunk and channel
    // offsets stays past the end of the range, so such a load reads 0.
    uint32_t goff[CPT][4];
    float gwt[CPT][4];
    int gk = -1, gq = -1;

    // (tap, offset group) of this lane's chunk at K step `step`: the step
    // covers channels cbase .. cbase+SE-1 of tap k (SE divides C/group).
    const int spt = a.Cg / SE;                   // steps per tap
    const float r_spt = 1.0f / float(spt), r_cdg = 1.0f / float(a.Cdg);
    auto step_tap = [&](int step, int &k, int &q, int &cbase) {
        k = div_small(step, spt, r_spt);
        cbase = g * a.Cg + (step - k * spt) * SE;               // uniform first channel
        q = div_small(cbase + c * EV, a.Cdg, r_cdg);
    };
    // Geometry of step `step` (from the table when the tap or offset group
    // changed); returns the step's uniform channel byte offset.
    auto geo_for = [&](int step) -> int {
        int k, q, cbase;
        step_tap(step, k, q, cbase);
        if (k != gk || q != gq) {
            const char *ent = tab + (size_t((q - qf) * a.K + k) * BN + r0) * 32;
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const uint4 o = *reinterpret_cast<const uint4 *>(ent + i * ROWS * 32);
                const float4 w = *reinterpret_cast<const float4 *>(ent + i * ROWS * 32 + 16);
                goff[i][0] = o.x + uint32_t(c * 16);
                goff[i][1] = o.y + uint32_t(c * 16);
                goff[i][2] = o.z + uint32_t(c * 16);
                goff[i][3] = o.w + uint32_t(c * 16);
                gwt[i][0] = w.x;
                gwt[i][1] = w.y;
                gwt[i][2] = w.z;
                gwt[i][3] = w.w;
            }
            gk = k;
            gq = q;
        }
        return __builtin_amdgcn_readfirstlane(cbase * int(sizeof(T)));
    };
    // A register set: the corner chunks of one step and the weights they are
    // blended with (the weights of later steps may differ).
    struct BSet {
        uint4 v[CPT][4];
        float w[CPT][4];
    };
    // Round i: record the current weights in b, issue the four corner loads.
    auto refill_round = [&](int i, int soff, BSet &b) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            b.w[i][s] = gwt[i][s];
            const auto r = __builtin_amdgcn_raw_buffer_load_b128(rx, goff[i][s], soff, 0);
            __builtin_memcpy(&b.v[i][s], &r, 16);
        }
    };
    // Round i: blend, convert and store the lane's chunk of row r0 + ROWS*i.
    auto blend_round = [&](int i, const BSet &b, int stage) {
        float accv[EV];
#pragma unroll
        for (int e = 0; e < EV; ++e)
            accv[e] = 0.0f;
#pragma unroll
        for (int s = 0; s < 4; ++s)
            fma_chunk<T>(accv, b.v[i][s], b.w[i][s]);
        Vec16<T> o;
#pragma unroll
        for (int e = 0; e < EV; ++e)
            o.e[e] = from_f32<T>(accv[e]);
        const int row = r0 + ROWS * i;
        lds_store16(b_lds + stage * STAGE_BYTES + row * STEP + swz_chunk(row, c) * 16, o.raw);
    };
    auto load_b = [&](int step, BSet &b) {
        const int soff = geo_for(step);
#pragma unroll
        for (int i = 0; i < CPT; ++i)
            refill_round(i, soff, b);
    };
    // Blend one step from set b into `stage` and, round by round, refill b
    // with the corners of the step geo_for last set up (when `more`; soff is
    // its channel offset): the loads go out between
    // the rounds of the blend, so the texture unit is fed while the VALU
    // works, and each load has two steps to land.
    auto blend_and_refill = [&](BSet &b, int stage, int soff, bool more) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            blend_round(i, b, stage);
            if (more)
                refill_round(i, soff, b);
            __builtin_amdgcn_sched_barrier(0);   // keep the rounds interleaved
        }
    };

    // Two register sets: s0 holds the even steps, s1 the odd ones.  Step
    // st+1's B is finished while the consumers run step st, and its set is
    // refilled with step st+3.  At a barrier the wave's LDS writes and A DMA
    // must be complete but the corner loads behind them stay in flight, so the
    // wait is explicit (a fence would wait for every load): s_waitcnt
    // vmcnt(4*CPT) lgkmcnt(0), in the gfx9 encoding (vmcnt in bits 3:0 and
    // 15:14, expcnt 6:4 at its maximum, lgkmcnt 11:8).
    constexpr int WAIT_A = ((4 * CPT) & 15) | ((((4 * CPT) >> 4) & 3) << 14) | 0x70;
    BSet s0, s1;
    // A of step 0, then B of steps 0, 1 and 2 (the last step again when there
    // are fewer, so that no load sits behind a branch and the compiler's
    // waits count exactly).
    issue_a_rows<IPWA>(smem, ra, voff_a, pw, 0);
    load_b(0, s0);
    load_b(min(1, a.steps - 1), s1);
    blend_and_refill(s0, 0, geo_for(min(2, a.steps - 1)), true);
    // Body of step st: after the barrier, the DMA of step st+1's A rows,
    // then step st+1's B.  The previous body issued its A DMA before its
    // 4*CPT corner loads (when it had any), so at this barrier everything but
    // those loads must have landed.
    auto body = [&](int st, BSet &b, bool more, bool prev_loaded) {
        const int stage = st & 1;
        // The compiler barrier and scheduling fences keep the B stores before
        // the barrier and step st+1's B arithmetic after it, so the consumers
        // are released as soon as step st's operands are in LDS.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        if (prev_loaded)
            __builtin_amdgcn_s_waitcnt(WAIT_A);
        else
            __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();    // step st's A and B are in LDS
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        if (st + 1 < a.steps) {
            // table reads first: an LDS access after an LDS-writing DMA is
            // made to wait for the DMA (and so for every older load)
            const int soff = more ? geo_for(st + 3) : 0;
            issue_a_rows<IPWA>(smem + (stage ^ 1) * STAGE_BYTES, ra, voff_a, pw, st + 1);
            blend_and_refill(b, stage ^ 1, soff, more);
        }
    };
    // Main loop: every body loads (st + 4 < steps); then at most four steps,
    // loading while st + 3 < steps.
    int st = 0;
    for (; st + 4 < a.steps; st += 2) {
        body(st, s1, true, true);
        body(st + 1, s0, true, true);
    }
    // body(t) loads when t + 3 < steps; the prologue loaded before body(0)
    if (st < a.steps)
        body(st, s1, st + 3 < a.steps, st == 0 || st + 2 < a.steps);
    if (st + 1 < a.steps)
        body(st + 1, s0, st + 4 < a.steps, st + 3 < a.steps);
    if (st + 2 < a.steps)
        body(st + 2, s1, false, st + 4 < a.steps);
    if (st + 3 < a.steps)
        body(st + 3, s0, false, false);
    __syncthreads();                     // matches the consumers' barrier before the epilogue
}

template <typename T, int BM, int BN, int CWM, int CWN, int PW, bool ONE = false>
hipError_t fused_cfg(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                     const void *xt, const void *offset, const void *mask, const void *bias,
                     void *out, hipStream_t s, const OneArgs *one = nullptr)
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
    a.DG = int(p.DG);
    a.nq = int(fused_offset_groups(p));
    a.img_bytes = uint32_t(size_t(p.H) * p.W * p.C * sizeof(T));
    a.chunk_bytes = uint32_t(size_t(cnt) * a.img_bytes);
    a.steps = int(p.Kg * int64_t(sizeof(T)) / 128);
    const uint64_t blocks = uint64_t(p.G) * a.tiles_m * a.tiles_n;
    // The geometry table is the dynamic part of the LDS; the plan only picks
    // tiles whose stages and table fit.
    const size_t table = fused_table_bytes(p, BN);
    // (the one-launch variant has a few more bytes of static LDS)
    const size_t stages = size_t(2) * (BM + BN) * 128 + (ONE ? 256 : 0);
    if (stages + table > kLdsBytes)
        return ONE ? hipErrorNotSupported : hipErrorInvalidValue;
    if (ONE && (!one || blocks > uint64_t(kOneMaxBlocks)))
        return hipErrorInvalidValue;
    auto kern = fused_kernel<T, BM, BN, CWM, CWN, PW, ONE>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
        int(kLdsBytes - stages));
    if (attr != hipSuccess)
        return attr;
    hipLaunchKernelGGL(kern, dim3(uint32_t(blocks)), dim3((CWM * CWN + PW) * 64), table, s,
                       static_cast<const T *>(wpack),
                       static_cast<const T *>(xt), static_cast<const T *>(offset),
                       static_cast<const T *>(mask), static_cast<const T *>(bias),
                       static_cast<T *>(out), a, one ? *one : OneArgs{});
    return hipGetLastError();
}

template <typename T>
hipError_t fused_t(const Problem &p, const Plan &plan, int64_t cnt, const void *wpack,
                   const void *xt, const void *offset, const void *mask, const void *bias,
                   void *out, hipStream_t s, const OneArgs *one = nullptr)
{
    if (one) {
        // the one-launch variant exists for the 64-column tiles (the ones a
        // grid of at most one workgroup per CU gets)
        if (plan.fused_tile == FusedTile::M256_N64)
            return fused_cfg<T, 256, 64, 4, 2, 4, true>(p, plan, cnt, wpack, xt, offset, mask,
                                                         bias, out, s, one);
        if (plan.fused_tile == FusedTile::M128_N64)
            return fused_cfg<T, 128, 64, 2, 2, 4, true>(p, plan, cnt, wpack, xt, offset, mask,
                                                         bias, out, s, one);
        return hipErrorNotSupported;
    }
    switch (plan.fused_tile) {
    // <BM, BN, consumer wave grid CWM x CWN, producer waves>: 16, 16, 12 and
    // 8 waves, i.e. 4, 4, 3 and 2 waves per SIMD (at most 128, 128, 168 and
    // 256 registers each), half of them producers or close to it.
    case FusedTile::M256_N128:
        return fused_cfg<T, 256, 128, 4, 2, 8>(p, plan, cnt, wpack, xt, offset, mask, bias, out, s);
    case FusedTile::M128_N128:
        return fused_cfg<T, 128, 128, 2, 4, 8>(p, plan, cnt, wpack, xt, offset, mask, bias, out, s);
    case FusedTile::M256_N64:
        return fused_cfg<T, 256, 64, 4, 2, 4>(p, plan, cnt, wpack, xt, offset, mask, bias, out, s);
    case FusedTile::M128_N64:
        return fused_cfg<T, 128, 64, 2, 2, 4>(p, plan, cnt, wpack, xt, offset, mask, bias, out, s);
    }
    return hipErrorInvalidValue;
}

// Device address of g_one_flags on the current device (asked once per device).
uint64_t *one_flags_address()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        return nullptr;
    static std::mutex mu;
    static std::map<int, uint64_t *> known;
    std::lock_guard<std::mutex> lock(mu);
    auto it = known.find(dev);
    if (it == known.end()) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(g_one_flags)) != hipSuccess || ptr == nullptr)
            return nullptr;
        it = known.emplace(dev, static_cast<uint64_t *>(ptr)).first;
    }
    return it->second;
}

}  // namespace

hipError_t launch_fused_one(const Problem &p, const Plan &plan, int64_t cnt, const void *x,
                            const void *weight, void *wpack, void *xt, const void *offset,
                            const void *mask, const void *bias, void *out, hipStream_t stream)
{
    // opt-in (MDCN_FUSED_ONE=1): measured on the strided/grouped bf16 stage
    // (N=2, C=128, Co=256, 128x128, 256 workgroups), the two launches take
    // 20.8 us and the one launch 23.0 us -- the NHWC copy written through to
    // where every XCD sees it and the flag round trip take about 6 us after
    // the last store is issued, more than the kernel boundary they replace
    const char *env = std::getenv("MDCN_FUSED_ONE");
    if (!env || std::atoi(env) != 1)
        return hipErrorNotSupported;
    if (plan.fused_tile != FusedTile::M128_N64 && plan.fused_tile != FusedTile::M256_N64)
        return hipErrorNotSupported;
    // a captured launch would replay with the same ticket: two launches there
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone)
        return hipErrorNotSupported;
    // at most one workgroup per CU, so that the whole grid is resident
    const int64_t bm = plan.fused_tile == FusedTile::M256_N64 ? 256 : 128;
    const int64_t blocks = p.G * ((p.Mg + bm - 1) / bm) * ((cnt * p.P + 63) / 64);
    if (blocks > std::min<int64_t>(device_cu_count(), kOneMaxBlocks))
        return hipErrorNotSupported;
    const int64_t ev = 16 / int64_t(p.elem);
    const int64_t HW = p.H * p.W;
    if (p.Co * plan.Kp * int64_t(p.elem) >= (int64_t(1) << 32))
        return hipErrorNotSupported;
    uint64_t *flags = one_flags_address();
    if (!flags)
        return hipErrorNotSupported;
    static std::atomic<uint64_t> tickets{0};
    // the slot by workspace address: launches that may overlap use different
    // workspaces; two that share a slot anyway only wait until one gives up
    const uint64_t h = (uint64_t(reinterpret_cast<uintptr_t>(xt)) >> 8) * 0x9E3779B97F4A7C15ull;
    OneArgs o{};
    o.x = x;
    o.w = weight;
    o.xt = xt;
    o.wp = wpack;
    o.flags = flags + size_t(h >> 58) * kOneMaxBlocks;
    o.ticket = ++tickets;
    o.spin_limit = kOneSpinLimit;
    // MDCN_FUSED_ONE_SPIN=<polls> shortens the wait (tests force the
    // fallback with 0)
    if (const char *env = std::getenv("MDCN_FUSED_ONE_SPIN")) {
        const long long v = std::atoll(env);
        if (v >= 0 && v <= (long long)kOneSpinLimit)
            o.spin_limit = uint32_t(v);
    }
    o.vec = p.C % ev == 0 && HW % ev == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
            reinterpret_cast<uintptr_t>(xt) % 16 == 0;
    o.HW = int(HW);
    o.cnt = int(cnt);
    o.total = int(p.Co * plan.Kp);
    o.Kg = int(p.Kg);
    switch (p.dtype) {
    case MDCN_F32:
        return fused_t<float>(p, plan, cnt, wpack, xt, offset, mask, bias, out, stream, &o);
    case MDCN_F16:
        return fused_t<half_t>(p, plan, cnt, wpack, xt, offset, mask, bias, out, stream, &o);
    case MDCN_BF16:
        return fused_t<bf16_t>(p, plan, cnt, wpack, xt, offset, mask, bias, out, stream, &o);
    }
    return hipErrorInvalidValue;
}

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
