// plan.cpp -- validation and planning (host only).
#include "plan.h"

#include <algorithm>
#include <climits>
#include <cstdlib>

namespace mdcn {

namespace {

constexpr int64_t kMaxPerImage = (int64_t(1) << 31) - 1;   // elements per image tensor

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// Product of non-negative values, saturating at INT64_MAX (dims come from the
// caller, so their products must not overflow).
int64_t mul(int64_t a, int64_t b)
{
    int64_t r;
    if (__builtin_mul_overflow(a, b, &r))
        return INT64_MAX;
    return r;
}

int64_t mul(int64_t a, int64_t b, int64_t c) { return mul(mul(a, b), c); }

// GEMM tile: the tallest tile the group's weight rows fill, then the widest
// column count that still gives about one workgroup per CU or more.
// MDCN_GEMM_TILE=<0..5> overrides the choice (for tuning).
GemmTile choose_gemm_tile(const Problem &p, int64_t chunk)
{
    if (const char *env = std::getenv("MDCN_GEMM_TILE")) {
        const int v = std::atoi(env);
        if (v >= 0 && v < kGemmTileCount)
            return static_cast<GemmTile>(v);
    }
    const int64_t ncols = chunk * p.P;
    auto tiles = [&](int64_t bm, int64_t bn) {
        return p.G * ((p.Mg + bm - 1) / bm) * ((ncols + bn - 1) / bn);
    };
    constexpr int64_t kFill = 192;   // workgroups that count as filling the GPU
    if (p.Mg > 128)
        return tiles(256, 256) >= kFill ? GemmTile::M256_N256_W2x4 : GemmTile::M256_N128_W4x2;
    if (p.Mg > 64) {
        if (tiles(128, 256) >= kFill)
            return GemmTile::M128_N256_W2x4;
        return tiles(128, 128) >= kFill ? GemmTile::M128_N128_W2x2 : GemmTile::M128_N64_W2x2;
    }
    return GemmTile::M64_N128_W2x2;
}

// Fused tile: as for the GEMM, the tallest tile the group fills, then the
// widest that still gives about one workgroup per CU; among tiles whose LDS
// fits.  MDCN_FUSED_TILE=<0..3> overrides the choice (for tuning) when that
// tile fits.  Returns false when no tile fits.
bool choose_fused_tile(const Problem &p, int64_t chunk, FusedTile *out)
{
    auto fits = [&](FusedTile t) { return fused_lds_bytes(p, t) <= kLdsBytes; };
    if (const char *env = std::getenv("MDCN_FUSED_TILE")) {
        const int v = std::atoi(env);
        if (v >= 0 && v < kFusedTileCount && fits(static_cast<FusedTile>(v))) {
            *out = static_cast<FusedTile>(v);
            return true;
        }
    }
    const int64_t ncols = chunk * p.P;
    auto tiles = [&](int64_t bm, int64_t bn) {
        return p.G * ((p.Mg + bm - 1) / bm) * ((ncols + bn - 1) / bn);
    };
    constexpr int64_t kFill = 192;
    FusedTile pref;
    if (p.elem == 4)
        pref = FusedTile::M128_N64;     // fp32: half the channels per step; the
                                        // 8-wave tile with 256 registers a wave wins
    else if (p.Mg > 128)
        pref = tiles(256, 128) >= kFill ? FusedTile::M256_N128 : FusedTile::M256_N64;
    else
        pref = tiles(128, 128) >= kFill ? FusedTile::M128_N128 : FusedTile::M128_N64;
    const FusedTile order[] = {pref, p.Mg > 128 ? FusedTile::M256_N64 : FusedTile::M128_N64,
                               FusedTile::M128_N128, FusedTile::M128_N64};
    for (FusedTile t : order)
        if (fits(t)) {
            *out = t;
            return true;
        }
    return false;
}

}  // namespace

GemmTile gemm_tile_for(const Problem &p, int64_t chunk) { return choose_gemm_tile(p, chunk); }

size_t dtype_size(mdcn_dtype t)
{
    switch (t) {
    case MDCN_F32: return 4;
    case MDCN_F16: return 2;
    case MDCN_BF16: return 2;
    }
    return 0;
}

// [plugin guide §三]: stride and dilation components > 0, padding >= 0,
// group and deformable_group > 0; all five are required.
mdcn_status check_attrs(const int32_t stride[2], const int32_t padding[2],
                        const int32_t dilation[2], int32_t group, int32_t dgroup)
{
    if (!stride || !padding || !dilation)
        return MDCN_E_NULL;
    for (int i = 0; i < 2; ++i) {
        if (stride[i] <= 0 || dilation[i] <= 0 || padding[i] < 0)
            return MDCN_E_ATTR;
    }
    if (group <= 0 || dgroup <= 0)
        return MDCN_E_ATTR;
    return MDCN_OK;
}

mdcn_status derive_problem(const Attrs &a, mdcn_dtype dtype, const int64_t dims[16],
                           Problem *out)
{
    if (!dims || !out)
        return MDCN_E_NULL;
    if (dtype != MDCN_F32 && dtype != MDCN_F16 && dtype != MDCN_BF16)
        return MDCN_E_DTYPE;
    for (int i = 0; i < 16; ++i)
        if (dims[i] < 0)
            return MDCN_E_SHAPE;
    const int64_t *x = dims, *off = dims + 4, *msk = dims + 8, *w = dims + 12;
    Problem p{};
    p.dtype = dtype;
    p.elem = dtype_size(dtype);
    p.N = x[0]; p.C = x[1]; p.H = x[2]; p.W = x[3];
    p.Co = w[0]; p.kh = w[2]; p.kw = w[3];
    p.Ho = off[2]; p.Wo = off[3];
    if (p.N > kMaxPerImage)
        return MDCN_E_SHAPE;
    p.G = a.group; p.DG = a.dgroup;
    p.sh = a.sh; p.sw = a.sw; p.ph = a.ph; p.pw = a.pw; p.dh = a.dh; p.dw = a.dw;
    if (p.C == 0 || p.H == 0 || p.W == 0 || p.Co == 0 || p.kh == 0 || p.kw == 0)
        return MDCN_E_SHAPE;
    // Bindings of [plugin guide §四]: batch of offset and mask equals x's,
    // mask spatial dims equal offset's, offset has at least 2 channels.
    if (off[0] != p.N || msk[0] != p.N)
        return MDCN_E_SHAPE;
    if (msk[2] != off[2] || msk[3] != off[3])
        return MDCN_E_SHAPE;
    if (off[1] < 2)
        return MDCN_E_SHAPE;
    // Bindings that keep every read in bounds.
    if (p.kh > kMaxCoord || p.kw > kMaxCoord || mul(p.kh, p.kw) > kMaxPerImage)
        return MDCN_E_SHAPE;
    p.K = p.kh * p.kw;
    if (p.C % p.G != 0 || p.Co % p.G != 0 || p.C % p.DG != 0)
        return MDCN_E_SHAPE;
    if (mul(w[1], p.G) != p.C)
        return MDCN_E_SHAPE;
    if (off[1] != mul(2, p.DG, p.K) || msk[1] != mul(p.DG, p.K))
        return MDCN_E_SHAPE;
    p.Cg = p.C / p.G;
    p.Mg = p.Co / p.G;
    p.Cdg = p.C / p.DG;
    p.Kg = mul(p.Cg, p.K);
    if (p.Kg > kMaxPerImage)
        return MDCN_E_SHAPE;
    // Size limits of this implementation: 32-bit indexing within an image,
    // exact float anchors.
    if (p.H >= kMaxCoord || p.W >= kMaxCoord || p.Ho >= kMaxCoord || p.Wo >= kMaxCoord)
        return MDCN_E_SHAPE;
    p.P = p.Ho * p.Wo;
    const int64_t kp = round_up(p.Kg, 64);
    // image bytes (per-image buffer ranges are 31-bit) and offset groups per
    // group (the gather's per-workgroup geometry table holds them all)
    if (mul(mul(p.C, p.H, p.W), int64_t(p.elem)) > kMaxPerImage ||
        (p.Cg + p.Cdg - 1) / p.Cdg + 1 > 2048 || mul(p.Co, p.P) > kMaxPerImage ||
        mul(off[1], p.P) > kMaxPerImage || mul(p.G, p.P, kp) > kMaxPerImage ||
        mul(p.Co, kp) > kMaxPerImage)
        return MDCN_E_SHAPE;
    const int64_t amax_h = mul(std::max<int64_t>(0, p.Ho - 1), p.sh) + mul(p.kh - 1, p.dh);
    const int64_t amax_w = mul(std::max<int64_t>(0, p.Wo - 1), p.sw) + mul(p.kw - 1, p.dw);
    if (amax_h < 0 || amax_w < 0 || amax_h >= kMaxCoord || amax_w >= kMaxCoord ||
        p.ph >= kMaxCoord || p.pw >= kMaxCoord)
        return MDCN_E_SHAPE;
    *out = p;
    return MDCN_OK;
}

int64_t fused_offset_groups(const Problem &p)
{
    if (p.Cdg % p.Cg == 0)
        return 1;                                   // a group lies inside one offset group
    if (p.Cg % p.Cdg == 0)
        return p.Cg / p.Cdg;                        // offset groups tile the group
    return (p.Cg + p.Cdg - 1) / p.Cdg + 1;          // bound for a misaligned start
}

size_t fused_table_bytes(const Problem &p, int64_t bn)
{
    return size_t(fused_offset_groups(p)) * size_t(p.K) * size_t(bn) * 32;
}

size_t fused_lds_bytes(const Problem &p, FusedTile t)
{
    int64_t bm = 128, bn = 64;
    switch (t) {
    case FusedTile::M256_N128: bm = 256; bn = 128; break;
    case FusedTile::M128_N128: bm = 128; bn = 128; break;
    case FusedTile::M256_N64: bm = 256; bn = 64; break;
    case FusedTile::M128_N64: bm = 128; bn = 64; break;
    }
    return size_t(2 * (bm + bn) * 128) + fused_table_bytes(p, bn);
}

bool fused_eligible(const Problem &p)
{
    const int64_t se = 128 / int64_t(p.elem);      // K elements per 128-byte step
    const int64_t ev = 16 / int64_t(p.elem);       // elements per 16-byte chunk
    const int64_t img_bytes = p.C * p.H * p.W * int64_t(p.elem);
    FusedTile t;
    // (channel and step indices below 2^16 keep the kernel's division by
    // fp32 reciprocal exact)
    return p.Cg % se == 0 && p.Cdg % ev == 0 && img_bytes <= kMaxPerImage &&
           p.C < 65536 && p.Kg < 65536 && choose_fused_tile(p, 1, &t);
}

int64_t window_extent(int64_t tile, int64_t stride, int64_t k, int64_t dil, int64_t margin)
{
    return (tile - 1) * stride + (k - 1) * dil + 2 + 2 * margin;
}

int64_t window_flat_rows(int64_t Wo, int64_t n)
{
    return (Wo - 1 + n - 1) / Wo + 1;
}

bool window_tile_wide(WindowTile t)
{
    return int(t) >= kWindowWideFirst;
}

namespace {

void window_tile_dims(WindowTile t, int64_t *th, int64_t *tw)
{
    switch (t) {
    case WindowTile::H16_W16: *th = 16; *tw = 16; return;
    case WindowTile::H8_W32: *th = 8; *tw = 32; return;
    case WindowTile::H32_W8: *th = 32; *tw = 8; return;
    case WindowTile::FLAT: *th = 1; *tw = 256; return;
    case WindowTile::H8_W16: *th = 8; *tw = 16; return;
    case WindowTile::H16_W8: *th = 16; *tw = 8; return;
    case WindowTile::FLAT128: *th = 1; *tw = 128; return;
    }
    *th = 16;
    *tw = 16;
}

bool window_tile_flat(WindowTile t)
{
    return t == WindowTile::FLAT || t == WindowTile::FLAT128;
}

// pixels and output channels of one tile
int64_t window_tile_pixels(WindowTile t)
{
    return window_tile_wide(t) ? 128 : 256;
}
int64_t window_tile_channels(WindowTile t)
{
    return window_tile_wide(t) ? 512 : 256;
}

// Output rows and columns a tile's window must cover: the rectangle, or for
// a flat tile every column and the rows that its consecutive pixels starting
// anywhere in a row can reach.
void window_cover(const Problem &p, WindowTile t, int64_t *rows, int64_t *cols)
{
    if (window_tile_flat(t)) {
        *rows = window_flat_rows(p.Wo, window_tile_pixels(t));
        *cols = p.Wo;
        return;
    }
    window_tile_dims(t, rows, cols);
}

// Output pixels the tiles of one image and group cover (ragged edges).
int64_t window_padded_pixels(const Problem &p, WindowTile t)
{
    if (window_tile_flat(t)) {
        const int64_t n = window_tile_pixels(t);
        return (p.P + n - 1) / n * n;
    }
    int64_t th, tw;
    window_tile_dims(t, &th, &tw);
    return ((p.Ho + th - 1) / th) * th * ((p.Wo + tw - 1) / tw) * tw;
}

// Largest margin <= cap whose window fits (-1 when not even 0 fits).
int64_t window_margin_fit(const Problem &p, WindowTile t, int64_t cap)
{
    int64_t th, tw;
    window_cover(p, t, &th, &tw);
    const int64_t cap_px = window_tile_wide(t) ? kWindowPixelsWide : kWindowPixels;
    for (int64_t m = cap; m >= 0; --m) {
        const int64_t wr = window_extent(th, p.sh, p.kh, p.dh, m);
        const int64_t wc = window_extent(tw, p.sw, p.kw, p.dw, m);
        if (wr * wc <= cap_px && wc * 16 + 32 <= kWindowZeroBytes)
            return m;
    }
    return -1;
}

}  // namespace

// Tile: the fewest padded output pixels (ragged edges), then the widest
// margin, among tiles of the asked kind whose window fits with a margin >= 2.
// MDCN_WIN_TILE=<tile> and MDCN_WIN_MARGIN=<m> override (for tuning).
bool choose_window(const Problem &p, bool wide, WindowTile *tile, int64_t *margin)
{
    const int first = wide ? kWindowWideFirst : 0;
    const int count = wide ? kWindowWideCount : kWindowTileCount;
    int64_t cap = kWindowMaxMargin;
    if (const char *env = std::getenv("MDCN_WIN_MARGIN")) {
        const int v = std::atoi(env);
        if (v >= 0 && v <= 64)
            cap = v;
    }
    const int64_t min_margin = std::min<int64_t>(2, cap);
    if (const char *env = std::getenv("MDCN_WIN_TILE")) {
        const int v = std::atoi(env);
        if (v >= first && v < first + count) {
            const int64_t m = window_margin_fit(p, static_cast<WindowTile>(v), cap);
            if (m >= min_margin) {
                *tile = static_cast<WindowTile>(v);
                *margin = m;
                return true;
            }
        }
    }
    bool found = false;
    int64_t best_pad = 0, best_m = 0;
    for (int i = first; i < first + count; ++i) {
        const WindowTile t = static_cast<WindowTile>(i);
        const int64_t m = window_margin_fit(p, t, cap);
        if (m < min_margin)
            continue;
        const int64_t pad = window_padded_pixels(p, t);
        if (!found || pad < best_pad || (pad == best_pad && m > best_m)) {
            found = true;
            best_pad = pad;
            best_m = m;
            *tile = t;
            *margin = m;
        }
    }
    return found;
}

int64_t window_tiles_per_image(const Problem &p, WindowTile t)
{
    const int64_t m = window_tile_channels(t);
    return p.G * (window_padded_pixels(p, t) / window_tile_pixels(t)) * ((p.Mg + m - 1) / m);
}

namespace {

// Greedy fill of one run's units [0, U) (nch per tile) into `per` ranges of
// cost <= T, cost = 4 x chunks + seg_x4 x tiles touched; returns the number of
// units placed (U when T is feasible).  ends[k] receives each range's end.
int64_t split_fill(int64_t U, int64_t nch, int64_t per, int64_t seg_x4, int64_t T,
                   int64_t *ends)
{
    int64_t pos = 0;
    for (int64_t k = 0; k < per; ++k) {
        const int64_t start = pos;
        while (pos < U) {
            const int64_t touched = pos / nch - start / nch + 1;
            if (4 * (pos + 1 - start) + seg_x4 * touched > T)
                break;
            ++pos;
        }
        if (ends)
            ends[k] = pos;
    }
    return pos;
}

}  // namespace

bool window_split(int64_t tiles, int64_t nch, int64_t ncta, int64_t seg_cost_x4,
                  uint32_t *bounds)
{
    if (tiles <= 0 || nch <= 0 || ncta <= 0 || ncta > kWindowSlots || seg_cost_x4 < 0 ||
        tiles * nch > int64_t(0xffffffffll))
        return false;
    const int64_t ngrp = (ncta % 8 == 0 && tiles >= ncta) ? 8 : 1;
    const int64_t per = ncta / ngrp;
    int64_t ends[kWindowSlots];
    for (int64_t grp = 0; grp < ngrp; ++grp) {
        const int64_t tg0 = grp * tiles / ngrp, tg1 = (grp + 1) * tiles / ngrp;
        const int64_t U = (tg1 - tg0) * nch;
        // smallest feasible bound on the per-range cost
        int64_t lo = 0, hi = 4 * U + seg_cost_x4 * (tg1 - tg0);
        while (lo < hi) {
            const int64_t mid = lo + (hi - lo) / 2;
            if (split_fill(U, nch, per, seg_cost_x4, mid, nullptr) >= U)
                hi = mid;
            else
                lo = mid + 1;
        }
        split_fill(U, nch, per, seg_cost_x4, lo, ends);
        for (int64_t k = 0; k < per; ++k)
            bounds[grp * per + k] = uint32_t(tg0 * nch + (k ? ends[k - 1] : 0));
    }
    bounds[ncta] = uint32_t(tiles * nch);
    return true;
}

bool window_eligible(const Problem &p, bool wide)
{
    const int64_t img_bytes = p.C * p.H * p.W * int64_t(p.elem);
    WindowTile t;
    int64_t m;
    return p.elem == 2 && p.kh == 3 && p.kw == 3 && p.Cg % 16 == 0 && p.Cdg % p.Cg == 0 &&
           img_bytes <= kMaxPerImage && (!wide || p.Mg > 256) && choose_window(p, wide, &t, &m);
}

// The windowed kernel is the faster of the two MFMA paths when its tiles are
// nearly full: at least 7/8 of the padded output pixels x padded output
// channels of the chosen tiling are real (measured: 15% faster than the fused
// kernel at 100%, 4% at 89%; fewer than 256 channels per group waste rows of
// every tile).
bool window_preferred(const Problem &p)
{
    if (!window_eligible(p))
        return false;
    WindowTile t;
    int64_t m;
    choose_window(p, false, &t, &m);
    const int64_t pad_px = window_padded_pixels(p, t);
    const int64_t pad_m = ((p.Mg + 255) / 256) * 256;
    return 8 * p.Ho * p.Wo * p.Mg >= 7 * pad_px * pad_m;
}

// Small problems: one launch of the direct kernel costs less than the
// launches of the other paths (a few microseconds each) up to about 2^20
// multiply-adds.
bool direct_preferred(const Problem &p)
{
    return double(p.N) * double(p.Co) * double(p.P) * double(p.Cg) * double(p.K) <=
           double(kDirectMaxMacs);
}

mdcn_status choose_path(const Attrs &a, const Problem &p, Path *out)
{
    switch (a.path) {
    case MDCN_PATH_AUTO:
        *out = direct_preferred(p)      ? Path::Direct
               : (p.Cg == 1)            ? Path::Depthwise
               : window_preferred(p)   ? Path::Window
               : fused_eligible(p)     ? Path::Fused
                                       : Path::GatherGemm;
        return MDCN_OK;
    case MDCN_PATH_DIRECT:
        if (uint64_t(p.N) * uint64_t(p.Co) * uint64_t(p.P) > kDirectMaxOutputs)
            return MDCN_E_PATH;
        *out = Path::Direct;
        return MDCN_OK;
    case MDCN_PATH_WINDOW:
        if (!window_eligible(p))
            return MDCN_E_PATH;
        *out = Path::Window;
        return MDCN_OK;
    case MDCN_PATH_WINDOW_FP8:
        if (!window_eligible(p) && !window_eligible(p, true))
            return MDCN_E_PATH;
        *out = Path::WindowFp8;
        return MDCN_OK;
    case MDCN_PATH_FUSED:
        if (!fused_eligible(p))
            return MDCN_E_PATH;
        *out = Path::Fused;
        return MDCN_OK;
    case MDCN_PATH_GATHER_GEMM:
        *out = Path::GatherGemm;
        return MDCN_OK;
    case MDCN_PATH_GATHER_GEMM_FP8:
        *out = Path::GatherGemmFp8;
        return MDCN_OK;
    case MDCN_PATH_DEPTHWISE:
        if (p.Cg != 1)
            return MDCN_E_PATH;
        *out = Path::Depthwise;
        return MDCN_OK;
    }
    return MDCN_E_PATH;
}

mdcn_status make_plan(const Attrs &a, const Problem &p, size_t workspace_bytes,
                      bool default_sizing, Plan *out)
{
    Plan plan{};
    mdcn_status st = choose_path(a, p, &plan.path);
    if (st != MDCN_OK)
        return st;
    if (plan.path == Path::Direct) {
        plan.chunk = std::max<int64_t>(p.N, 1);    // one launch, no workspace
        *out = plan;
        return MDCN_OK;
    }
    if (plan.path == Path::Depthwise) {
        // The staged kernel reads each (offset group, tap, pixel)'s sampling
        // record (corner entry and weight factors), computed once per image
        // by a geometry kernel: 16 bytes each.  Chunks of images within a
        // 256 MiB budget.
        plan.chunk = std::max<int64_t>(p.N, 1);
        if (dw_default_entry(p) == 0) {
            *out = plan;                        // plain kernel: no workspace
            return MDCN_OK;
        }
        plan.geo_bytes_per_image = align_up(size_t(p.DG * p.K * p.P) * 16, kAlign);
        const int64_t img = int64_t(std::max<size_t>(plan.geo_bytes_per_image, 1));
        int64_t chunk = std::max<int64_t>(1, std::min<int64_t>(
            {std::max<int64_t>(p.N, 1), int64_t(kColumnBudget) / img, kMaxPerImage / img}));
        if (!default_sizing) {
            if (workspace_bytes < kAlign + size_t(img))
                return MDCN_E_WORKSPACE;
            chunk = std::max<int64_t>(1, std::min<int64_t>(
                chunk, int64_t((workspace_bytes - kAlign) / size_t(img))));
        }
        plan.chunk = chunk;
        plan.ws_bytes = size_t(chunk) * plan.geo_bytes_per_image;
        *out = plan;
        return MDCN_OK;
    }
    plan.Kp = round_up(p.Kg, 64);
    plan.wpack_off = 0;
    const bool windowed = plan.path == Path::Window || plan.path == Path::WindowFp8;
    if (plan.path == Path::Fused || windowed) {
        // Workspace: packed weight + the chunk's images in NHWC.  A chunk's
        // NHWC bytes stay below 2^31 (one buffer range) and within 512 MiB.
        plan.wpack_bytes = align_up(size_t(p.G * p.Mg * plan.Kp) * p.elem, kAlign);
        if (plan.path == Path::WindowFp8) {
            // E4M3 chunk layout, then the row scales
            plan.wscale_off = align_up(size_t(p.G * (p.Cg / 16) * p.Mg) *
                                           size_t(kWindowFp8ChunkBytesPerRow),
                                       kAlign);
            plan.wpack_bytes = plan.wscale_off + align_up(size_t(p.Co) * sizeof(float), kAlign);
        }
        plan.xt_bytes_per_image = align_up(size_t(p.H * p.W * p.C) * p.elem, kAlign);
        plan.col_bytes_per_image = 0;
        const int64_t img = int64_t(plan.xt_bytes_per_image);
        int64_t chunk = std::max<int64_t>(1, std::min<int64_t>(
            {std::max<int64_t>(p.N, 1), kMaxPerImage / img, int64_t(kFusedBudget) / img}));
        if (!default_sizing) {
            if (workspace_bytes < kAlign + plan.wpack_bytes + size_t(img))
                return MDCN_E_WORKSPACE;
            const int64_t fit =
                int64_t((workspace_bytes - kAlign - plan.wpack_bytes) / size_t(img));
            chunk = std::max<int64_t>(1, std::min(chunk, fit));
        }
        if (plan.path == Path::Fused && !choose_fused_tile(p, chunk, &plan.fused_tile))
            return MDCN_E_PATH;                 // fused_eligible said some tile fits
        plan.xt_off = plan.wpack_bytes;
        if (windowed) {
            // E4M3 on groups of more than 256 output channels: the wide
            // tiles (128 pixels x 512 channels; each sample is blended once
            // for all of them rather than once per 256), unless
            // MDCN_WIN_WIDE=0 or none fits
            plan.win_wide = false;
            if (plan.path == Path::WindowFp8 && p.Mg > 256) {
                const char *env = std::getenv("MDCN_WIN_WIDE");
                if (!(env && std::atoi(env) == 0))
                    plan.win_wide = choose_window(p, true, &plan.win_tile, &plan.win_margin);
            }
            if (!plan.win_wide && !choose_window(p, false, &plan.win_tile, &plan.win_margin))
                return MDCN_E_PATH;
            // the weight copies run 5 K steps ahead (the kernel's barrier
            // schedule needs exactly that); MDCN_WIN_CTAS=<n> caps the
            // workgroups (more tiles split between two of them)
            plan.win_lead = kWindowLead;
            plan.win_max_ctas = 0;
            if (const char *env = std::getenv("MDCN_WIN_CTAS")) {
                const int v = std::atoi(env);
                if (v > 0)
                    plan.win_max_ctas = v;
            }
            // a tile a workgroup touches costs about 4 chunks of main loop
            // (its prologue and epilogue), in quarter chunks (measured on the
            // OCDNet-like stage: 8, 12, 16, 20, 24, 32 -> 16 best)
            plan.win_seg_cost_x4 = 16;
            if (const char *env = std::getenv("MDCN_WIN_SEG_X4")) {
                const int v = std::atoi(env);
                if (v >= 0 && v <= 1024)
                    plan.win_seg_cost_x4 = v;
            }
            // MDCN_WIN_SPIN_LIMIT=<polls> shortens the bounded hand-over wait
            // (tests force the give-up report with it)
            plan.win_spin_limit = kWindowSpinLimit;
            if (const char *env = std::getenv("MDCN_WIN_SPIN_LIMIT")) {
                const long long v = std::atoll(env);
                if (v >= 0 && v <= (long long)kWindowSpinLimit)
                    plan.win_spin_limit = uint32_t(v);
            }
            // the chunk's offsets and masks are each one buffer range
            const int64_t om_img = 2 * p.DG * p.K * p.P * int64_t(p.elem);
            chunk = std::max<int64_t>(1, std::min<int64_t>(chunk, kMaxPerImage / std::max<int64_t>(om_img, 1)));
            // Partial-sum slots and flags for the chunk's tiles (one slot per
            // workgroup, at most kWindowSlots); with a given workspace, the
            // largest chunk whose layout fits.
            plan.win_tiles_per_image = window_tiles_per_image(p, plan.win_tile);
            auto layout = [&](int64_t c, Plan *pl) {
                pl->win_slots = std::min<int64_t>(kWindowSlots, c * pl->win_tiles_per_image);
                pl->part_off = align_up(pl->xt_off + size_t(c) * pl->xt_bytes_per_image, kAlign);
                pl->flag_off = pl->part_off + size_t(pl->win_slots) * kWindowSlotBytes;
                return pl->flag_off + align_up(size_t(pl->win_slots + 1) * 4, kAlign);
            };
            if (!default_sizing) {
                if (workspace_bytes < kAlign + layout(1, &plan))
                    return MDCN_E_WORKSPACE;
                int64_t lo = 1, hi = chunk;             // largest fitting chunk in [1, chunk]
                while (lo < hi) {
                    const int64_t mid = lo + (hi - lo + 1) / 2;
                    if (kAlign + layout(mid, &plan) <= workspace_bytes)
                        lo = mid;
                    else
                        hi = mid - 1;
                }
                chunk = lo;
            }
            plan.chunk = chunk;
            plan.ws_bytes = layout(chunk, &plan);
            plan.col_off = plan.ws_bytes;
            *out = plan;
            return MDCN_OK;
        }
        plan.chunk = chunk;
        plan.col_off = plan.xt_off + size_t(chunk) * plan.xt_bytes_per_image;
        plan.ws_bytes = plan.col_off;
        *out = plan;
        return MDCN_OK;
    }
    // FP8: one-byte operands, so a 128-byte K step is 128 elements; the row
    // scales follow the weight bytes
    const bool fp8 = plan.path == Path::GatherGemmFp8;
    const size_t op_elem = fp8 ? 1 : p.elem;
    if (fp8)
        plan.Kp = round_up(p.Kg, 128);
    plan.wpack_bytes = align_up(size_t(p.G * p.Mg * plan.Kp) * op_elem, kAlign);
    if (fp8) {
        plan.wscale_off = plan.wpack_bytes;
        plan.wpack_bytes += align_up(size_t(p.Co) * sizeof(float), kAlign);
    }
    plan.xt_bytes_per_image = align_up(size_t(p.H * p.W * p.C) * p.elem, kAlign);
    plan.col_bytes_per_image = align_up(size_t(p.G * p.P * plan.Kp) * op_elem, kAlign);
    // Default chunk: as many images as fit a 256 MiB column buffer, at least
    // one; also keep every launch's element count within 32-bit indexing.
    int64_t by_budget = int64_t(kColumnBudget / std::max<size_t>(plan.col_bytes_per_image, 1));
    // (byte offsets within one launch's columns must fit in 31 bits)
    int64_t by_index = kMaxPerImage /
                       std::max<int64_t>(p.G * std::max<int64_t>(p.P, 1) * plan.Kp * int64_t(op_elem), 1);
    int64_t chunk = std::max<int64_t>(1, std::min<int64_t>({std::max<int64_t>(p.N, 1),
                                                           by_budget, by_index}));
    const size_t per_image = plan.xt_bytes_per_image + plan.col_bytes_per_image;
    if (!default_sizing) {
        // kAlign bytes may be lost to aligning the caller's pointer
        if (workspace_bytes < kAlign + plan.wpack_bytes + per_image)
            return MDCN_E_WORKSPACE;
        int64_t fit = int64_t((workspace_bytes - kAlign - plan.wpack_bytes) / per_image);
        chunk = std::max<int64_t>(1, std::min(chunk, fit));
    }
    plan.chunk = chunk;
    plan.gemm_tile = choose_gemm_tile(p, chunk);
    plan.xt_off = plan.wpack_bytes;
    plan.col_off = plan.xt_off + size_t(chunk) * plan.xt_bytes_per_image;
    plan.ws_bytes = plan.col_off + size_t(chunk) * plan.col_bytes_per_image;
    // the caller's pointer is aligned up to kAlign inside the library
    *out = plan;
    return MDCN_OK;
}

size_t min_workspace(const Problem &p, const Plan &plan)
{
    (void)p;
    if (plan.path == Path::Direct)
        return 0;
    if (plan.path == Path::Depthwise)
        return plan.geo_bytes_per_image ? kAlign + plan.geo_bytes_per_image : 0;
    if (plan.path == Path::Window || plan.path == Path::WindowFp8) {
        const int64_t slots = std::min<int64_t>(kWindowSlots, plan.win_tiles_per_image);
        return kAlign + align_up(plan.wpack_bytes + plan.xt_bytes_per_image, kAlign) +
               size_t(slots) * kWindowSlotBytes + align_up(size_t(slots + 1) * 4, kAlign);
    }
    return kAlign + plan.wpack_bytes + plan.xt_bytes_per_image + plan.col_bytes_per_image;
}


size_t workspace_request(const Plan &plan)
{
    if (plan.ws_bytes == 0)
        return 0;
    return kAlign + plan.ws_bytes;
}

bool dw_entry_allowed(const Problem &p, int ent)
{
    const int ch = ent / int(p.elem);
    const size_t positions = size_t(p.H + 4) * size_t(p.W + 4);
    // one image's geometry (16 bytes per offset group, tap and pixel) is one
    // buffer range
    const double geo = double(p.DG) * double(p.K) * double(p.P) * 16.0;
    return ent >= int(p.elem) && ch >= 1 && p.Cdg % ch == 0 && geo <= double(kMaxPerImage) &&
           positions * size_t(ent) + 9 * size_t(ch) * sizeof(float) <= kLdsBytes;
}

int dw_default_entry(const Problem &p)
{
    for (int e : {16, 8, 4, 2})
        if (dw_entry_allowed(p, e))
            return e;
    return 0;
}

}  // namespace mdcn
