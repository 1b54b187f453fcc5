// plan.h -- host-side problem derivation, validation and execution planning
// for the modulated deformable convolution forward.  Pure host C++: nothing
// here touches the GPU, so every rule can be exercised without one.
#pragma once

#include <cstddef>
#include <cstdint>

#include "mdcn.h"

namespace mdcn {

// The five attributes of the operator, kept as int64
// [plugin guide §三: stride, padding, dilation, group, deformable_group].
struct Attrs {
    int64_t sh, sw;   // stride
    int64_t ph, pw;   // padding
    int64_t dh, dw;   // dilation
    int64_t group;
    int64_t dgroup;   // deformable_group
    mdcn_path path;
};

// Everything one forward needs to know about its shapes.
struct Problem {
    mdcn_dtype dtype;
    size_t elem;                 // bytes per element
    int64_t N, C, H, W;          // x
    int64_t Co, kh, kw;          // weight [Co, C/group, kh, kw]
    int64_t Ho, Wo;              // from offset dims 2, 3 [plugin guide §二]
    int64_t G, DG;               // group, deformable_group
    int64_t Cg, Mg, Cdg;         // C/G, Co/G, C/DG
    int64_t K, Kg, P;            // kh*kw, Cg*K, Ho*Wo
    int64_t sh, sw, ph, pw, dh, dw;
};

enum class Path { GatherGemm, Depthwise, Fused, Window, Direct, GatherGemmFp8, WindowFp8 };

// The windowed kernel's E4M3 weight: per group and 16-channel chunk, 144 bytes
// per output channel in three regions -- taps 0-3 [2 halves][2 parts][Mg][16
// bytes] (part 0: taps 0 and 1, part 1: taps 2 and 3), taps 4-7 likewise,
// tap 8 [2 halves][Mg][8 bytes] -- each 8-byte piece the E4M3 values of
// channels 8h..8h+7 of the chunk at one tap.
constexpr int64_t kWindowFp8ChunkBytesPerRow = 144;

// Workgroup tile of the GEMM (rows of the packed weight x columns) and its
// wave grid; every wave owns a block of 32x32 accumulator tiles.
enum class GemmTile : int {
    M256_N256_W2x4 = 0,
    M256_N128_W4x2 = 1,
    M128_N256_W2x4 = 2,
    M128_N128_W2x2 = 3,
    M128_N64_W2x2 = 4,
    M64_N128_W2x2 = 5,
};
constexpr int kGemmTileCount = 6;

// Workgroup tile of the fused gather-GEMM.
// (2 x 2 consumer waves plus producer waves.)
enum class FusedTile : int {
    M256_N128 = 0,
    M128_N128 = 1,
    M256_N64 = 2,
    M128_N64 = 3,
};
constexpr int kFusedTileCount = 4;

// Output-pixel tile (rows x columns) of the windowed fused kernel: 256
// pixels x 256 output channels, or -- the wide tiles of the E4M3 variant on
// groups of more than 256 output channels -- 128 pixels x 512 channels.
enum class WindowTile : int {
    H16_W16 = 0,
    H8_W32 = 1,
    H32_W8 = 2,
    FLAT = 3,        // 256 consecutive output pixels in raster order (narrow images)
    H8_W16 = 4,      // wide tiles
    H16_W8 = 5,
    FLAT128 = 6,     // 128 consecutive output pixels in raster order
};
constexpr int kWindowTileCount = 4;      // tiles 0..3: 256 pixels
constexpr int kWindowWideFirst = 4;      // tiles 4..6: 128 pixels x 512 channels
constexpr int kWindowWideCount = 3;
constexpr int kWindowPixels = 1280;      // input positions one LDS window can hold
constexpr int kWindowPixelsWide = 1024;  // (wide tiles: their weight slots take the rest)
constexpr int kWindowZeroBytes = 1024;   // zeroed LDS after each window (>= 16*columns + 32)
constexpr int64_t kWindowMaxMargin = 8;  // default offset margin around the anchors
constexpr int kWindowLead = 5;           // weight copies issued this many K steps ahead
constexpr int64_t kDirectMaxMacs = int64_t(1) << 20;   // automatic direct path, at most
constexpr uint64_t kDirectMaxOutputs = 0xffffff00ull;  // one 32-bit thread index
constexpr int64_t kWindowSlots = 256;    // partial-sum slots at most (one per workgroup)
constexpr size_t kWindowSlotBytes = size_t(256) * 256 * 4;   // fp32 256 x 256 tile
// Polls of a partial-sum flag before the waiting workgroup gives up (about
// 4 s at 2 GHz with a 128-cycle sleep between polls): the status word after
// the flags is then set to kWindowGaveUp and the tile's output to NaN.
constexpr uint32_t kWindowSpinLimit = 1u << 25;
constexpr uint32_t kWindowGaveUp = 1u;

// Workspace layout (all offsets 256-byte aligned):
//   gather + GEMM: [packed weight: G x Mg x Kp] [x in NHWC: chunk images] [columns: G x chunk*P x Kp]
//   FP8:           [E4M3 weight: Co x Kp bytes] [row scales: Co floats] [x in NHWC: chunk images]
//                  [E4M3 columns: G x chunk*P x Kp bytes], Kp a multiple of 128
//   fused:         [packed weight: G x Mg x Kp] [x in NHWC: chunk images]
//   window:        [packed weight] [x in 8-channel blocks: chunk images]
//                  [partial sums: slots x 256 KiB] [flags: slots x 4 bytes] [status: 4 bytes]
//   window FP8:    as window, with the packed weight replaced by the E4M3 chunk
//                  layout (G x Cg/16 x 144 x Mg bytes) and the Co fp32 row scales
//   depthwise:     [sampling geometry: chunk images x DG x K x 5 x P words]
struct Plan {
    Path path;
    int64_t chunk;               // images per pass through gather + GEMM
    int64_t Kp;                  // contraction length padded to 128 bytes (64 or 32 elements; FP8: 128)
    size_t wpack_off, wpack_bytes;   // (FP8: the weight bytes and the row scales after them)
    size_t wscale_off;           // FP8 paths: offset of the Co fp32 row scales in the weight area
    size_t xt_off, xt_bytes_per_image;
    size_t col_off, col_bytes_per_image;
    size_t geo_bytes_per_image;  // depthwise: sampling geometry of one image (0: none)
    size_t ws_bytes;             // bytes this plan uses
    GemmTile gemm_tile;
    FusedTile fused_tile;
    WindowTile win_tile;
    int64_t win_margin;          // window: pixels of margin around the tile's anchors
    bool win_wide;               // window FP8: 128-pixel x 512-channel tiles
    int win_lead;                // window: K steps the weight copies run ahead (5)
    int64_t win_tiles_per_image; // window: output tiles (256 x 256) of one image, all groups
    int64_t win_slots;           // window: partial-sum slots
    int64_t win_max_ctas;        // window: cap on the workgroups (0: none; tuning and tests)
    int64_t win_seg_cost_x4;     // window: cost of one tile segment, quarter chunks
    uint32_t win_spin_limit;     // window: polls of a hand-over flag before giving up
    size_t part_off, flag_off;   // window: offsets of the partial sums and the flags
                                 // (the status word follows the win_slots flags)
};

constexpr size_t kColumnBudget = size_t(256) << 20;   // default column-buffer cap
constexpr size_t kAlign = 256;                         // workspace sub-buffer alignment
constexpr size_t kFusedBudget = size_t(512) << 20;    // default NHWC chunk cap (fused)
constexpr int64_t kMaxCoord = int64_t(1) << 24;        // spatial extents and anchors
constexpr size_t kLdsBytes = size_t(160) << 10;        // LDS of one gfx950 workgroup

size_t dtype_size(mdcn_dtype t);
// GEMM tile for a gather + GEMM chunk of `chunk` images (MDCN_GEMM_TILE overrides).
GemmTile gemm_tile_for(const Problem &p, int64_t chunk);
// Depthwise: the widest LDS entry (bytes of channels per plane position) the
// staged kernel can use for this problem -- its channels share an offset
// group and the zero-ringed plane fits in LDS -- or 0 when none can.
int dw_default_entry(const Problem &p);
// Whether entry width `ent` is usable for this problem.
bool dw_entry_allowed(const Problem &p, int ent);
// Whether the fused gather-GEMM can run this problem: channel blocks that
// align with its 128-byte K steps and 16-byte chunks, and some tile whose LDS
// (operand stages plus geometry table) fits.
bool fused_eligible(const Problem &p);
// Offset groups that one group's channels can span (an upper bound where the
// group and offset-group sizes divide neither way).
int64_t fused_offset_groups(const Problem &p);
// Bytes of the fused kernel's per-tile geometry table for a BN-column tile:
// 32 bytes per (offset group, tap, column).
size_t fused_table_bytes(const Problem &p, int64_t bn);
// Operand stages plus geometry table of a fused tile.
size_t fused_lds_bytes(const Problem &p, FusedTile t);
// Window rows (or columns) that a tile of `tile` output rows (columns) needs:
// its anchors for every tap, both bilinear corners, and `margin` pixels on
// each side.
int64_t window_extent(int64_t tile, int64_t stride, int64_t k, int64_t dil, int64_t margin);
// Whether the windowed fused kernel can run this problem: fp16/bf16, 3x3
// kernels, C/group a multiple of 16 inside one offset group, and some tile
// (wide: some wide tile, on groups of more than 256 output channels) whose
// window (with a margin of at least 2) fits in LDS.
bool window_eligible(const Problem &p, bool wide = false);
// Tile and margin for the windowed kernel among the 256-pixel tiles, or
// (wide) the 128-pixel ones (false when none fits).
bool choose_window(const Problem &p, bool wide, WindowTile *tile, int64_t *margin);
// Whether a tile is one of the wide (128-pixel x 512-channel) tiles.
bool window_tile_wide(WindowTile t);
// Output tiles of one image (all groups) for a window tile shape.
int64_t window_tiles_per_image(const Problem &p, WindowTile t);
// Output rows a flat tile of n consecutive pixels (of rows Wo wide) can span.
int64_t window_flat_rows(int64_t Wo, int64_t n);

// Split the windowed kernel's (tile, chunk) units over `ncta` workgroups
// (ncta <= kWindowSlots): bounds[j]..bounds[j+1] is the range of workgroup
// slot j, slots ordered run by run (the tiles are first cut into 8 runs of
// whole tiles, one per XCD, when ncta is a multiple of 8 and tiles >= ncta).
// Within a run the ranges are contiguous and chosen to even out
// chunks + seg_cost x (tiles touched): each tile a workgroup touches costs a
// prologue and an epilogue.  Empty ranges only come last in a run.  Returns
// false when the sizes do not fit (more than 2^32 units).
bool window_split(int64_t tiles, int64_t nch, int64_t ncta, int64_t seg_cost_x4,
                  uint32_t *bounds);
mdcn_status check_attrs(const int32_t stride[2], const int32_t padding[2],
                        const int32_t dilation[2], int32_t group, int32_t dgroup);
mdcn_status derive_problem(const Attrs &a, mdcn_dtype dtype, const int64_t dims[16],
                           Problem *out);
mdcn_status choose_path(const Attrs &a, const Problem &p, Path *out);
// Plan for a given workspace size; with default_sizing the plan uses the
// library's default chunking regardless of workspace_bytes.
mdcn_status make_plan(const Attrs &a, const Problem &p, size_t workspace_bytes,
                      bool default_sizing, Plan *out);
size_t min_workspace(const Problem &p, const Plan &plan);
// Bytes to ask the caller for: the plan's layout plus alignment slack.
size_t workspace_request(const Plan &plan);

}  // namespace mdcn
