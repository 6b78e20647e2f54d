// Launch plans: pure host functions (no HIP calls) that fix the grid, the
// split-K factor and the workspace size of each kernel from the problem shape.
// The ABI layer validates arguments against them; the launchers execute them.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace w4 {

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---- M == 1 fused dequant-GEMV ---------------------------------------------
// A lane owns 16 consecutive columns (8 bytes of one packed row) and all 32
// rows of one K-block; 16 lanes cover a 256-column tile, the 4 lane groups of
// a wave take 4 different K-blocks.  A workgroup of `waves` waves covers one
// column tile and `blocks_per_wg` K-blocks; `splits` workgroups along K
// write partial sums to the workspace, summed by a second kernel.
struct GemvPlan {
    enum Kind { kEmpty = 0, kBiasOnly = 1, kFast = 2, kGeneric = 3 } kind;
    int64_t tiles = 0;          // column tiles (fast path)
    int64_t splits = 1;         // workgroups along K per column tile
    int64_t blocks_per_wg = 0;  // K-blocks per workgroup
    int waves = 1;              // waves per workgroup
    int64_t npad = 0;           // tiles * 256
    size_t workspace = 0;       // bytes
};

constexpr int kGemvTileCols = 256;
constexpr int kGemvGroups = 4;  // lane groups per wave

GemvPlan plan_gemv(int64_t K, int64_t N);

// ---- int8 head logits (last row) -------------------------------------------
// Same geometry as the GEMV: a lane owns 16 columns (16 bytes of a row) and
// 32 rows; 16 lanes make a 256-column tile; 4 lane groups per wave.
// kWhole: one workgroup of `waves` waves per 16 * lanes_per_row columns over
// all K = rows_per_lane * waves * 64 / lanes_per_row rows, one launch, no
// workspace.
struct HeadPlan {
    enum Kind { kEmpty = 0, kZero = 1, kRun = 2, kWhole = 3 } kind;
    int64_t tiles = 0, splits = 1, rows_per_wg = 0, npad = 0;
    int waves = 1;
    int rows_per_lane = 0, lanes_per_row = 8;
    size_t workspace = 0;
};

HeadPlan plan_head(int64_t K, int64_t N);

// ---- small-M matmul (M > 1) ----------------------------------------------
// A workgroup (4 waves) owns a 256-column tile, up to 64 rows of M (1..4
// MFMA m-tiles) and `blocks_per_wg` K-blocks; `mgroups` = ceil(M / 64).
struct SmallMPlan {
    enum Kind { kEmpty = 0, kBiasOnly = 1, kMfma = 2, kGeneric = 3 } kind;
    int64_t mtiles = 0;         // 16-row MFMA tiles per workgroup (1..4)
    int64_t mgroups = 1;        // 64-row groups of M
    int depth = 1;              // blocks of loads in flight ahead of the MFMAs
    int64_t tiles = 0;          // column tiles
    int64_t splits = 1;
    int64_t blocks_per_wg = 0;
    int64_t npad = 0;
    size_t workspace = 0;
};

SmallMPlan plan_small_m(int64_t M, int64_t K, int64_t N);

// ---- matmul on the K-major (prepacked) layout -------------------------------
// A workgroup of `threads` lanes holds `groups` column slots of
// `lanes_per_col` lanes; lane (slot, b) owns K-block b of its column.  The
// workgroup runs `passes` columns per slot (groups * passes columns in all)
// for `rows` rows of x; grid = ceil(N / columns) x ceil(M / rows).
struct KmajorPlan {
    enum Kind { kEmpty = 0, kBiasOnly = 1, kRun = 2 } kind;
    int rows = 1, passes = 1, groups = 1, lanes_per_col = 64, threads = 64;
    bool xc = true;  // activations in whole runs through LDS where the geometry allows
    int xs = 0;      // 2: two column slots read the activations once per workgroup
};

// even_cols: a workgroup's column count (groups * passes) must be even, so
// that the SwiGLU epilogue's column pairs stay within one workgroup.
KmajorPlan plan_kmajor(int64_t M, int64_t K, int64_t N, bool even_cols = false);

// ---- M >= 3 rows on the K-major layout: matrix cores, fp32 accuracy -----------
// Workgroup: 4 waves x nt tiles of 16 columns, the rows of one group of
// 16 mt rows (mt tiles of 16, mt = 1..4), quads_per_wg quads of 4 K-blocks;
// grid = col_wgs x splits x mgroups.  dq quads of loads in flight.  Needs
// K % 128 == 0 and K < 2^22.
struct X3Plan {
    // kRun: the split-K kernel (k_mm_x3, partial sums + reduce);
    // kFullK: one workgroup per 16 nt columns over all of K (k_mm_x3k)
    enum Kind { kNone = 0, kRun = 1, kFullK = 2 } kind = kNone;
    int mt = 1, nt = 1, dq = 2;
    int mb = 4, waves = 4;  // kFullK: rows built, waves per workgroup
    bool p3 = false;        // kFullK, mb == 4: the three parts share one MFMA
    int nqc = 0;            // kFullK: quads per wave when fixed at compile time (3 or 8), else 0
    int64_t col_wgs = 0, mgroups = 0, splits = 1, quads_per_wg = 0, npad = 0;
    size_t workspace = 0;
};

X3Plan plan_x3(int64_t M, int64_t K, int64_t N);

}  // namespace w4
