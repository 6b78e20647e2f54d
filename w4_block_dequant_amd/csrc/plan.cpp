// Launch plans (pure host code, no HIP calls; see plan.h).
#include "plan.h"

#include <stdlib.h>

namespace w4 {
namespace {

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Optional tuning overrides, read once (0 = automatic).
int64_t env_int(const char *name) {
    const char *v = getenv(name);
    return v ? atoll(v) : 0;
}
int64_t env_int_or(const char *name, int64_t unset) {
    const char *v = getenv(name);
    return v ? atoll(v) : unset;
}

// partial planes part[splits][rows][npad] (fp32)
size_t splitk_bytes(int64_t splits, int64_t npad, int64_t rows) {
    if (splits <= 1) return 0;
    return (size_t)splits * rows * npad * 4;
}

// Pick the number of K-blocks each lane group takes: one, unless that makes
// more workgroups than are useful (they only add partial-sum traffic).
int64_t blocks_per_group(int64_t tiles, int64_t units, int slots) {
    constexpr int64_t kTargetWgs = 2048;
    int64_t t = 1;
    while (tiles * cdiv(units, (int64_t)slots * t) > kTargetWgs && t < 64) t *= 2;
    return t;
}

}  // namespace

GemvPlan plan_gemv(int64_t K, int64_t N) {
    GemvPlan p{};
    if (N == 0) {
        p.kind = GemvPlan::kEmpty;
        return p;
    }
    if (K == 0) {
        p.kind = GemvPlan::kBiasOnly;
        return p;
    }
    if (N % 16 != 0) {
        p.kind = GemvPlan::kGeneric;
        return p;
    }
    static const int64_t env_waves = env_int("W4_GEMV_WAVES");
    static const int64_t env_t = env_int("W4_GEMV_BLOCKS_PER_GROUP");
    p.kind = GemvPlan::kFast;
    p.waves = (env_waves == 1 || env_waves == 2 || env_waves == 4) ? (int)env_waves : 4;
    const int slots = p.waves * kGemvGroups;
    const int64_t NB = K / 32;
    p.tiles = cdiv(N, kGemvTileCols);
    p.npad = p.tiles * kGemvTileCols;
    const int64_t t = env_t > 0 ? env_t : blocks_per_group(p.tiles, NB, slots);
    p.blocks_per_wg = (int64_t)slots * t;
    p.splits = cdiv(NB, p.blocks_per_wg);
    p.workspace = splitk_bytes(p.splits, p.npad, 1);
    return p;
}

HeadPlan plan_head(int64_t K, int64_t N) {
    HeadPlan p{};
    if (N == 0) {
        p.kind = HeadPlan::kEmpty;
        return p;
    }
    if (K == 0) {
        p.kind = HeadPlan::kZero;
        return p;
    }
    // The whole-K kernel wherever K is 256, 512, 768 or 1024 (L = K / 64 rows
    // per lane): 16 waves per 256 columns (16 lanes per row) where that forms
    // at least 128 workgroups, else 8 waves per 128 columns (8 lanes per row).
    // GPT-2's 768 x 50257 (8 cold copies read in turn, us per head for
    // ldq 50257 / 50272): split-K kernel and its reduce 18.9 / 15.9; whole-K
    // with (lanes per row, waves) = (8, 8) 14.5 / 12.8, (4, 8) 20.3 / 18.3,
    // (16, 8) 12.3 / 10.9, (8, 16) 14.1 / 12.8, (8, 4) 15.8 / 14.4, (4, 16)
    // 20.8 / 19.3, (16, 16) 11.4 / 10.2: wider rows per instruction win.
    // W4_HEAD_WHOLE=0: the split-K kernel always.
    static const int64_t env_whole = env_int_or("W4_HEAD_WHOLE", 1);
    const int64_t L = K / 64;
    if (env_whole != 0 && K % 64 == 0 && (L == 4 || L == 8 || L == 12 || L == 16) &&
        N >= 128 * 128 && N < ((int64_t)1 << 31)) {
        const bool wide = N >= 128 * 256;
        p.kind = HeadPlan::kWhole;
        p.rows_per_lane = (int)L;
        p.lanes_per_row = wide ? 16 : 8;
        p.waves = wide ? 16 : 8;
        p.workspace = 0;
        return p;
    }
    static const int64_t env_waves = env_int("W4_HEAD_WAVES");
    p.kind = HeadPlan::kRun;
    p.waves = (env_waves == 1 || env_waves == 2 || env_waves == 4) ? (int)env_waves : 1;
    const int slots = p.waves * kGemvGroups;
    const int64_t RB = cdiv(K, 32);
    p.tiles = cdiv(N, kGemvTileCols);
    p.npad = p.tiles * kGemvTileCols;
    const int64_t t = blocks_per_group(p.tiles, RB, slots);
    p.rows_per_wg = (int64_t)slots * t * 32;
    p.splits = cdiv(K, p.rows_per_wg);
    p.workspace = splitk_bytes(p.splits, p.npad, 1);
    return p;
}

SmallMPlan plan_small_m(int64_t M, int64_t K, int64_t N) {
    SmallMPlan p{};
    if (N == 0 || M == 0) {
        p.kind = SmallMPlan::kEmpty;
        return p;
    }
    if (K == 0) {
        p.kind = SmallMPlan::kBiasOnly;
        return p;
    }
    if (N % 8 != 0) {
        p.kind = SmallMPlan::kGeneric;
        return p;
    }
    static const int64_t env_wgs = env_int("W4_MFMA_TARGET_WGS");
    const int64_t target = env_wgs > 0 ? env_wgs : 512;
    p.kind = SmallMPlan::kMfma;
    p.mgroups = cdiv(M, 64);
    p.mtiles = cdiv(M < 64 ? M : 64, 16);
    p.tiles = cdiv(N, 256);
    p.npad = p.tiles * 256;
    const int64_t NB = K / 32;
    int64_t splits = cdiv(target, p.tiles * p.mgroups);
    if (splits > NB) splits = NB;
    if (splits < 1) splits = 1;
    p.blocks_per_wg = cdiv(NB, splits);
    p.splits = cdiv(NB, p.blocks_per_wg);
    p.workspace = splitk_bytes(p.splits, p.npad, M);
    // prefetch depth: enough MFMA work in flight to cover memory latency (one
    // block of MFMAs is 8 * mtiles per wave), without idle ring steps
    static const int64_t env_d = env_int("W4_MFMA_DEPTH");
    const int max_d = p.mtiles <= 2 ? 3 : 2;
    p.depth = 1;
    for (int d = max_d; d >= 2; --d)
        if (p.blocks_per_wg % d == 0 || p.blocks_per_wg > 4 * d) {
            p.depth = d;
            break;
        }
    if (env_d >= 1 && env_d <= max_d) p.depth = (int)env_d;
    return p;
}

KmajorPlan plan_kmajor(int64_t M, int64_t K, int64_t N, bool even_cols) {
    KmajorPlan p{};
    if (N == 0 || M == 0) {
        p.kind = KmajorPlan::kEmpty;
        return p;
    }
    if (K == 0) {
        p.kind = KmajorPlan::kBiasOnly;
        return p;
    }
    p.kind = KmajorPlan::kRun;
    p.rows = M >= 4 ? 4 : (M >= 2 ? (M == 2 ? 2 : 4) : 1);
    const int64_t NB = K / 32;
    // the smallest workgroup whose lanes split evenly into whole columns of blocks
    int threads = 0;
    for (int w = 1; w <= 4; ++w)
        if ((64 * w) % NB == 0) {
            threads = 64 * w;
            break;
        }
    // (Always, for 17 to 32 blocks: the general branch below would give
    // K = 1024 64-thread workgroups of two 32-lane column slots, a layout
    // that produced wrong results in parity tests and is not used.)
    if (p.rows <= 2 && NB > 16 && NB <= 32) {
        // 17 to 32 blocks: one 32-lane half per column (the lanes past NB
        // idle), whose sum stays in registers and is stored by its last
        // lane: no LDS and no barrier for the sums.  GPT-2's K = 768.
        p.threads = 256;
        p.lanes_per_col = 32;
        p.groups = 8;
    } else if (threads) {
        p.threads = threads;
        // a column needs at least `rows` lanes for the final per-output sums;
        // for very short K the extra lanes idle (NB < 4 only)
        int lanes = (int)NB;
        while (lanes < p.rows) lanes *= 2;
        p.lanes_per_col = lanes;
        p.groups = threads / lanes;
    } else {  // no exact fit within 256 lanes: one column slot, lanes loop over blocks
        const int64_t lanes = NB < 256 ? NB : 256;
        p.threads = (int)(cdiv(lanes, 64) * 64);
        p.lanes_per_col = p.threads;
        p.groups = 1;
    }
    static const int64_t env_p = env_int("W4_KMAJOR_PASSES");
    static const int allowed1[] = {16, 12, 8, 6, 4, 3, 2, 1};
    static const int allowed2[] = {4, 2, 1};
    static const int allowed4[] = {2, 1};
    const int *allowed = p.rows == 1 ? allowed1 : p.rows == 2 ? allowed2 : allowed4;
    const int nallowed = p.rows == 1 ? 8 : p.rows == 2 ? 3 : 2;
    // Workgroup count: whole multiples of the 256 compute units keep every CU
    // equally loaded (all workgroups are resident at once), which measures
    // better than any other choice; among those, up to 8 passes per lane.
    // Otherwise: enough workgroups to fill the chip, about 512 column groups.
    const int64_t want = env_p > 0 ? env_p : N / ((int64_t)p.groups * 512);
    p.passes = 1;
    bool found = false;
    if (env_p <= 0 && p.rows == 2) {
        // Two rows: the most passes that leave two workgroups per compute
        // unit, else one, whether or not the count divides evenly (with the
        // workgroup-shared activations, us per launch: 3072 x 3072 2 passes
        // 4.42 against 4.81 with 4; 3072 x 9216, 3072 x 16384 and 8192 x
        // 3072 keep 4: 7.97 / 11.0 / 7.47 against 8.12 / 11.7 / 9.75 with 2)
        for (int64_t min_wgs = 512; min_wgs >= 256 && !found; min_wgs /= 2)
            for (int i = 0; i < nallowed && !found; ++i) {
                const int P = allowed[i];
                if (cdiv(N, (int64_t)p.groups * P) * cdiv(M, p.rows) >= min_wgs) {
                    p.passes = P;
                    found = true;
                }
            }
    }
    if (env_p <= 0) {
        // at least two workgroups per compute unit where that is possible
        // (3072 x 3072 at M = 1: 3 passes, 512 workgroups, 3.95 -> 3.92 us
        // against 6 passes and 256)
        for (int pass2 = 0; pass2 < 2 && !found; ++pass2)
            for (int i = 0; i < nallowed && !found; ++i) {
                const int P = allowed[i];
                const int64_t wgs = cdiv(N, (int64_t)p.groups * P) * cdiv(M, p.rows);
                if (P <= 8 && wgs >= (pass2 ? 256 : 512) && wgs % 256 == 0) {
                    p.passes = P;
                    found = true;
                }
            }
    }
    for (int i = 0; i < nallowed && !found; ++i)
        if (allowed[i] <= want) {
            p.passes = allowed[i];
            found = true;
        }
    // Small matrices that fall to one pass: two passes halve the activation
    // loads per column and cost nothing while at least 128 workgroups remain
    // (GPT-2 768 x 2304, 768 x 3072, 3072 x 768: 3.6-3.9 -> 3.3-3.4 us; at
    // 768 x 768 two passes would leave 48 workgroups and are slower)
    // Not where two column slots can share one read of the activations at
    // one pass with at least 256 workgroups (below): GPT-2 3072 x 768 3.45 us
    // with two passes, 3.28 with one pass and the shared activations.
    const bool shared1 = p.groups == 2 && p.lanes_per_col == NB && NB % 8 == 0 &&
                         p.threads == 2 * p.lanes_per_col && cdiv(N, 2) >= 256;
    if (env_p <= 0 && p.rows == 1 && p.passes == 1 && !shared1 &&
        cdiv(N, (int64_t)p.groups * 2) * cdiv(M, p.rows) >= 128)
        p.passes = 2;
    // an odd column count only arises with one column slot and 1 or 3 passes
    if (even_cols && (p.groups * p.passes) % 2 != 0) p.passes = p.passes == 3 ? 4 : 2;
    // Activations in whole 1 KB runs through LDS where the lane layout allows
    // it (one row, one block per lane) and the matrix fills the chip with
    // workgroups: 3.8B M=1 pass 0.905 -> 0.838 ms (3072 x 9216: 7.09 -> 6.40
    // us, 3072 x 16384: 8.86 -> 8.38, 8192 x 3072: 6.75 -> 6.21, 3072 x 3072
    // unchanged); the GPT-2 matrices (48-144 workgroups, 3.2-3.4 us, bound by
    // launch latency) lose 0.05-0.15 us to the extra LDS round trip.
    // W4_KMAJOR_XC=1 forces it on, 2 off.
    static const int64_t env_xc = env_int("W4_KMAJOR_XC");
    const int64_t wgs = cdiv(N, (int64_t)p.groups * p.passes) * cdiv(M, p.rows);
    p.xc = env_xc == 1 || (env_xc != 2 && wgs >= 256);
    // Two column slots per workgroup with one block per lane (K = 3072: 96
    // lanes per column, 192 threads): the workgroup reads the activations
    // once and shares them through LDS (xs), and then 4 passes where they
    // leave at least 512 workgroups, else 3, 2 or 1 (3.8B M=1 shapes, us per
    // launch: 3072 x 9216 4 passes 5.62 against 5.79 with 6; 3072 x 16384 4
    // passes 7.89 against 8.53 with 8; 3072 x 3072 3 passes 3.60; the M=1
    // pass 0.733 -> 0.711 ms), a multiple of 256 workgroups first (below).  Two rows keep their passes (M=2 pass 1.153
    // -> 1.079 ms).  Four rows stay on the matrix cores: with the shared
    // activations the four-row GEMV is bound by its arithmetic (M=4 pass
    // 2.40 ms against 1.50).  K = 8192 keeps one 256-lane column slot per
    // workgroup: two slots in 512 threads were slower (8192 x 3072 at M = 1:
    // 5.67 against 5.47 us; M = 2: 10.3 against 7.5).  W4_KMAJOR_XS=0 turns
    // it off.
    static const int64_t env_xs = env_int_or("W4_KMAJOR_XS", 1);
    // passes for the shared mode (0: none qualifies): the most, up to 4, that
    // leave at least 512 workgroups, preferring a count that is a multiple of
    // the 256 compute units (3072 x 9216: 3 passes, 1536 workgroups, 5.55 us
    // against 5.65 with 4 passes and 4.5 workgroups per compute unit;
    // interleaved runs in one session)
    auto shared_passes = [&]() -> int {
        if (env_p > 0 || p.rows != 1) return p.passes;
        static const int cand[] = {4, 3, 2, 1};
        for (int even = 1; even >= 0; --even)
            for (int P : cand) {
                const int64_t wgs = cdiv(N, 2 * (int64_t)P);
                if (wgs >= 512 && (!even || wgs % 256 == 0)) return P;
            }
        return cdiv(N, 2) >= 256 ? 1 : 0;  // small N: one pass, still shared
    };
    if (p.xc && env_xs != 0 && p.rows <= 2 && p.groups == 2 &&
        p.lanes_per_col == NB && p.lanes_per_col % 8 == 0 && p.threads == 2 * p.lanes_per_col) {
        const int P = shared_passes();
        if (P > 0) {
            p.passes = P;
            p.xs = 2;
        }
    }
    return p;
}

X3Plan plan_x3(int64_t M, int64_t K, int64_t N) {
    X3Plan p;
    // From 3 rows on the matrix cores beat the GEMV, whose lanes then hold
    // 4 rows of activations in registers (measured on the 3.8B shapes: 64
    // against 116 us per layer at M = 3 and 4; at M = 2 the GEMV still wins
    // on three shapes of four).
    static const int64_t env_min = env_int("W4_X3_MIN_ROWS");
    const int64_t min_rows = env_min >= 2 ? env_min : 3;
    // K < 2^22: activation offsets within a row group stay below 2^32 bytes
    if (M < min_rows || K <= 0 || N <= 0 || K % 128 != 0 || K >= ((int64_t)1 << 22)) return p;
    const int64_t NQ = K / 128;
    // Up to 16 rows, the whole-K kernel: one launch and no partial sums, as
    // long as its workgroups (one per 16 nt columns) fill the chip.  Measured
    // on the 3.8B shapes (kernel trace, us per matmul for 3072x9216 /
    // 3072x3072 / 3072x16384 / 8192x3072): at M = 8 14.8 / 6.9 / 17.2 / 14.4
    // against 16.3 / 10.7 / 24.1 / 16.5 for the split-K kernel and its
    // reduce; at M = 16 19.0 / 8.1 / 20.2 / 18.0 against 18.2 / 11.2 / 24.8 /
    // 17.9.  W4_X3K=n caps it at n rows (0 turns it off).
    static const int64_t env_k = env_int_or("W4_X3K", 16);
    static const int64_t env_tpw = env_int("W4_X3K_TPW");
    static const int64_t env_waves = env_int("W4_X3K_WAVES");
    // Past 16 rows: row groups of 16 (grid.y) of the same kernel, each
    // streaming the matrix again (from the caches), on small matrices (at
    // most 2^22 weights), where the split-K kernel's second launch costs
    // more than converting each code once per 16 rows: GPT-2 body (48
    // matmuls) at M = 17 / 32 / 58 / 65 / 96 / 128: 0.357 / 0.377 / 0.375 /
    // 0.447 / 0.467 / 0.503 -> 0.307 / 0.317 / 0.311 / 0.322 / 0.415 / 0.455
    // ms.  On the 3.8B matrices the split-K kernel's 64-row tiles, which
    // convert each code once for 64 rows, stay ahead (M = 17 / 58: 2.72 /
    // 4.72 against 3.32 / 5.88 ms per pass).  W4_X3K_ROWS=n moves the row
    // limit (0: never past 16 rows).
    static const int64_t env_rows = env_int_or("W4_X3K_ROWS", 128);
    const bool row_groups = M > 16 && M <= env_rows && K * N <= ((int64_t)1 << 22);
    if (env_k != 0 && (M <= 16 ? M <= env_k : row_groups)) {
        // two column tiles per wave (each activation split serves 32 columns)
        // from 5 rows on, where that still leaves 512 workgroups: 3072x16384
        // at M = 8 19.9 -> 17.2 us, at M = 16 25.4 -> 20.2; at M = 4 and on
        // 3072x9216 (288 workgroups) one tile is ahead
        int64_t tpw = (M > 4 && cdiv(N, 32) >= 512) ? 2 : 1;
        if (env_tpw == 1 || env_tpw == 2) tpw = env_tpw;
        if (tpw == 2 && cdiv(N, 32) < 128) tpw = 1;
        const int64_t wgs = cdiv(N, 16 * tpw);
        const int64_t mgroups = cdiv(M, 16);
        // Narrow matrices form few workgroups; the whole-K kernel with more
        // waves (below) still beats the split-K kernel and its reduce launch
        // from 32 workgroups on (GPT-2 body, 12 x 4 matmuls: M = 4 0.260 ->
        // 0.183 ms, M = 16 0.291 -> 0.238, M = 17 0.300 -> 0.256; 768 x 768
        // and 3072 x 768 at M = 4, us per launch: 5.94 -> 3.17, 8.00 -> 5.79).
        const int64_t nwg = wgs * mgroups;
        if (nwg >= 32) {
            p.kind = X3Plan::kFullK;
            p.mb = M <= 4 ? 4 : (M <= 8 ? 8 : 16);
            // up to 4 rows the three bf16 parts of each row are rows of one
            // MFMA (12 of its 16), instead of three MFMAs with 4 rows each
            // (W4_X3K_P3=0: three MFMAs)
            static const int64_t env_p3 = env_int_or("W4_X3K_P3", 1);
            p.p3 = p.mb == 4 && env_p3 != 0;
            p.nt = (int)tpw;
            // 8 waves, each loading one quad ahead of its arithmetic; 4 where K
            // is short.  3.8B pass (128 launches) at M = 4 / 8 in the runtime
            // loop: 4 quads ahead 1.68 / 1.93 ms, 2 ahead 1.55 / 1.85, 1 ahead
            // 1.50 / 1.77 ms (4 or 16 waves at 1 ahead: 1.87 / 1.71 ms at
            // M = 4).  That loop waits for every load in flight at its head
            // (its loads sit under a runtime condition), so depth there only
            // costs registers; the straight-line kernels below (NQC) wait for
            // each quad's own loads.
            p.waves = NQ <= 8 ? 4 : 8;
            // Fewer than 256 workgroups: twice the waves, each with fewer
            // quads, for grids below 128, for row groups and for short K
            // (GPT-2 at M = 58, us per launch: 768 x 768 4.42 -> 3.92 with
            // 8 waves, 3072 x 768 7.47 -> 7.13 with 16; at M = 4 768 x 2304
            // 3.58 -> 3.24 with 8).  The 3.8B N = 3072 shapes (192 workgroups,
            // K = 3072 or 8192) keep 8 (16 waves: 8192 x 3072 at M = 4 12.4 ->
            // 14.0 us).
            if (nwg < 256 && (nwg < 128 || M > 16 || NQ <= 8)) p.waves = NQ <= 8 ? 8 : 16;
            if (env_waves == 4 || env_waves == 8 || env_waves == 16) p.waves = (int)env_waves;
            if (p.nt == 2 && p.waves == 16) p.waves = 8;  // 1024 threads leave too few registers
            // quads of loads in flight per wave (0: the kernel's default for its row count)
            static const int64_t env_d = env_int("W4_X3K_D");
            p.dq = (env_d >= 1 && env_d <= 4) ? (int)env_d : 0;
            // Up to 4 rows with 3 or 8 quads per wave (K = 3072 or 8192): the
            // straight-line kernel, every load of a quad in flight before its
            // arithmetic (all three at K = 3072, two at a time at 8192); 3.8B
            // pass at M = 4 1.481 -> 1.441 ms.  At 8 and 16 rows it is not
            // faster (1.703 -> 1.730, 2.080 -> 2.123 ms at two ahead: the
            // larger activation buffers cost occupancy).  W4_X3K_NQC=0 turns
            // it off, =1 also allows it past 4 rows.
            static const int64_t env_nqc = env_int_or("W4_X3K_NQC", 2);
            if (env_nqc != 0 && (p.mb == 4 || env_nqc == 1) && p.waves == 8 && NQ % 8 == 0 &&
                (NQ / 8 == 3 || NQ / 8 == 8)) {
                p.nqc = (int)(NQ / 8);
                if (p.dq == 0 && p.mb == 4 && p.nt == 1) p.dq = p.nqc == 3 ? 3 : 2;
            }
            p.col_wgs = wgs;
            p.mgroups = mgroups;
            p.splits = 1;
            p.workspace = 0;
            return p;
        }
    }
    p.kind = X3Plan::kRun;
    const int64_t rows = M < 64 ? M : 64;
    p.mt = (int)cdiv(rows, 16);
    // Row tiles per workgroup.  Taller tiles convert each code once for more
    // rows, but a small matrix then forms too few workgroups to fill the
    // chip: with the workgroups that 64-row tiles allow (column groups x
    // quads x row groups), measured best were 16-row tiles below 512 (every
    // GPT-2 shape at M = 58 and 130), 32 rows below 2048 (3072 x 3072), 64
    // rows above (the larger 3.8B shapes).
    const int64_t w64 = cdiv(N, 64) * (K / 128) * cdiv(M, 64);
    if (w64 < 512) p.mt = 1;
    else if (w64 < 2048 && p.mt > 2) p.mt = 2;
    static const int64_t env_mt = env_int("W4_X3_MT");
    if (env_mt >= 1 && env_mt <= 4) p.mt = (int)(env_mt < cdiv(rows, 16) ? env_mt : cdiv(rows, 16));
    static const int64_t env_nt = env_int("W4_X3_NT");
    p.nt = (env_nt == 2 && p.mt <= 2) ? 2 : 1;
    // quads of loads in flight ahead of the arithmetic (one 16-row tile: 2,
    // 2.196 -> 2.175 ms per M = 16 3.8B pass against 3)
    p.dq = p.mt == 1 && p.nt == 1 ? 2 : (p.mt <= 2 ? 3 : 2);
    if (p.mt == 2 && p.nt == 2) p.dq = 2;
    static const int64_t env_dq = env_int("W4_X3_DQ");
    if (p.mt == 1 && p.nt == 1 && env_dq >= 1 && env_dq <= 3) p.dq = (int)env_dq;
    p.col_wgs = cdiv(N, 64 * p.nt);
    p.mgroups = cdiv(M, 16 * p.mt);
    p.npad = p.col_wgs * 64 * p.nt;
    // enough workgroups to fill the chip; larger row tiles carry more matrix
    // work per weight byte, so fewer (and less split-K partial traffic)
    static const int64_t env_wgs = env_int("W4_X3_TARGET_WGS");
    // about four workgroups per compute unit, measured best at M = 16 and 58
    // on the 3.8B shapes (the extra split-K partials cost less than idle CUs)
    const int64_t target = env_wgs > 0 ? env_wgs : 1024;
    int64_t splits = cdiv(target, p.col_wgs * p.mgroups);
    // No split when the matrix already forms half a chip of workgroups and
    // each one's K loop is short (K <= 1024): the split-K reduce is a second
    // launch, which costs more there than the idle compute units (GPT-2
    // 768 x 2304 and 768 x 3072 at M = 58: 9.5 -> 8.1 and 10.2 -> 8.0 us)
    if (env_wgs <= 0 && p.col_wgs * p.mgroups >= 128 && NQ <= 8) splits = 1;
    if (splits > NQ) splits = NQ;
    if (splits < 1) splits = 1;
    const int64_t qmax = 12;
    const int64_t want = cdiv(NQ, splits);  // quads per workgroup, then the largest
    static const int allowed[] = {12, 8, 6, 4, 3, 2, 1};  // instantiated count <= want
    p.quads_per_wg = 1;
    for (int a : allowed)
        if (a <= want && a <= qmax) {
            p.quads_per_wg = a;
            break;
        }
    p.splits = cdiv(NQ, p.quads_per_wg);
    p.workspace = splitk_bytes(p.splits, p.npad, M);
    return p;
}

}  // namespace w4
