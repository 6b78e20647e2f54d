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
    if (threads) {
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
        // Two rows: the most passes that still give a workgroup to every
        // compute unit, whether or not the count divides evenly (3072 x 9216:
        // 4 passes 11.2 us against 16.8 us for the even 2; 3072 x 3072: 6.2
        // against 6.9 us)
        for (int i = 0; i < nallowed && !found; ++i) {
            const int P = allowed[i];
            if (cdiv(N, (int64_t)p.groups * P) * cdiv(M, p.rows) >= 256) {
                p.passes = P;
                found = true;
            }
        }
    }
    if (env_p <= 0) {
        for (int i = 0; i < nallowed && !found; ++i) {
            const int P = allowed[i];
            const int64_t wgs = cdiv(N, (int64_t)p.groups * P) * cdiv(M, p.rows);
            if (P <= 8 && wgs >= 256 && wgs % 256 == 0) {
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
    if (env_p <= 0 && p.rows == 1 && p.passes == 1 &&
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
    if (M < min_rows || K <= 0 || N <= 0 || K % 128 != 0) return p;
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
    p.dq = p.mt <= 2 ? 3 : 2;
    if (p.mt == 2 && p.nt == 2) p.dq = 2;
    p.col_wgs = cdiv(N, 64 * p.nt);
    p.mgroups = cdiv(M, 16 * p.mt);
    p.npad = p.col_wgs * 64 * p.nt;
    const int64_t NQ = K / 128;
    // M <= 16 (one 16-row tile): the fp16 kernel, which builds all of its A
    // operands before the first quad (3.8B layer at M = 4: 62 -> 55 us; at
    // M = 16: 70 -> 62 us; at M = 58 the bf16 kernel stays ahead)
    static const int64_t env_bf16 = env_int("W4_X3_BF16");
    p.h3 = p.mt == 1 && p.nt == 1 && p.mgroups == 1 && env_bf16 != 1;
    // enough workgroups to fill the chip; larger row tiles carry more matrix
    // work per weight byte, so fewer (and less split-K partial traffic)
    static const int64_t env_wgs = env_int("W4_X3_TARGET_WGS");
    // bf16: about four workgroups per compute unit, measured best at M = 16
    // and 58 on the 3.8B shapes (the extra split-K partials cost less than
    // idle CUs); fp16 (its workgroups hold up to 52 KB of LDS): about two
    const int64_t target = env_wgs > 0 ? env_wgs : (p.h3 ? 512 : 1024);
    int64_t splits = cdiv(target, p.col_wgs * p.mgroups);
    // No split when the matrix already forms half a chip of workgroups and
    // each one's K loop is short (K <= 1024): the split-K reduce is a second
    // launch, which costs more there than the idle compute units (GPT-2
    // 768 x 2304 and 768 x 3072 at M = 58: 9.5 -> 8.1 and 10.2 -> 8.0 us)
    if (env_wgs <= 0 && p.col_wgs * p.mgroups >= 128 && NQ <= 8) splits = 1;
    if (splits > NQ) splits = NQ;
    if (splits < 1) splits = 1;
    const int64_t qmax = p.h3 ? 4 : 12;
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

int plan_head_kmajor_waves(int64_t K, int64_t N) {
    (void)N;
    static const int64_t env_w = env_int("W4_HEAD_MFMA_WAVES");
    if (K > 1024) return 4;
    if (env_w == 1 || env_w == 2 || env_w == 4) return (int)env_w;
    return 4;
}

}  // namespace w4
