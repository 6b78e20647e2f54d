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

size_t splitk_bytes(int64_t tiles, int64_t splits, int64_t npad, int64_t rows) {
    if (splits <= 1) return 0;
    return align_up((size_t)tiles * 4, kCounterAlign) + (size_t)splits * rows * npad * 4;
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
    p.waves = (env_waves == 1 || env_waves == 2 || env_waves == 4) ? (int)env_waves : 1;
    const int slots = p.waves * kGemvGroups;
    const int64_t NB = K / 32;
    p.tiles = cdiv(N, kGemvTileCols);
    p.npad = p.tiles * kGemvTileCols;
    const int64_t t = env_t > 0 ? env_t : blocks_per_group(p.tiles, NB, slots);
    p.blocks_per_wg = (int64_t)slots * t;
    p.splits = cdiv(NB, p.blocks_per_wg);
    p.workspace = splitk_bytes(p.tiles, p.splits, p.npad, 1);
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
    p.workspace = splitk_bytes(p.tiles, p.splits, p.npad, 1);
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
    p.kind = SmallMPlan::kGeneric;
    return p;
}

}  // namespace w4
