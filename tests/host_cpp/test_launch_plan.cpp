// Host test of the attention launch plan (launch_plan.hpp): the invariants
// the launcher and the workspaces rely on, over a sweep of shapes, device
// sizes and workspace budgets, and the plans the GPU tests and the benchmark
// are written against (256 CUs). Plain C++, built with g++ under sanitizers.
#include <cstdio>

#include "launch_plan.hpp"

using namespace attnblk;

static int g_fail = 0;
static void check(bool ok, const char *what, long H, long sq, long skv, long budget, long cus) {
    if (!ok) {
        ++g_fail;
        if (g_fail < 20)
            std::printf("FAIL %s: H=%ld sq=%ld skv=%ld budget=%ld cus=%ld\n", what, H, sq, skv, budget, cus);
    }
}

static void invariants(int cus, int H, int sq, int skv, int64_t budget) {
    const AttnPlan p = plan_attention(cus, H, sq, skv, budget);
    auto c = [&](bool ok, const char *what) { check(ok, what, H, sq, skv, (long)budget, cus); };
    c(p.nq == 2 || p.nq == 3, "nq is 2 or 3");
    c(p.tail_nq == 2 || p.tail_nq == 3, "tail_nq is 2 or 3");
    c(p.main_rows >= 0 && p.main_rows <= sq, "main rows within the query rows");
    if (p.main_rows >= sq) {  // plain launch
        c(p.n_split <= 1 && p.o_elems == 0 && p.lse_elems == 0, "plain launch has no split");
        return;
    }
    c(p.main_rows % (plan::kRowsPerNq * p.nq) == 0, "main rows are whole query blocks");
    const int tail = sq - p.main_rows;
    if (p.n_split <= 1) {
        c(p.tail_nq != p.nq, "a whole-key tail uses the other workgroup size");
        c(p.o_elems == 0 && p.lse_elems == 0, "a whole-key tail needs no workspace");
        return;
    }
    c(skv >= 2 * plan::kMinSplitKeys, "keys are split only from 1024 on");
    c(p.n_split >= 2 && p.n_split <= plan::kMaxSplit, "2..16 key ranges");
    c(p.split_len % plan::kKeyStep == 0, "key ranges are whole stages");
    c(p.split_len >= plan::kMinSplitKeys, "key ranges of at least 512 keys");
    c((int64_t)(p.n_split - 1) * p.split_len < skv && (int64_t)p.n_split * p.split_len >= skv,
      "the ranges cover every key and none is empty");
    c(p.o_elems == (int64_t)p.n_split * H * tail * plan::kHeadDim, "partial O size");
    c(p.lse_elems * plan::kHeadDim == p.o_elems, "partial LSE size");
    c(p.o_elems <= budget, "partials fit the workspace");
}

static void expect(int H, int sq, int skv, int64_t budget, int main_rows, int nq, int tail_nq, int n_split,
                   int split_len) {
    const AttnPlan p = plan_attention(256, H, sq, skv, budget);
    const bool ok = p.main_rows == main_rows && p.nq == nq && (main_rows == sq || p.tail_nq == tail_nq) &&
                    p.n_split == n_split && (n_split <= 1 || p.split_len == split_len);
    if (!ok) {
        ++g_fail;
        std::printf("FAIL plan H=%d sq=%d skv=%d: got main %d nq %d tail_nq %d split %d x %d\n", H, sq, skv,
                    p.main_rows, p.nq, p.tail_nq, p.n_split, p.split_len);
    }
}

int main() {
    const int heads[] = {1, 2, 3, 4, 8, 16, 32, 40, 48, 64, 128};
    const int rows[] = {1, 2, 63, 64, 100, 127, 128, 255, 256, 383, 384, 385, 700, 1000, 2000, 3100, 4096, 8192,
                        16384, 32768, 65536};
    const int keys[] = {1, 63, 64, 511, 512, 1000, 1023, 1024, 2048, 4097, 8192, 32768, 65536};
    const int64_t budgets[] = {int64_t(1) << 20, int64_t(16) << 20, int64_t(64) << 20};
    const int devices[] = {80, 256, 304};
    long n = 0;
    for (int cus : devices)
        for (int64_t b : budgets)
            for (int H : heads)
                for (int sq : rows)
                    for (int skv : keys) {
                        invariants(cus, H, sq, skv, b);
                        ++n;
                    }
    // degenerate arguments: a plain launch
    const AttnPlan z = plan_attention(256, 0, 100, 100, 1 << 20);
    check(z.main_rows == 100 && z.n_split == 1, "no heads: plain", 0, 100, 100, 1 << 20, 256);

    const int64_t block_ws = int64_t(64) << 20, partial_ws = int64_t(16) << 20;
    // the block at seq 8192 / 16384 / 32768 / 65536, hidden 4096 (32 heads) and 8192 (64 heads)
    expect(32, 8192, 8192, block_ws, 6144, 3, 2, 1, 0);
    expect(32, 16384, 16384, block_ws, 15360, 3, 2, 2, 8192);
    expect(32, 32768, 32768, block_ws, 30720, 3, 2, 1, 0);
    expect(32, 65536, 65536, block_ws, 64512, 3, 2, 2, 32768);
    expect(64, 8192, 8192, block_ws, 7680, 3, 2, 2, 4096);
    // the tensor-parallel share (4 heads), the Ulysses share (4 heads over 32768 rows)
    expect(4, 8192, 8192, block_ws, 0, 3, 2, 2, 4096);
    expect(4, 32768, 32768, block_ws, 24576, 3, 2, 2, 16384);
    // the rank share: one block of 4096 keys, and all 32768 keys at once
    expect(32, 4096, 4096, partial_ws, 4096, 2, 2, 1, 0);
    expect(32, 4096, 32768, partial_ws, 3072, 3, 2, 2, 16384);
    // shapes the GPU tests pick for each path
    expect(40, 2000, 1000, partial_ws, 2000, 3, 3, 1, 0);     // 384-row workgroups only
    expect(40, 3100, 1000, partial_ws, 2304, 3, 2, 1, 0);     // whole-key tail of 256-row workgroups
    expect(32, 3500, 3500, partial_ws, 3072, 3, 2, 4, 896);   // split tail
    expect(40, 2400, 2048, partial_ws, 2304, 3, 2, 4, 512);   // ring one-sequence launch, split tail
    expect(48, 2000, 2000, block_ws, 1920, 3, 2, 4, 512);     // block with a split tail
    expect(2, 1000, 1000, partial_ws, 1000, 2, 2, 1, 0);      // 256-row workgroups only

    std::printf("%ld shapes, %s (%d failures)\n", n, g_fail ? "FAILED" : "OK", g_fail);
    return g_fail ? 1 : 0;
}
