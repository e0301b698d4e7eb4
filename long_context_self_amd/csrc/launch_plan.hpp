// Launch plan of one fp16 attention over H heads, sq query rows and skv keys
// (plain C++, no HIP: the attention launcher calls it with the device's CU
// count, and a host test checks its invariants).
//
// The attention kernel runs one workgroup per (head, query block) item,
// rounds of one workgroup per CU; its workgroups hold 3 or 2 query blocks of
// 128 rows per wave group (384 or 256 rows). A last round that is only partly
// full leaves CUs idle for a whole workgroup time (10% of the time at 32
// heads and seq 16384). The plan keeps the first query blocks of every head
// whole, in one workgroup size, and runs the rows after them as a tail that
// fills its rounds: in the other workgroup size over all keys, straight into
// the outputs, or split into key ranges whose fp32 partials are merged into
// the outputs by LSE. It takes the plan of least modelled time, counting the
// merge traffic and the extra launches, and none unless it gains at least 1%
// over the plain launch of 384-row workgroups.
#pragma once

#include <algorithm>
#include <cstdint>

namespace attnblk {

// The launch plan: the query rows [0, main_rows) of every head run as
// whole-key workgroups of nq query blocks per wave; the rows [main_rows, sq)
// (the tail) run in workgroups of tail_nq blocks per wave, over all keys
// straight into the outputs (n_split <= 1), or split into n_split key ranges
// of split_len keys whose fp32 partials (o_elems and lse_elems floats of
// workspace) are then merged into the outputs. main_rows == sq: one plain
// launch.
struct AttnPlan {
    int main_rows, n_split, split_len;
    int64_t o_elems, lse_elems;
    int nq;       // 16-row query blocks per wave of the whole-key launch (3: 384-row workgroups, 2: 256)
    int tail_nq;  // the same for the rows from main_rows on
};

namespace plan {

constexpr int kRowsPerNq = 128;   // query rows per workgroup per query block per wave (8 waves x 16)
constexpr int kMaxNQ = 3;         // 384-row workgroups; 2 gives 256
constexpr int kKeyStep = 64;      // keys per stage: key ranges are multiples of it
constexpr int kHeadDim = 128;
constexpr int kMaxSplit = 16;       // key ranges of a split tail
constexpr int kMinSplitKeys = 512;  // shortest key range worth a workgroup
// Cost model of a plan, in seconds: a workgroup over L keys takes about
// kItemPerKey * L (384 rows at the kernel's rate on one CU) plus a fixed
// start-up and epilogue kItemFixed; the partials of a split tail are written
// once and read once by the merge at about kMergeBw; the tail and merge
// launches cost kExtraLaunch (a tail over all keys, with no merge, half that).
constexpr double kItemPerKey = 3.95e-8, kItemFixed = 8e-6, kMergeBw = 4.0e12, kExtraLaunch = 1.5e-5;
// A 256-row workgroup's time per key relative to a 384-row one (it moves more
// LDS bytes per product: measured 0.71 at seq 65536, 0.75 at 8192).
constexpr double kRows256Cost = 0.75;

}  // namespace plan

// The plan for num_heads heads, sq query rows and skv keys on a device with
// `cus` compute units, whose split workspace holds at most max_o_elems floats
// of partial rows.
inline AttnPlan plan_attention(int64_t cus, int num_heads, int sq, int skv, int64_t max_o_elems) {
    using namespace plan;
    AttnPlan p{sq, 1, 0, 0, 0, kMaxNQ, kMaxNQ};
    if (num_heads <= 0 || sq <= 0 || skv <= 0 || cus <= 0) return p;
    auto rounds = [cus](int64_t n) { return (double)((n + cus - 1) / cus); };
    auto blocks = [](int rows, int nq) { return (rows + kRowsPerNq * nq - 1) / (kRowsPerNq * nq); };
    auto item = [](int nq, int keys) {
        return kItemPerKey * (nq == kMaxNQ ? 1.0 : kRows256Cost) * keys + kItemFixed;
    };
    // the plain launch of 384-row workgroups is what any other plan must beat by 1%
    double best = 0.99 * rounds((int64_t)blocks(sq, kMaxNQ) * num_heads) * item(kMaxNQ, skv);
    for (int nq = kMaxNQ; nq >= 2; --nq) {
        const int bq = kRowsPerNq * nq;
        const int nqb = blocks(sq, nq);
        if (nq != kMaxNQ && rounds((int64_t)nqb * num_heads) * item(nq, skv) < best) {
            best = rounds((int64_t)nqb * num_heads) * item(nq, skv);
            p = AttnPlan{sq, 1, 0, 0, 0, nq, nq};
        }
        const int tb_max = (int)std::min<int64_t>(nqb, 2 * cus / num_heads + 1);
        for (int tb = 1; tb <= nqb; ++tb) {
            if (tb > tb_max && tb != nqb) continue;
            const int main_rows = (nqb - tb) * bq;
            const int tail_rows = sq - main_rows;
            const double t_main = rounds((int64_t)(nqb - tb) * num_heads) * item(nq, skv);
            for (int tq = kMaxNQ; tq >= 2; --tq) {
                const int ntb = blocks(tail_rows, tq);
                if (tq != nq) {  // the tail over all keys straight into the outputs: one more launch
                    const double t = t_main + rounds((int64_t)ntb * num_heads) * item(tq, skv) + 0.5 * kExtraLaunch;
                    if (t < best) {
                        best = t;
                        p = AttnPlan{main_rows, 1, 0, 0, 0, nq, tq};
                    }
                }
                if (skv < 2 * kMinSplitKeys) continue;
                for (int k = 2; k <= kMaxSplit; ++k) {
                    const int len = ((skv + k - 1) / k + kKeyStep - 1) / kKeyStep * kKeyStep;
                    if (len < kMinSplitKeys) break;
                    const int ke = (skv + len - 1) / len;
                    const int64_t o_el = (int64_t)ke * num_heads * tail_rows * kHeadDim;
                    if (o_el > max_o_elems) break;
                    const double merge =
                        ((double)o_el * 8.0 + (double)num_heads * tail_rows * kHeadDim * 2.0) / kMergeBw;
                    const double t =
                        t_main + rounds((int64_t)ntb * num_heads * ke) * item(tq, len) + merge + kExtraLaunch;
                    if (t < best) {
                        best = t;
                        p = AttnPlan{main_rows, ke, len, o_el, (int64_t)ke * num_heads * tail_rows, nq, tq};
                    }
                }
            }
        }
    }
    return p;
}

}  // namespace attnblk
