// Host check of the proportional-block decode plan, built from the library's own
// header (csrc/kernels.h) with the host compiler.  Over seeded random batches (empty,
// short and long sequences, several compute-unit and head-block counts, 1 to 300
// state slots) it checks what the split and merge kernels rely on:
//   - every sequence gets at least one block (the first block holds the sink);
//   - the blocks of all sequences number extra + batch, no more than the grid's
//     block columns;
//   - no sequence gets more blocks than the workspace has state slots;
//   - each sequence's blocks of ceil(L / n) keys cover its keys.
// Prints the number of cases and exits 0 when every one holds, 1 at the first that
// does not (with the case).
#include "kernels.h"

#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

int main() {
    std::mt19937_64 rng(20261202);
    long cases = 0;
    for (int iter = 0; iter < 20000; ++iter) {
        const int units = iter % 3 == 0 ? 256 : (iter % 3 == 1 ? 304 : 80);
        const int head_blocks = 1 + static_cast<int>(rng() % 4);
        const int per_round = std::max(1, units / head_blocks);
        const int batch = 1 + static_cast<int>(rng() % (iter % 10 == 0 ? 4000 : 300));
        const int64_t ranges =
            (int64_t)per_round * ((batch + per_round / 2 + per_round - 1) / per_round);
        const int slots = 1 + static_cast<int>(rng() % 300);
        std::vector<int> len(batch);
        int64_t total64 = 0;
        int max_len = 0;
        for (int& l : len) {
            const int kind = static_cast<int>(rng() % 4);
            l = kind == 0 ? 0
                : kind == 1 ? static_cast<int>(rng() % 64)
                : kind == 2 ? static_cast<int>(rng() % 5000)
                            : static_cast<int>(rng() % 200000);
            total64 += l;
            max_len = std::max(max_len, l);
        }
        if (total64 > INT_MAX) continue;
        const int total = static_cast<int>(total64);
        const sa::DecodePlan plan{0, static_cast<int>(ranges), max_len, slots};
        const int extra = sa::balanced_extra_blocks(total, batch, plan);
        auto bad = [&](const char* what, int b, long long got) {
            std::printf("FAIL %s: iter %d batch %d units %d head_blocks %d slots %d total %d "
                        "extra %d sequence %d value %lld\n", what, iter, batch, units,
                        head_blocks, slots, total, extra, b, got);
            return 1;
        };
        if (extra < 0) return bad("extra < 0", -1, extra);
        int64_t before = 0;
        int first = sa::balanced_first_block(0, 0, total, extra);
        if (first != 0) return bad("first block of sequence 0", 0, first);
        for (int b = 0; b < batch; ++b) {
            before += len[b];
            const int next = sa::balanced_first_block(static_cast<int>(before), b + 1, total, extra);
            const int n = next - first;
            if (n < 1) return bad("a sequence without a block", b, n);
            if (n > std::max(slots, 1)) return bad("more blocks than state slots", b, n);
            const int64_t per = (len[b] + n - 1) / n;
            if (per * n < len[b]) return bad("blocks do not cover the keys", b, per * n);
            first = next;
        }
        if (first != extra + batch) return bad("block count", -1, first);
        if (first > ranges) return bad("more blocks than block columns", -1, first);
        ++cases;
    }
    std::printf("%ld cases\n", cases);
    return 0;
}
