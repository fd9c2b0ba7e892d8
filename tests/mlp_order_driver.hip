// Host checks of the one-launch expert MLP's work order (csrc/mlp_order.hpp):
// every item handed out once, each row's down-projection items after all of its
// SwiGLU-projection items with a group's L1 work between, queue ranges that
// cover the row tiles.  Prints "ok" or the first failures.
#include <stdio.h>

#include <map>
#include <set>
#include <tuple>
#include <vector>

#include "../moe_grouped_gemm_sizes_amd/csrc/mlp_order.hpp"

using namespace moegg;

static int fails = 0;
#define CHECK(cond, ...)                      \
    do {                                      \
        if (!(cond)) {                        \
            if (fails < 20) printf(__VA_ARGS__); \
            ++fails;                          \
        }                                     \
    } while (0)

int main() {
    for (int R = 0; R <= 41; ++R)
        for (int C1 = 1; C1 <= 6; ++C1)
            for (int C2 = 1; C2 <= 5; ++C2) {
                std::set<std::tuple<int, int, int>> seen;
                std::map<int, int> last_l1, first_l2;
                int k = 0, phase, row, c;
                while (mlp_item(k, R, C1, C2, phase, row, c)) {
                    CHECK(phase == 1 || phase == 2, "phase R=%d k=%d\n", R, k);
                    CHECK(row >= 0 && row < R && c >= 0 && c < (phase == 1 ? C1 : C2),
                          "range R=%d C1=%d C2=%d k=%d: phase %d row %d c %d\n", R, C1, C2, k, phase, row, c);
                    CHECK(seen.insert({phase, row, c}).second, "repeat R=%d k=%d\n", R, k);
                    if (phase == 1) last_l1[row] = k;
                    else if (!first_l2.count(row)) first_l2[row] = k;
                    if (++k > 100000) break;
                }
                CHECK(k == R * (C1 + C2), "count R=%d C1=%d C2=%d: %d\n", R, C1, C2, k);
                for (int r = 0; r < R; ++r) {
                    CHECK(last_l1.count(r) && first_l2.count(r), "row %d missing R=%d\n", r, R);
                    // the L1 items of the next group (if any) lie between a row's L1 and L2 items
                    const int g = r / kMlpGroup, next_rows = R - (g + 1) * kMlpGroup;
                    const int gap = next_rows <= 0 ? 0 : (next_rows < kMlpGroup ? next_rows : kMlpGroup) * C1;
                    CHECK(first_l2[r] - last_l1[r] > gap, "order R=%d C1=%d C2=%d row %d: %d .. %d\n", R, C1, C2,
                          r, last_l1[r], first_l2[r]);
                }
                for (int kk = k; kk < k + 64; ++kk) CHECK(!mlp_item(kk, R, C1, C2, phase, row, c), "past end\n");
            }
    for (int n_rt = 0; n_rt <= 300; ++n_rt)
        for (int nq = 1; nq <= 16; ++nq) {
            int next = 0, lo = 1 << 30, hi = -1;
            for (int x = 0; x < nq; ++x) {
                int r0, R;
                mlp_queue_rows(n_rt, x, nq, r0, R);
                CHECK(r0 == next && R >= 0, "queue rows n_rt=%d nq=%d x=%d\n", n_rt, nq, x);
                next = r0 + R;
                lo = R < lo ? R : lo;
                hi = R > hi ? R : hi;
            }
            CHECK(next == n_rt && hi - lo <= 1, "queue cover n_rt=%d nq=%d\n", n_rt, nq);
        }
    if (fails) {
        printf("%d failures\n", fails);
        return 1;
    }
    printf("ok\n");
    return 0;
}
