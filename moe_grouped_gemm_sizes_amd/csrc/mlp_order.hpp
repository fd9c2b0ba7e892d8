// Work order of the one-launch expert MLP: which row tiles each XCD queue holds
// and in which order a queue hands out its SwiGLU-projection (L1) and
// down-projection (L2) items.  Host and device code: the host tests check the
// order's invariants on the CPU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moegg {

// Work item k of one XCD's queue, which holds R consecutive row tiles in
// groups of kMlpGroup rows (the last group may hold fewer): first the L1
// items (SwiGLU projection, C1 column tiles per row) of group 0, then for each
// later group s its L1 items followed by the L2 items (C2 column tiles per row)
// of group s - 1, and last the L2 items of the final group.  Within a group's
// L1 or L2 run the column tile varies slowest, so the rows of a group that
// share an expert read each weight panel at about the same time.  Every L2 item
// thus comes after all L1 items of its own row, with a whole group's L1 work
// between them.  phase 1 = L1, 2 = L2; row is the row tile's index within the
// queue, c the column tile.  False past the end.
constexpr int kMlpGroup = 4;

__host__ __device__ inline bool mlp_item(int k, int R, int C1, int C2, int& phase, int& row, int& c) {
    if (R <= 0) return false;
    const int GM = kMlpGroup;
    const int NG = (R + GM - 1) / GM, gl = R - GM * (NG - 1);
    int g, i;
    if (k < (NG == 1 ? gl : GM) * C1) {
        phase = 1; g = 0; i = k;
    } else {
        k -= (NG == 1 ? gl : GM) * C1;
        const int full = (NG > 2 ? NG - 2 : 0), fb = GM * (C1 + C2);   // groups s = 1 .. NG-2 and s - 1 all full
        if (k < full * fb) {
            const int s = 1 + k / fb;
            i = k - (s - 1) * fb;
            if (i < GM * C1) { phase = 1; g = s; }
            else { phase = 2; g = s - 1; i -= GM * C1; }
        } else {
            k -= full * fb;
            if (NG >= 2 && k < gl * C1) {
                phase = 1; g = NG - 1; i = k;
            } else if (NG >= 2 && k < gl * C1 + GM * C2) {
                phase = 2; g = NG - 2; i = k - gl * C1;
            } else {
                if (NG >= 2) k -= gl * C1 + GM * C2;
                if (k >= gl * C2) return false;
                phase = 2; g = NG - 1; i = k;
            }
        }
    }
    const int gm = g == NG - 1 ? gl : GM;
    c = i / gm;
    row = g * GM + (i - c * gm);
    return true;
}

// Row tiles of queue x: the x-th of n_queues consecutive ranges of the n_rt row tiles.
__host__ __device__ inline void mlp_queue_rows(int n_rt, int x, int nq, int& r0, int& R) {
    r0 = (int)((int64_t)n_rt * x / nq);
    R = (int)((int64_t)n_rt * (x + 1) / nq) - r0;
}

}  // namespace moegg
