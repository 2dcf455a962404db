// Chiplet-aware workgroup -> output-tile order, shared by the tile kernel
// (device) and the library's host-side check.
//
// HipKittens talk notes, section 3 (Algorithm 1, Table 4): workgroups are
// dispatched to the 8 XCDs round-robin.  Step 1 renumbers them so that C
// consecutive logical ids run on one XCD (the tail past the last full block
// of 8 C keeps its id); step 2 walks the tile grid column-first inside
// windows W tile rows tall, so the workgroups one XCD runs together cover a
// compact block of tiles and share A rows and B columns in its L2.
#pragma once

#include <hip/hip_runtime.h>

namespace hkg {

__host__ __device__ inline void tile_order(int b, int tiles_m, int tiles_n, int win_w, int chunk_c,
                                           int& tm, int& tn)
{
    const int total = tiles_m * tiles_n;
    int L = b;
    if (chunk_c > 0) {
        const int group = 8 * chunk_c;
        const int full = (total / group) * group;
        if (b < full) {
            const int xcd = b & 7;
            const int r = b >> 3;
            L = ((r / chunk_c) * 8 + xcd) * chunk_c + (r % chunk_c);
        }
    }
    if (win_w > 0) {
        const int span = win_w * tiles_n;
        const int g = L / span;
        const int row0 = g * win_w;
        const int rest = tiles_m - row0;
        const int h = win_w < rest ? win_w : rest;
        const int within = L - g * span;
        tm = row0 + within % h;
        tn = within / h;
    } else {
        tm = L / tiles_n;
        tn = L - tm * tiles_n;
    }
}

}  // namespace hkg
