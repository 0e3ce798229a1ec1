// Work order of the expert kernel, shared by the kernels (dispatch and the
// expert kernel) and by the host-side query of it.
//
// The M pool blocks of a call are split into contiguous ranges, one per XCD;
// each XCD's workgroups take the tiles of their range from that XCD's queue,
// first every L1 tile, then every L2 tile.  Within a range of cnt pool blocks
// and nbs N blocks, queue position u names one (pool block, N block) pair.
#pragma once

#include <hip/hip_runtime.h>

namespace mega_moe {

// Pool blocks per group of the N-major order: a group's tiles of one N block
// run together, so they share that weight block through the XCD's L2.
__host__ __device__ inline int xcd_group_for(int block_m) { return block_m == 64 ? 2 : 4; }

// XCD x of n takes the pool blocks [lo, lo + cnt) = [x*M/n, (x+1)*M/n): the
// same number of blocks (+-1) on every XCD, consecutive blocks of one expert
// mostly on one XCD.
__host__ __device__ inline void xcd_range(int total_mb, int n_xcd, int x, int& lo, int& cnt) {
    lo = (int)((int64_t)total_mb * x / n_xcd);
    cnt = (int)((int64_t)total_mb * (x + 1) / n_xcd) - lo;
}

// Tile u of a range of cnt pool blocks x nbs N blocks: pool block j (relative
// to the range) and N block nb.  Row-major keeps a pool block's N blocks
// together; N-major runs each N block across the (at most G) pool blocks of a
// group.
__host__ __device__ inline void tile_coords(int u, int cnt, int nbs, int G, bool n_major, int& j,
                                            int& nb) {
    if (!n_major) {
        j = u / nbs;
        nb = u - j * nbs;
        return;
    }
    const int k = u / (G * nbs);
    const int within = u - k * G * nbs;
    const int g = min(G, cnt - k * G);
    nb = within / g;
    j = k * G + (within - nb * g);
}

}  // namespace mega_moe
