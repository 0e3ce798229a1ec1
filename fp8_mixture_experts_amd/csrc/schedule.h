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

// The XCD whose range holds pool block pb (0 <= pb < total_mb): the largest x
// with floor(total_mb * x / n_xcd) <= pb, in 32-bit arithmetic (total_mb *
// n_xcd stays far below 2^31).
__host__ __device__ inline int xcd_of_block(int pb, int total_mb, int n_xcd) {
    return ((pb + 1) * n_xcd - 1) / total_mb;
}

// Tile u of XCD range [first, first + cnt) with nbs N blocks: pool block pb
// and N block nb.  The range's pool blocks form groups: each run of one
// expert's blocks inside the range, cut into pieces of at most G blocks
// (G = 1 when n_major is false).  Groups run in order, and a group's tiles
// take each N block in turn over all of its pool blocks, so the tiles that
// read one weight block run together and share it through the XCD's L2;
// with G = 1 this is the row-major order.  A group of s blocks starting at
// block g0 holds tiles [(g0 - first) * nbs, (g0 - first + s) * nbs), so
// pool block first + u / nbs lies in the group of tile u.  expert_of(pb)
// gives a pool block's expert and block_start(e) an expert's first pool
// block (block_start(E) = the total).
// The group of pool block pq of the XCD range [first, first + cnt): its first
// block g0 and its size s (g0 = pq, s = 1 in the row-major order).
template <typename ExpertOf, typename BlockStart>
__host__ __device__ inline void tile_group(int pq, int first, int cnt, int G, bool n_major,
                                           ExpertOf&& expert_of, BlockStart&& block_start,
                                           int& g0, int& s) {
    g0 = pq;
    s = 1;
    if (n_major && G > 1) {
        const int e = expert_of(pq);
        const int r0 = max(block_start(e), first);
        const int r1 = min(block_start(e + 1), first + cnt);
        g0 = r0 + (pq - r0) / G * G;
        s = min(G, r1 - g0);
    }
}

// Tile u of a range whose pool block first + u / nbs lies in the group (g0, s).
__host__ __device__ inline void tile_in_group(int u, int first, int nbs, int g0, int s, int& pb,
                                              int& nb) {
    const int within = u - (g0 - first) * nbs;
    nb = within / s;
    pb = g0 + (within - nb * s);
}

template <typename ExpertOf, typename BlockStart>
__host__ __device__ inline void tile_coords(int u, int first, int cnt, int nbs, int G, bool n_major,
                                            ExpertOf&& expert_of, BlockStart&& block_start,
                                            int& pb, int& nb) {
    int g0, s;
    tile_group(first + u / nbs, first, cnt, G, n_major, expert_of, block_start, g0, s);
    tile_in_group(u, first, nbs, g0, s, pb, nb);
}

// Whether the expert kernel's tiles of this shape take an expert's short last
// pool block into the tile before it: the 128 x 128 FP8 tiles, whose LDS has
// room for a fifth 32-row slice.
__host__ __device__ constexpr bool merge_tail_for(bool mxfp4, int block_m, int block_n) {
    return !mxfp4 && block_m == 128 && block_n == 128;
}

// Rows of pool block m_local (of nblk) of an expert with count routes, at
// BLOCK_M rows per block: at most BLOCK_M; with merge_tail, a last block of at
// most 32 rows is taken by the tile of the block before it (0 rows for it,
// BLOCK_M + its rows for that one).
__host__ __device__ inline int tile_rows(int m_local, int nblk, int count, int block_m, bool merge_tail) {
    int valid = min(block_m, count - m_local * block_m);
    if (merge_tail && nblk >= 2 && count - (nblk - 1) * block_m <= 32) {
        if (m_local == nblk - 1) valid = 0;
        else if (m_local == nblk - 2) valid = count - m_local * block_m;
    }
    return valid;
}

}  // namespace mega_moe
