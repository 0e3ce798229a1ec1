// Dispatch of the expert layer: per-expert histogram, prefix scan into
// 128-aligned pool segments, a stable slot for every route and, when the
// layer keeps the pool, the copy of each routed token into its expert's pool
// ("MegaMoE SM90 Implementation Design (Final)" 3.3 phase 1 and 9.2; one GPU,
// so every source is local).  Without the pool copy the expert kernel's L1
// tiles read each route's row of x in place through `src`.
//
// Up to 4096 routes: one launch on the caller's stream,
//   moe_dispatch_small   one workgroup: histogram, scan, stable ranks, slot
//                        map and source metadata, resets
// larger batches: three,
//   moe_dispatch_count   one workgroup per chunk of 1024 routes: histogram
//   moe_dispatch_scan    one workgroup: per-expert scan over chunks, the
//                        wavefront prefix scan over experts (offsets, pool
//                        blocks), padding metadata, reset of the expert
//                        kernel's queue and arrival counters
//   moe_dispatch_scatter one workgroup per chunk: stable rank of every route
//                        inside its expert (wave ballots), slot map and source
//                        metadata
// then, for the expert kernel's 128-row tiles,
//   moe_pool_scales      the activation scales in pool order (one run per K
//                        block), which those tiles read instead of gathering
// and, with the pool kept, one more:
//   moe_dispatch_gather  copy of the FP8 row, its scales and its top-k weight
//                        into the pool row of every route
#include <hip/hip_runtime.h>

#include "moe_args.h"
#include "schedule.h"
#include "mega_moe.h"

namespace mega_moe {

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__global__ void __launch_bounds__(DISPATCH_THREADS)
moe_dispatch_count(MoeArgs a) {
    __shared__ int hist[MAX_EXPERTS];
    const int tid = threadIdx.x;
    for (int e = tid; e < a.E; e += DISPATCH_THREADS) hist[e] = 0;
    __syncthreads();
    const int f0 = blockIdx.x * DISPATCH_CHUNK;
    bool bad = false;
    for (int i = tid; i < DISPATCH_CHUNK; i += DISPATCH_THREADS) {
        const int f = f0 + i;
        if (f < a.R) {
            const int e = a.topk_idx[f];
            if (e >= 0 && e < a.E) atomicAdd(&hist[e], 1);
            else if (e >= a.E) bad = true;
        }
    }
    if (bad) atomicOr(&a.ctrl->error, MEGA_MOE_DEVERR_BAD_EXPERT);
    __syncthreads();
    for (int e = tid; e < a.E; e += DISPATCH_THREADS)
        a.chunk_hist[(size_t)blockIdx.x * a.E + e] = hist[e];
}

// Exclusive scan of one int per thread over a workgroup of SCAN_THREADS
// (wave64 inclusive scan by shuffles, then a scan of the wave totals).
constexpr int SCAN_THREADS = 1024;

__device__ int block_exclusive_scan(int v, int* s_wave, int* total) {
    const int lane = lane_id();
    const int wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int n = __shfl_up(incl, d, 64);
        if (lane >= d) incl += n;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const int nw = SCAN_THREADS / 64;
        int w = lane < nw ? s_wave[lane] : 0;
        int wi = w;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int n = __shfl_up(wi, d, 64);
            if (lane >= d) wi += n;
        }
        if (lane < nw) s_wave[lane] = wi - w;       // exclusive prefix of wave totals
        if (lane == nw - 1) s_wave[SCAN_THREADS / 64] = wi;
    }
    __syncthreads();
    const int out = s_wave[wave] + incl - v;
    *total = s_wave[SCAN_THREADS / 64];
    __syncthreads();
    return out;
}

// With every expert's count in s_count (one workgroup of SCAN_THREADS):
// the counts (also added to the caller's cumulative statistics when set),
// 128-aligned segment offsets and pool blocks by a wavefront prefix scan over
// the experts, the expert of every pool block with a cleared arrival counter,
// each XCD's range of pool blocks, the cleared queue heads, and -1 in `src`
// for the padding rows of every segment (the routed rows are written by the
// ranking).  Leaves the segment offsets in s_off.
__device__ void finish_counts(const MoeArgs& a, const int* s_count, int* s_off, int* s_mb,
                              int* s_wave) {
    const int tid = threadIdx.x;
    const int E = a.E;
    const int e = tid;
    const int cnt = e < E ? s_count[e] : 0;
    const int padded = (cnt + POOL_ALIGN - 1) / POOL_ALIGN * POOL_ALIGN;
    const int mbs = (cnt + a.block_m - 1) / a.block_m;
    int total_rows = 0, total_mb = 0;
    const int off = block_exclusive_scan(padded, s_wave, &total_rows);
    const int mb0 = block_exclusive_scan(mbs, s_wave, &total_mb);
    if (e < E) {
        s_off[e] = off;
        s_mb[e] = mb0;
        a.counts[e] = cnt;
        if (a.recv_stats) a.recv_stats[e] += cnt;
        a.offsets[e] = off;
    }
    if (tid == 0) {
        s_off[E] = total_rows;
        s_mb[E] = total_mb;
        a.offsets[E] = total_rows;
        a.ctrl->total_mb = total_mb;
        for (int x = 0; x < MAX_XCD; ++x) {
            a.ctrl->next_tile[x] = 0;
            a.ctrl->next_tile_l2[x] = 0;
        }
    }
    __syncthreads();

    // padding rows of each segment: [off + count, off + align128(count))
    for (int i = tid; i < E * POOL_ALIGN; i += SCAN_THREADS) {
        const int ex = i / POOL_ALIGN, r = i - ex * POOL_ALIGN;
        const int c = s_count[ex];
        const int pad = (c + POOL_ALIGN - 1) / POOL_ALIGN * POOL_ALIGN - c;
        if (r < pad) a.src[s_off[ex] + c + r] = -1;
    }

    // Per-XCD work: XCD x takes a contiguous range of the M pool blocks
    // (expert-major); with the phases on disjoint XCD sets only the L1 XCDs
    // hold ranges
    const int rx = range_xcds(a.phase, a.n_xcd);
    if (tid < a.n_xcd) {
        int lo = total_mb, cnt = 0;
        if (tid < rx) xcd_range(total_mb, rx, tid, lo, cnt);
        a.xcd_info[2 * tid] = lo;
        a.xcd_info[2 * tid + 1] = cnt;
    }

    // a cleared arrival counter for every pool block, and its record for the
    // expert kernel's tile set-up: expert, first pool row, the rows its tiles
    // compute, and its N-major group inside its XCD's range
    for (int pb = tid; pb < total_mb; pb += SCAN_THREADS) {
        int lo = 0, hi = E - 1;               // last expert with s_mb[ex] <= pb
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_mb[mid] <= pb) lo = mid; else hi = mid - 1;
        }
        a.ready[pb] = 0;
        const int ex = lo, m = pb - s_mb[ex];
        const int rows = tile_rows(m, s_mb[ex + 1] - s_mb[ex], s_count[ex], a.block_m, a.merge_tail != 0);
        const int x = xcd_of_block(pb, total_mb, rx);
        const int xlo = total_mb * x / rx;
        const int xcnt = total_mb * (x + 1) / rx - xlo;
        int g0, gs;
        tile_group(pb, xlo, xcnt, a.xcd_group, a.n_major != 0, [&](int) { return ex; },
                   [&](int ee) { return s_mb[ee]; }, g0, gs);
        *reinterpret_cast<int4*>(a.pb_rec + 4 * (size_t)pb) =
            int4{ex, s_off[ex] + m * a.block_m, rows, (g0 << 8) | gs};
    }
}

__global__ void __launch_bounds__(SCAN_THREADS)
moe_dispatch_scan(MoeArgs a) {
    __shared__ int s_count[MAX_EXPERTS];
    __shared__ int s_off[MAX_EXPERTS + 1];
    __shared__ int s_mb[MAX_EXPERTS + 1];
    __shared__ int s_wave[SCAN_THREADS / 64 + 1];
    const int tid = threadIdx.x;
    const int E = a.E;

    // per expert: running sum over chunks (relative chunk bases) and count
    for (int e = tid; e < E; e += SCAN_THREADS) {
        int run = 0;
        for (int c0 = 0; c0 < a.num_chunks; c0 += 8) {   // 8 loads in flight at a time
            int h[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                h[j] = c0 + j < a.num_chunks ? a.chunk_hist[(size_t)(c0 + j) * E + e] : 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (c0 + j < a.num_chunks) a.chunk_base[(size_t)(c0 + j) * E + e] = run;
                run += h[j];
            }
        }
        s_count[e] = run;
    }
    __syncthreads();
    finish_counts(a, s_count, s_off, s_mb, s_wave);

    // absolute chunk bases
    const size_t ce = (size_t)a.num_chunks * E;
    for (size_t i = tid; i < ce; i += SCAN_THREADS) a.chunk_base[i] += s_off[i % E];
}

// Stable rank of route f among the lanes of its wave with the same key, and
// the number of such lanes (keys 0..E, E = not routed), by ballots bit by bit.
__device__ __forceinline__ int wave_rank(int key, int key_bits, int* peers_count) {
    const int lane = lane_id();
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint64_t peers = __ballot(1);
    for (int b = 0; b < key_bits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t m = __ballot(bit);
        peers &= bit ? m : ~m;
    }
    *peers_count = __popcll(peers);
    return __popcll(peers & lt_mask);
}

// Small batches (at most SMALL_CHUNKS chunks of routes; each ranking round
// costs about as much as a launch, so larger batches take the multi-workgroup
// path): the whole dispatch but the pool copy in one workgroup: LDS
// histogram, the scan above, then
// stable ranks in rounds of SCAN_THREADS routes (ballots inside a wave, per
// wave counts in LDS across waves, a running base per expert across rounds).
constexpr int SMALL_CHUNKS = 4;
constexpr int SMALL_WAVES = SCAN_THREADS / 64;
constexpr int SMALL_ROUNDS = SMALL_CHUNKS * DISPATCH_CHUNK / SCAN_THREADS;

__global__ void __launch_bounds__(SCAN_THREADS)
moe_dispatch_small(MoeArgs a) {
    __shared__ int s_count[MAX_EXPERTS];
    __shared__ int s_off[MAX_EXPERTS + 1];
    __shared__ int s_mb[MAX_EXPERTS + 1];
    __shared__ int s_wave[SCAN_THREADS / 64 + 1];
    __shared__ int wcnt[SMALL_WAVES][MAX_EXPERTS];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int E = a.E;

    // every route's expert and top-k weight, read once (at most SMALL_CHUNKS
    // rounds of SCAN_THREADS routes) for the histogram and the ranking
    int re[SMALL_ROUNDS];
    float rw[SMALL_ROUNDS];
#pragma unroll
    for (int r = 0; r < SMALL_ROUNDS; ++r) {
        const int f = r * SCAN_THREADS + tid;
        re[r] = f < a.R ? a.topk_idx[f] : -1;
        rw[r] = f < a.R ? a.topk_w[f] : 0.0f;
    }
    for (int e = tid; e < E; e += SCAN_THREADS) s_count[e] = 0;
    __syncthreads();
    bool bad = false;
#pragma unroll
    for (int r = 0; r < SMALL_ROUNDS; ++r) {
        const int e = re[r];
        if (e >= 0 && e < E) atomicAdd(&s_count[e], 1);
        else if (e >= E) bad = true;
    }
    if (bad) atomicOr(&a.ctrl->error, MEGA_MOE_DEVERR_BAD_EXPERT);
    __syncthreads();
    finish_counts(a, s_count, s_off, s_mb, s_wave);

    int key_bits = 0;
    while ((1 << key_bits) <= E) ++key_bits;
    // s_off becomes the running base of each expert's next slot
#pragma unroll
    for (int round = 0; round < SMALL_ROUNDS; ++round) {
        if (round * SCAN_THREADS >= a.R) break;
        for (int i = tid; i < SMALL_WAVES * E; i += SCAN_THREADS) wcnt[i / E][i % E] = 0;
        __syncthreads();
        const int f = round * SCAN_THREADS + tid;
        const int e = re[round];
        const float wf = rw[round];
        const bool valid = e >= 0 && e < E;
        int n_same;
        const int rank = wave_rank(valid ? e : E, key_bits, &n_same);
        if (valid && rank == 0) wcnt[wave][e] = n_same;
        __syncthreads();
        if (valid) {
            int slot = s_off[e] + rank;
            for (int w = 0; w < wave; ++w) slot += wcnt[w][e];
            a.slot_map[f] = slot;
            a.src[slot] = f;
            a.pool_w[slot] = wf;
        } else if (f < a.R) {
            a.slot_map[f] = -1;
        }
        __syncthreads();
        for (int ex = tid; ex < E; ex += SCAN_THREADS) {
            int sum = 0;
            for (int w = 0; w < SMALL_WAVES; ++w) sum += wcnt[w][ex];
            s_off[ex] += sum;
        }
        __syncthreads();
    }
}

__global__ void __launch_bounds__(DISPATCH_THREADS)
moe_dispatch_scatter(MoeArgs a) {
    constexpr int NW = DISPATCH_THREADS / 64;
    __shared__ int running[MAX_EXPERTS];
    __shared__ int wcnt[NW][MAX_EXPERTS];
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid >> 6;
    const int E = a.E;
    const int c = blockIdx.x;
    int key_bits = 0;
    while ((1 << key_bits) <= E) ++key_bits;   // keys 0..E (E = "no expert")

    for (int e = tid; e < E; e += DISPATCH_THREADS) running[e] = 0;

    for (int round = 0; round < DISPATCH_CHUNK / DISPATCH_THREADS; ++round) {
        for (int i = tid; i < NW * E; i += DISPATCH_THREADS) wcnt[i / E][i % E] = 0;
        __syncthreads();
        const int f = c * DISPATCH_CHUNK + round * DISPATCH_THREADS + tid;
        int e = f < a.R ? a.topk_idx[f] : -1;
        const float wf = f < a.R ? a.topk_w[f] : 0.0f;
        const bool valid = e >= 0 && e < E;
        int n_same;
        const int rank = wave_rank(valid ? e : E, key_bits, &n_same);
        if (valid && rank == 0) wcnt[wave][e] = n_same;
        __syncthreads();
        if (valid) {
            int before = running[e] + rank;
            for (int w = 0; w < wave; ++w) before += wcnt[w][e];
            const int slot = a.chunk_base[(size_t)c * E + e] + before;
            a.slot_map[f] = slot;
            a.src[slot] = f;
            a.pool_w[slot] = wf;
        } else if (f < a.R) {
            a.slot_map[f] = -1;
        }
        __syncthreads();
        for (int ex = tid; ex < E; ex += DISPATCH_THREADS) {
            int s = 0;
            for (int w = 0; w < NW; ++w) s += wcnt[w][ex];
            running[ex] += s;
        }
        __syncthreads();
    }
}

__global__ void __launch_bounds__(256)
moe_dispatch_gather(MoeArgs a) {
    const int tid = threadIdx.x;
    const int H = a.H;
    const int kb_n = H / 128;
    for (int f = blockIdx.x; f < a.R; f += gridDim.x) {
        const int slot = a.slot_map[f];
        if (slot < 0) continue;
        const int t = f / a.k;
        const uint4* s = reinterpret_cast<const uint4*>(a.x + (size_t)t * H);
        uint4* d = reinterpret_cast<uint4*>(a.l1_acts + (size_t)slot * H);
        for (int i = tid; i < H / 16; i += blockDim.x) d[i] = s[i];
        for (int i = tid; i < kb_n; i += blockDim.x)
            a.l1_sf[(size_t)i * a.P_cap + slot] = a.x_sf[(size_t)t * kb_n + i];
        if (tid == 0) a.l1_w[slot] = a.topk_w[f];
    }
}

// The activation scales in pool order, for the 128-row tiles: l1_sf[kb, s] =
// x_sf[t, kb] for pool row s holding a route of token t, 0 for padding rows
// ("MegaMoE SM90 Implementation Design (Final)" 9.2: the pool keeps the
// scales MN-major).  A 128-row L1 tile then reads a step's scales as one
// contiguous run instead of one cache line per row, and the gather from x_sf
// happens once per pool row instead of once per N block.  A workgroup
// transposes POOL_SF_ROWS pool rows through LDS: it reads each row's scales
// as one contiguous run of x_sf and writes each K block's run of rows as one
// contiguous run of l1_sf.
constexpr int POOL_SF_ROWS = 16;

__global__ void __launch_bounds__(256)
moe_pool_scales(MoeArgs a) {
    __shared__ float tile[64 * POOL_SF_ROWS];          // [kb][row], H / 128 <= 64
    const int kb_n = a.H / 128;
    const int s0 = blockIdx.x * POOL_SF_ROWS;
    const int rows = min(POOL_SF_ROWS, a.offsets[a.E] - s0);
    if (rows <= 0) return;
    for (int i = threadIdx.x; i < POOL_SF_ROWS * kb_n; i += blockDim.x) {
        const int r = i / kb_n, kb = i - r * kb_n;
        const int f = r < rows ? a.src[s0 + r] : -1;
        tile[kb * POOL_SF_ROWS + r] = f >= 0 ? a.x_sf[(size_t)(f / a.k) * kb_n + kb] : 0.0f;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < POOL_SF_ROWS * kb_n; i += blockDim.x) {
        const int kb = i / POOL_SF_ROWS, r = i - kb * POOL_SF_ROWS;
        if (r < rows) a.l1_sf[(size_t)kb * a.P_cap + s0 + r] = tile[kb * POOL_SF_ROWS + r];
    }
}

__global__ void __launch_bounds__(256) moe_clear_words(uint32_t* p, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

// Clears n words at p with a kernel (not a memory set, so that a captured
// call records a kernel node).
void launch_clear_words(uint32_t* p, int n, hipStream_t stream) {
    hipLaunchKernelGGL(moe_clear_words, dim3(1), dim3(256), 0, stream, p, n);
}

void launch_dispatch(const MoeArgs& a, int gather_blocks, hipStream_t stream) {
    if (a.num_chunks <= SMALL_CHUNKS) {
        hipLaunchKernelGGL(moe_dispatch_small, dim3(1), dim3(SCAN_THREADS), 0, stream, a);
    } else {
        hipLaunchKernelGGL(moe_dispatch_count, dim3(a.num_chunks), dim3(DISPATCH_THREADS), 0, stream, a);
        hipLaunchKernelGGL(moe_dispatch_scan, dim3(1), dim3(SCAN_THREADS), 0, stream, a);
        hipLaunchKernelGGL(moe_dispatch_scatter, dim3(a.num_chunks), dim3(DISPATCH_THREADS), 0, stream, a);
    }
    // the pool copies are only for inspection (the expert kernel reads x)
    if (gather_blocks > 0)
        hipLaunchKernelGGL(moe_dispatch_gather, dim3(gather_blocks), dim3(256), 0, stream, a);
    // 128-row tiles read the activation scales in pool order
    if (a.block_m == 128) {
        const int64_t blocks = (a.P_cap + POOL_SF_ROWS - 1) / POOL_SF_ROWS;
        hipLaunchKernelGGL(moe_pool_scales, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    }
}

}  // namespace mega_moe
