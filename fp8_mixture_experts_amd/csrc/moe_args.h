// Shared between the host code and the kernels: the argument block every
// kernel of one forward call receives, and the small control record in the
// workspace.
#pragma once

#include <stdint.h>

namespace mega_moe {

constexpr int MAX_XCD = 16;
constexpr int PHASE_XCD_SPLIT = 3;   // phase 3 + n: L1 tiles on XCDs [0, n), L2 tiles on the others

// XCDs whose ranges hold the pool blocks: all of them, or the L1 XCDs of a
// split on disjoint XCD sets.
__host__ __device__ inline int range_xcds(int phase, int n_xcd) {
    return phase >= PHASE_XCD_SPLIT ? phase - PHASE_XCD_SPLIT : n_xcd;
}

// Control record in device memory, reset by the dispatch scan of every call.
struct MoeCtrl {
    int32_t next_tile[MAX_XCD];     // head of each XCD's queue of L1 tiles
    int32_t next_tile_l2[MAX_XCD];  // head of each XCD's queue of L2 tiles
    int32_t total_mb;               // number of pool blocks (BLOCK_M rows) over all experts
    uint32_t error;                 // sticky MEGA_MOE_DEVERR_* bits
    int32_t pad[2];
};

struct MoeArgs {
    // shapes of this call
    int32_t T, H, I, E, k;
    int32_t R;          // T * k routes
    int64_t P_cap;      // pool rows allocated (row stride of the pool-minor arrays)
    int32_t block_m;    // rows per pool block for the expert kernel
    int32_t block_n;    // output columns per expert-kernel tile (128 or 256)
    int32_t nb1;        // L1 N blocks: 2I / block_n
    int32_t nb2;        // L2 N blocks: H / block_n
    int32_t n_major;    // tile order of both phases: 1 = N-major (the pool blocks of a
                        // group take each weight N block in turn), 0 = row-major
    int32_t num_chunks; // dispatch chunks of DISPATCH_CHUNK routes
    uint32_t wait_spin_limit;  // bound on one L2 tile's wait for its L1 tiles
    int32_t n_xcd;      // accelerator complex dies (each with its own L2) of the device
    int32_t xcd_group;  // pool blocks per group of the N-major tile order
    float act_clamp;    // clamp of gate and up before SiLU (+inf: none)
    int32_t fast_math;  // 1: hardware exp2 and reciprocal in SiLU
    int32_t w_fmt;      // 0: FP8 weights with float block scales, 1: MXFP4 weights
    int32_t phase;      // expert kernel: 0 L1 and L2 tiles, 1 L1 tiles only, 2 L2 tiles only;
                        // 3 + n (1 <= n < n_xcd): the L1 and L2 tiles on disjoint XCD sets,
                        // the workgroups of XCDs [0, n) take only L1 tiles and the others
                        // only L2 tiles (the dispatch then gives the pool blocks to
                        // XCDs [0, n) only)
    int32_t steal;      // phase 0: workgroups out of tiles take L2 tiles queued on other XCDs
    int32_t merge_tail; // 1: an expert's last pool block of at most 32 rows joins the tile of
                        // the block before it (the expert kernel's 128-row FP8 tiles)

    // inputs (caller-owned)
    const uint8_t* x;
    const float* x_sf;
    const int32_t* topk_idx;
    const float* topk_w;
    const uint8_t* w1;      // FP8 [E, 2I, H] or E2M1 pairs [E, 2I, H/2]
    const float* w1_sf;     // FP8: [E, 2I/128, H/128]
    const uint8_t* w1_e8;   // MXFP4: UE8M0 [E, 2I, H/32]
    const uint8_t* w2;      // FP8 [E, H, I] or E2M1 pairs [E, H, I/2]
    const float* w2_sf;     // FP8: [E, H/128, I/128]
    const uint8_t* w2_e8;   // MXFP4: UE8M0 [E, H, I/32]
    uint16_t* y;

    // workspace (handle-owned)
    int32_t* counts;      // [E]
    int32_t* offsets;     // [E+1]
    int32_t* pb_rec;      // [PB_cap][4] per pool block: expert, first pool row, rows its
                          // tiles compute (tile_rows), N-major group (first block << 8 | size)
    int32_t* slot_map;    // [R]
    int32_t* src;         // [P_cap]
    float* pool_w;        // [P_cap] the top-k weight of each routed pool row (others unset)
    int32_t* chunk_hist;  // [num_chunks, E]
    int32_t* chunk_base;  // [num_chunks, E]
    uint8_t* l1_acts;     // [P_cap, H]  pool copy of the routed rows (kept pool only)
    float* l1_sf;         // [H/128, P_cap]  their scales (with the kept pool; for
                          //                 128-row tiles always, written by the dispatch)
    float* l1_w;          // [P_cap]  their top-k weights (kept pool only)
    uint8_t* l2_acts;     // [P_cap, I]
    float* l2_sf;         // [I/64, P_cap]
    uint16_t* comb;       // [R, H]
    uint32_t* ready;      // [PB_cap] finished L1 tiles per pool block, plus
                          // READY_PUBLISHED once the block is written back
    int32_t* recv_stats;  // [E] caller-owned cumulative routes per expert, or null
    int32_t* xcd_info;    // [2 * MAX_XCD] first pool block and block count of each XCD
    MoeCtrl* ctrl;
    // 1: the combine moves the call's device error bits out of ctrl (ORs them
    // into *err_out when that is set) and clears them, so that every call
    // reports its own; 0: they stay sticky in ctrl until the host reads them
    int32_t err_move;
    uint32_t* err_out;
};

// ready[pb] bit set when the pool block's L1 output has been written back
// from its XCD's L2 (readable from every XCD)
constexpr uint32_t READY_PUBLISHED = 0x80000000u;

constexpr int DISPATCH_CHUNK = 1024;    // routes per dispatch workgroup
constexpr int DISPATCH_THREADS = 256;
constexpr int POOL_ALIGN = 128;         // pool segment alignment (largest BLOCK_M)
constexpr int MAX_EXPERTS = 1024;

}  // namespace mega_moe
