/*
 * mega_moe.h - C ABI of the fused FP8 mixture-of-experts expert layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer is the one the page "MegaMoE SM90 Implementation Design (Final)"
 * describes (cited as "SM90 design" with its section numbers), run as one
 * GPU's share of expert parallelism: all E experts are local and every routed
 * token is local.  One forward call computes, on the caller's HIP stream:
 *
 *   1. dispatch       per-expert counts, 128-aligned pool offsets, a stable
 *                     slot per (token, top-k slot) route and source metadata;
 *                     the L1 tiles then read each route's FP8 row, float
 *                     scales and top-k weight in place (with keep_pool, the
 *                     dispatch also copies them into the permuted per-expert
 *                     pool)                               (SM90 design 3.3, 9.2)
 *   2. L1 GEMM        FP8 x FP8 with one float scale per 128 K for the
 *                     activations (per token) and per 128x128 block for W1;
 *                     W1 rows are gate/up interleaved by 8  (5.1-5.3, 15.1-15.2)
 *   3. SwiGLU         silu(gate) * up * top-k weight            (10.1 steps 1-3)
 *   4. re-quantise    per row and 64 columns: sf = amax / 448,
 *                     code = e4m3(h / sf)                        (10.1 steps 4-6)
 *   5. L2 GEMM        FP8 x FP8, each 128-K block split in two 64-K halves with
 *                     their own activation scales; result cast to BF16 (5.4, 11.1)
 *   6. combine        per token, FP32 sum of the BF16 partials of its active
 *                     slots in slot order, cast to BF16        (11.2; "PR357
 *                     Green-Context Split MegaMoE code review" 6.3)
 *
 * Conventions for every entry point:
 *   - Device pointers are owned by the caller, row-major and contiguous.
 *     x, W1, W2 and y must be 16-byte aligned; float and int arrays 4-byte.
 *   - FP8 is OCP E4M3 ("fn": no infinities, 0x7F/0xFF are NaN, max 448).
 *     BF16 is passed as uint16_t bit patterns.
 *   - Return value 0 (MEGA_MOE_OK) or a negative mega_moe_status; on error
 *     mega_moe_last_error() gives a message for the calling thread.
 *   - Streams are hipStream_t passed as void* (NULL = the null stream).
 */
#ifndef MEGA_MOE_H_
#define MEGA_MOE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mega_moe_status {
    MEGA_MOE_OK = 0,
    MEGA_MOE_ERR_INVALID_ARG = -1,   /* bad shape, null or misaligned pointer   */
    MEGA_MOE_ERR_UNSUPPORTED = -2,   /* device is not gfx950, or option not built */
    MEGA_MOE_ERR_HIP = -3,           /* a HIP runtime call failed               */
    MEGA_MOE_ERR_OUT_OF_MEMORY = -4, /* workspace allocation failed             */
    MEGA_MOE_ERR_DEVICE = -5         /* the device flagged an error (see get_status) */
} mega_moe_status;

/* Device error bits reported by mega_moe_get_status (sticky until read). */
#define MEGA_MOE_DEVERR_BAD_EXPERT 0x1u   /* a topk_idx >= num_experts (route skipped) */
#define MEGA_MOE_DEVERR_WAIT_TIMEOUT 0x2u /* an L2 tile gave up waiting for its L1 tiles */
#define MEGA_MOE_DEVERR_SCALE_RANGE 0x4u  /* an MXFP4 W1 block scale outside 2^-23..2^13 */

/*
 * Layer configuration (SM90 design 16.1: the expert count, top-k, the
 * per-rank token bound and the activation options are fixed per layer).
 */
typedef struct mega_moe_config {
    int32_t num_experts;      /* E, local experts, >= 1                          */
    int32_t hidden;           /* H, multiple of 128                              */
    int32_t intermediate;     /* I, multiple of 128 (W1 has 2*I rows)            */
    int32_t num_topk;         /* k, 1 <= k                                        */
    int32_t max_tokens;       /* largest T a forward call may pass, >= 0          */
    float activation_clamp;   /* > 0: gate and up are clamped to [-clamp, clamp]
                                 before SwiGLU (SM90 design 10.1 step 3);
                                 +inf: no clamp                                  */
    int32_t fast_math;        /* 0: expf and IEEE division in SiLU; 1: hardware
                                 exp2 and reciprocal (a few float32 ulps)        */
    int32_t block_m;          /* 0 = automatic (SM90 design 13.1), else 32/64/128 */
    int32_t l2_n_major;       /* -1 automatic (12.2), 0 M-major, 1 N-major L2 order;
                                 the N-major schedule (large batches) also lets
                                 workgroups whose XCD ran out of tiles take L2
                                 tiles queued on other XCDs                      */
    int32_t block_n;          /* output columns per expert-kernel tile: 0 = automatic,
                                 128, or 256 (needs 2I % 256 == 0, H % 256 == 0 and
                                 block_m != 32) */
    int32_t split_l2_cus;     /* 0: one persistent kernel takes the L1 and L2 tiles.
                                 n > 0: the L1 and L2 tiles run as two concurrent
                                 kernels on streams of their own (the green-context
                                 split of the PR357 review, sections 1 and 5.2): the
                                 L2 kernel gets n CUs' worth of workgroups on every
                                 XCD, the L1 kernel the rest; n < CUs per XCD (32) */
    int32_t keep_pool;        /* 0 (default): the L1 tiles read each route's row of x,
                                 its scales and top-k weight in place.  1: the dispatch
                                 also copies them into the expert pool (the pages'
                                 pull into the pool, SM90 design 9.2) so that the
                                 l1_* views show them; results are the same */
    int32_t split_l2_xcds;    /* 0: off.  n > 0: the L1 and L2 tiles run on
                                 disjoint sets of XCDs (accelerator dies of 32 CUs)
                                 inside the one persistent launch: the workgroups of
                                 the last n XCDs take only L2 tiles, the others only
                                 L1 tiles, and every pool block's L1 output is
                                 written back through memory for the L2 set (the
                                 green-context split of the PR357 review, sections 1
                                 and 5.2, with partitions of whole dies).  n < the
                                 device's XCD count (8); excludes split_l2_cus.
                                 Results are the same */
} mega_moe_config;

typedef struct mega_moe_handle mega_moe_handle;

/*
 * Validates cfg (H % 128 == 0, I % 128 == 0, k >= 1, E >= 1, unsupported
 * options rejected) on the current HIP device, checks that it is gfx950 and
 * that its XCDs pass mega_moe_check_xcd_layout (with the XCD ids a small
 * probe kernel reports; UNSUPPORTED otherwise), and allocates the
 * handle-owned workspace for max_tokens (re-quantised activations, BF16
 * partials, counters, metadata; the pool copies only with keep_pool).
 * Synchronises the device.  *out is set to NULL on error.
 */
int mega_moe_create(const mega_moe_config* cfg, mega_moe_handle** out);

/*
 * One forward pass of the layer, asynchronous on `stream` (no host
 * synchronisation, no allocation, no memory sets: every counter it uses is
 * reset by its own kernels, so a call may be captured in a HIP graph and the
 * graph replayed; the split phases, split_l2_cus > 0, fork to streams of
 * their own and are not meant for capture).  Shapes (T = num_tokens):
 *   x            [T, H]            uint8 E4M3 activations
 *   x_sf         [T, H/128]        float scale per token per 128 channels
 *   topk_idx     [T, k]            int32 expert of each slot; < 0 = inactive
 *                                  slot; >= E sets MEGA_MOE_DEVERR_BAD_EXPERT
 *                                  and the slot is treated as inactive
 *   topk_weights [T, k]            float
 *   w1           [E, 2I, H]        uint8 E4M3, rows gate/up interleaved by 8:
 *                                  row 16g+r (r < 8) is the gate row of output
 *                                  8g+r, row 16g+8+r its up row (SM90 design 15.1)
 *   w1_sf        [E, 2I/128, H/128] float, one per 128x128 block of w1 as stored
 *   w2           [E, H, I]         uint8 E4M3
 *   w2_sf        [E, H/128, I/128] float
 *   y            [T, H]            uint16 BF16 output; rows of tokens with no
 *                                  active slot are +0
 * num_tokens == 0 is a valid no-op; num_tokens > max_tokens is INVALID_ARG.
 * One handle must not run on two streams at once (the workspace is shared);
 * every call resets the workspace state it uses, so calls may follow each
 * other freely on one stream.
 */
int mega_moe_forward(mega_moe_handle* h, int32_t num_tokens,
                     const uint8_t* x, const float* x_sf,
                     const int32_t* topk_idx, const float* topk_weights,
                     const uint8_t* w1, const float* w1_sf,
                     const uint8_t* w2, const float* w2_sf,
                     uint16_t* y, void* stream);

/*
 * mega_moe_forward with MXFP4 weights: the FP4 E2M1 weights with UE8M0 scale
 * factors, one per 32 K elements, of the SM100 kernel (SM90 design 2.1 and
 * 15.2); activations, routing and output as in mega_moe_forward.
 *   w1        [E, 2I, H/2]  uint8, two E2M1 codes per byte, the even K in the
 *                           low nibble; rows gate/up interleaved by 8 as in
 *                           mega_moe_forward
 *   w1_scale  [E, 2I, H/32] uint8 UE8M0: element c of row n is
 *                           e2m1(code) * 2^(w1_scale[n][c/32] - 127)
 *   w2        [E, H, I/2]   uint8, E2M1 pairs
 *   w2_scale  [E, H, I/32]  uint8 UE8M0
 * The L1 product is exact (F16 matrix cores on the scaled codes) when every
 * w1_scale lies in [104, 140] (block scales 2^-23 .. 2^13); a block outside
 * that range sets MEGA_MOE_DEVERR_SCALE_RANGE and the rows of its tile are
 * unspecified.  w2_scale may be any finite exponent (0..254).  The tiles are
 * 128 columns wide whatever cfg.block_n says.  Errors as mega_moe_forward.
 */
int mega_moe_forward_mxfp4(mega_moe_handle* h, int32_t num_tokens,
                           const uint8_t* x, const float* x_sf,
                           const int32_t* topk_idx, const float* topk_weights,
                           const uint8_t* w1, const uint8_t* w1_scale,
                           const uint8_t* w2, const uint8_t* w2_scale,
                           uint16_t* y, void* stream);

/*
 * mega_moe_forward without a handle, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It calls no hipMalloc, hipFree or other allocating
 * routine.  Its workspace is a device array inside the library of
 * MEGA_MOE_NOALLOC_SCRATCH_BYTES (128 MiB), one per GPU, held from the first
 * use until the process ends.
 *   cfg         as for mega_moe_create; keep_pool, split_l2_cus and
 *               split_l2_xcds must be 0.
 *               num_tokens <= cfg->max_tokens.
 *   num_tokens  a call needs mega_moe_workspace_bytes(cfg with max_tokens =
 *               num_tokens) + 256 bytes of the array; a larger call returns
 *               MEGA_MOE_ERR_INVALID_ARG (up to 948 tokens of top-8 at hidden 7168,
 *               intermediate 2048 and 32 experts; a handle has no such limit).
 *   tensors     as for mega_moe_forward (FP8 weights).
 *   dev_errors  optional device word (NULL: discarded) into which the call
 *               ORs its MEGA_MOE_DEVERR_* bits on the stream, after its last
 *               kernel; each call starts with no bits set.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (two streams, two threads) race and
 * must be ordered by the caller.  The first call on each device does a
 * one-time host set-up (device checks and the array's address) and issues one
 * small clearing kernel on `stream`; later calls launch the same kernels as
 * mega_moe_forward and nothing else.  Errors as mega_moe_forward.
 */
#define MEGA_MOE_NOALLOC_SCRATCH_BYTES (128u << 20)
int mega_moe_forward_noalloc(const mega_moe_config* cfg, int32_t num_tokens,
                             const uint8_t* x, const float* x_sf,
                             const int32_t* topk_idx, const float* topk_weights,
                             const uint8_t* w1, const float* w1_sf,
                             const uint8_t* w2, const float* w2_sf,
                             uint16_t* y, uint32_t* dev_errors, void* stream);

/* Frees the workspace and the handle; NULL is accepted. */
int mega_moe_destroy(mega_moe_handle* h);

/*
 * Synchronises `stream`, then returns (and clears) the sticky device error
 * bits (MEGA_MOE_DEVERR_*) as a non-negative value, or a negative status.
 */
int mega_moe_get_status(mega_moe_handle* h, void* stream);

/* Message for the last non-zero return on the calling thread ("" if none). */
const char* mega_moe_last_error(void);

/*
 * The device check mega_moe_create applies (host-only; needs no GPU).  The
 * expert kernel keeps one work queue per XCD (accelerator die with its own
 * L2), so the L1 tiles of a pool block and the L2 tiles that read their
 * output run on one XCD and meet in its L2 (the single-GPU form of the L2
 * arrival mask handoff, SM90 design 14.3).  MEGA_MOE_OK when num_xcds is in
 * 1..16 and divides num_cus and, if seen_ids is non-zero (a mask of the XCD
 * ids workgroups reported, bit i for id i), the ids number num_xcds and fall
 * into num_xcds distinct queues (id % num_xcds); MEGA_MOE_ERR_UNSUPPORTED
 * otherwise.
 */
int mega_moe_check_xcd_layout(int32_t num_xcds, int32_t num_cus, uint32_t seen_ids);

/* Workspace bytes mega_moe_create would allocate for cfg (-1 if invalid).
 * Host-only; needs no GPU. */
int64_t mega_moe_workspace_bytes(const mega_moe_config* cfg);

/* Row alignment of every expert's pool segment (= the largest BLOCK_M, 128;
 * SM90 design 13.1).  Host-only. */
int32_t mega_moe_token_alignment(void);

/*
 * Host plan of one call (SM90 design 12.2 and 13.1): expected routes per
 * expert T*k/E; BLOCK_M chosen from it (thresholds measured for this kernel
 * on MI355X: <= 50.5 -> 64, else 128) unless cfg->block_m forces one; the
 * tile width block_n (unless cfg->block_n forces one); and whether the tiles
 * run N-major (expected >= 256, unless forced).  Host-only; needs no GPU.
 */
typedef struct mega_moe_plan_info {
    float expected_tokens_per_expert;
    int32_t block_m;
    int32_t l2_n_major;
    int32_t l1_n_blocks;      /* 2I / block_n: L1 tiles per pool block */
    int32_t l2_n_blocks;      /* H / block_n: L2 tiles per pool block */
    int32_t block_n;          /* output columns per expert-kernel tile */
} mega_moe_plan_info;
int mega_moe_plan(const mega_moe_config* cfg, int32_t num_tokens, mega_moe_plan_info* out);

/*
 * The expert kernel's tile order for a plan (a host-side query; needs no GPU).
 * block_start[e] is expert e's first pool block, block_start[E] the number M
 * of pool blocks (host array of num_experts + 1 non-decreasing entries from
 * 0; for a forward call, block_start[e + 1] - block_start[e] is
 * ceil(counts[e] / plan->block_m)).  The M pool blocks are
 * split into n_xcd contiguous ranges, XCD x taking [x*M/n_xcd,
 * (x+1)*M/n_xcd); that XCD's workgroups take the tiles of its range from its
 * own queue, all L1 tiles (phase 1) before the L2 tiles (phase 2), each tile
 * one pool block times one N block of plan->block_n columns.  Row-major when
 * plan->l2_n_major is 0.  N-major (SM90 design 12.2) otherwise, with groups
 * aligned to experts: each run of one expert's pool blocks inside a range,
 * cut into groups of at most 4 blocks (2 at block_m 64), takes every N block
 * in turn over the group's blocks, so the tiles that read one weight block
 * run together.  Fills pb_out[i], nb_out[i] (host arrays of M * N entries,
 * N = plan->l1_n_blocks or plan->l2_n_blocks) with the pool block and N
 * block of the i-th tile: XCD 0's tiles in queue order, then XCD 1's, and so
 * on.  Returns MEGA_MOE_ERR_INVALID_ARG for a NULL argument, a block_m other
 * than 32/64/128, num_experts < 1, a block_start that does not start at 0 or
 * decreases, n_xcd outside [1, 16] or a phase other than 1 or 2.
 */
int mega_moe_tile_order(const mega_moe_plan_info* plan, int32_t num_experts,
                        const int32_t* block_start, int32_t n_xcd, int32_t phase,
                        int32_t* pb_out, int32_t* nb_out);

/*
 * Device views of the intermediates of the last forward call (the buffer views
 * of SM90 design 16.1 / "PR357 review" 3.1), valid once its stream has
 * synchronised and until the next call.  P = pool_rows_capacity.
 */
typedef struct mega_moe_views {
    int32_t* counts;        /* [E]     routes per expert                         */
    int32_t* offsets;       /* [E+1]   pool segment starts, 128-aligned          */
    int32_t* slot_map;      /* [T*k]   pool row of route t*k+j, -1 if inactive   */
    int32_t* src;           /* [P]     route t*k+j held by a pool row, -1 = pad  */
    uint8_t* l1_acts;       /* [P, H]  pool of FP8 rows (allocated and written
                               only when the config sets keep_pool, else NULL)   */
    float* l1_acts_sf;      /* [H/128, P] their scales (pool-row minor; keep_pool,
                               else NULL)                                        */
    float* l1_topk_weights; /* [P]     their top-k weights (keep_pool, else NULL) */
    uint8_t* l2_acts;       /* [P, I]  re-quantised SwiGLU output                */
    float* l2_acts_sf;      /* [I/64, P] its per-64 scales (pool-row minor)      */
    uint16_t* combine_buf;  /* [T*k, H] BF16 L2 partial of each active route     */
    int64_t pool_rows_capacity;
    int32_t last_num_tokens;
} mega_moe_views;
int mega_moe_get_views(mega_moe_handle* h, mega_moe_views* out);

/*
 * Gate/up interleave of W1 for this layer (SM90 design 15.1), run once when
 * the weights are loaded.  In: the plain W1 [E, 2I, H] E4M3 (all I gate rows,
 * then all I up rows) and its float32 scales [E, 2I/128, H/128], one per
 * 128x128 block of that tensor (finite, >= 0).  Out: the stored layout that
 * mega_moe_forward takes (row 16g + r = gate row 8g + r for r < 8, up row
 * 8g + r - 8 otherwise) and one scale per 128x128 block of it: the larger of
 * the block's two source scales; the rows whose source scale is smaller are
 * re-rounded to E4M3 (nearest, ties to even) at the ratio of the two, in
 * float64; a block with both scales 0 gets scale 0 and codes 0.  H and I
 * multiples of 128.  Device pointers owned by the caller; in and out must
 * not overlap; 8-byte aligned codes, 4-byte aligned scales.  Asynchronous on
 * `stream`; W2 needs no transform.
 */
int mega_moe_transform_w1(int32_t num_experts, int32_t hidden, int32_t intermediate,
                          const uint8_t* w1_plain, const float* w1_sf_plain, uint8_t* w1_out,
                          float* w1_sf_out, void* stream);

/*
 * Optional cumulative per-expert route counts (the cumulative local expert
 * receive statistics of the pages' interface, SM90 design 16.1).  Once set,
 * every forward call on the handle adds the number of routes each local
 * expert received in that call to stats[e] (int32 [E], device memory owned
 * by the caller, which zeroes it when it wants to start over), inside the
 * dispatch on the call's stream.  NULL turns it off (the default).  The
 * pointer must stay valid while forward calls that use it may run.
 */
int mega_moe_set_recv_stats(mega_moe_handle* h, int32_t* stats);

/*
 * Optional timing of the three kernel groups of the next forward calls with
 * HIP events recorded on each call's stream (for benchmarks; the layer
 * computes the same thing with or without it).  profile_begin arms it for up
 * to max_calls calls (1..4096); profile_end waits for those events and writes
 * n_out rows of three float milliseconds per call (dispatch, expert kernel,
 * combine) into ms_out[capacity][3], then disarms.  Calls beyond max_calls
 * are not timed.
 */
int mega_moe_profile_begin(mega_moe_handle* h, int32_t max_calls);
int mega_moe_profile_end(mega_moe_handle* h, float* ms_out, int32_t capacity, int32_t* n_out);

#ifdef __cplusplus
}
#endif

#endif /* MEGA_MOE_H_ */
