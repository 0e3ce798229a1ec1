// The expert path of the layer in one persistent kernel: L1 FP8 grouped GEMM
// (gate/up interleaved) with per-128 float scales, SwiGLU times the top-k
// weight, per-row per-64 amax and FP8 re-quantisation, then the L2 FP8
// grouped GEMM with per-64 activation scales and the BF16 partial of every
// route ("MegaMoE SM90 Implementation Design (Final)" 3.3 phases 2-3, 5.1-5.4,
// 10.1, 11.1, 12).
//
// Work is tiles of BLOCK_M pool rows x 128 output columns: L1 tiles (pool
// block pb, 128 interleaved W1 rows = 64 outputs = one per-64 scale group) and
// L2 tiles (pool block pb, 128 columns of H).  The dispatch gives every XCD
// (accelerator die, each with its own L2) a contiguous range of pool blocks,
// and every XCD keeps two queues: the L1 tiles of its pool blocks and their
// L2 tiles.  A workgroup reads its XCD from the XCC_ID hardware register and
// takes tiles with one atomic each, first from its XCD's L1 queue, then from
// its L2 queue.  An L2 tile of pb waits until all 2I/128 L1 tiles of pb have
// published their output through an arrival counter (the role of the L2
// arrival mask of 14.3).  Producer and consumer of pb normally share one XCD
// and so one L2: the producer waits for its stores to be acknowledged before
// bumping the counter and the consumer reads that data with device-scope
// loads (cache policy SC1, which miss the CU's vector L1 and are served by
// the XCD's L2), so no L2 write-back or cache invalidation is needed.  XCDs
// do not run at quite the same speed, and a range of pool blocks is not
// divisible into equal shares, so with large batches (the N-major schedule,
// many pool blocks per XCD) a workgroup whose XCD has no tiles left takes L2
// tiles still queued on other XCDs.  For those, the last L1 tile of every
// pool block writes its XCD's L2 back (an agent-scope release) and marks the
// block published; a workgroup of another XCD waits for that mark and
// invalidates its own L2 (an agent-scope acquire) before reading.  (With few
// pool blocks per XCD the write-backs and invalidations cost more than the
// balance gains: measured on MI355X, prefill 2.4% faster, decode and the
// 4096-token top-2 batch 1.5-2% slower.)  L1
// tiles never wait, and an XCD's workgroups dequeue all of its L1 tiles
// before any L2 tile (of their own XCD or another), so every L1 tile an L2
// tile waits for is taken by a running workgroup that finishes it: the wait
// always ends whatever the number of co-resident workgroups; it is still
// bounded by a spin limit that raises MEGA_MOE_DEVERR_WAIT_TIMEOUT.  With
// the L1 and L2 phases on disjoint XCD sets (the argument phase = 3 + n) the
// dispatch gives the pool blocks to XCDs [0, n) only, their workgroups take
// only L1 tiles and publish every pool block through memory, and the
// workgroups of the other XCDs take only L2 tiles, all of them through the
// cross-XCD path above.
//
// Matrix core use (CDNA4).  The FP8 MFMA of gfx950 does not sum its
// products exactly: within a group of adjacent K it aligns them to the
// largest with fewer than 18 bits, so 448*448 + 1 loses the 1 (measured).
// The L1 output is re-quantised to FP8 and must reproduce the exact-dot
// codes, so the L1 GEMM converts its FP8 operand fragments to F16 in
// registers (v_cvt_scalef32_pk_f16_fp8, exact for every E4M3 value) and runs
// v_mfma_f32_32x32x16_f16, whose products are exact and whose sums round in
// float32.  The L2 result only feeds BF16 partials and stays on
// v_mfma_f32_32x32x64_f8f6f4 with FP8 operands.  Scales are applied on the
// float accumulators: L1 promotes once per 128-K block (acc += (sa*sw) * D),
// L2 once per 64-K half (acc += (sa_half*sw) * D_half), as 5.3 and 5.4
// describe.
//
// MXFP4 weights (the SM100 kernel's FP4 E2M1 codes with a UE8M0 scale per
// 32 K, same page 2.1 and 15.2) run the same tiles from a second set of
// instances: weight rows of 64 bytes per step plus the step's scale dword of
// every row.  L1 converts the codes to F16 with the block scale folded in
// (v_cvt_scalef32_pk_f16_fp4, exact for scales 2^-23 .. 2^13; others raise
// MEGA_MOE_DEVERR_SCALE_RANGE) and keeps the exact F16 products; L2 feeds
// the codes to the scaled MFMA with FP4 weights and FP8 activations, whose
// per-lane E8M0 scale is exactly one 32-wide block of the lane's row.
//
// Memory pipeline.  A workgroup is 4 waves.  Each 128-K step of a tile is one
// LDS stage: BLOCK_M activation rows and 128 weight rows of 128 bytes, then
// the step's per-row activation scales.  Stages are filled by direct
// global-to-LDS buffer loads (16 bytes per lane, no register staging), S
// stages deep: at step kb the loads of step kb + S - 1 are issued into the
// stage that step kb - 1 used, after one wait (this wave's loads of step kb
// done) and one barrier (every wave's).  Rows are 128 bytes; the 16-byte
// chunk c of row n sits at position c ^ f(n), f(n) = (n & 7) ^ ((n >> 3) & 1),
// so each load instruction covers 8 whole rows (fully coalesced) and the MFMA
// fragment reads (32 rows, one chunk each) hit distinct banks.  The tile's
// 32-row slices x 32-column groups are split over the four waves: at 32- and
// 64-row tiles wave w computes column group w over all slices, at 128-row
// tiles each wave computes 2 slices x 2 column groups (a slice's A operand
// and a group's B operand are then converted and read once for two output
// blocks).  Each wave sums the whole K step of its blocks, so no partial sums
// cross waves.  The weights are the MFMA's A operand and the activations its
// B operand, so a 32x32 result block is transposed: lane l holds activation
// row l%32 and its register v weight row 8(v/4) + 4(l/32) + v%4.  A lane then
// needs the scale of one activation row per block (one LDS read and one
// multiply), and since a column group's 32 stored W1 rows are four interleave
// groups of 8 (gate, up, gate, up), registers v and v + 4 of one lane hold
// the gate and up values of the same output.  32-row slices that hold no
// routes are skipped.
#include <hip/hip_runtime.h>

#include "moe_args.h"
#include "schedule.h"
#include "mega_moe.h"

namespace mega_moe {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int BK = 128;              // K elements per step (bytes of an FP8 row)
constexpr int MAX_W_SF = 64;         // K scale blocks of a weight row block (H/128, I/128 <= 64)
constexpr int W_FP8 = 0;             // weight formats: FP8 E4M3 with float 128x128 block scales
constexpr int W_MXFP4 = 1;           // FP4 E2M1 pairs with a UE8M0 scale per 32 K of a row

__device__ __forceinline__ v16f mfma_f8(const v8i& a, const v8i& b, const v16f& c) {
    // scale operands 0 select the plain (unscaled) FP8 x FP8 instruction
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// FP4 E2M1 weights (A: 32 values of one row, four dwords, the lane's 32-wide
// K block) times FP8 activations (B), the A values scaled by 2^(scale_a - 127)
// in the instruction (the lane's UE8M0 byte in bits 0..7).
__device__ __forceinline__ v16f mfma_mx(const v4i& a, const v8i& b, const v16f& c, int scale_a) {
    const v8i a8 = v8i{a[0], a[1], a[2], a[3], 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b, c, 4, 0, 0, scale_a, 0, 127);
}

__device__ __forceinline__ v16f mfma_f16(const v8h& a, const v8h& b, const v16f& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Buffer resource over `bytes` bytes at `base` (gfx9 word 3: raw 32-bit data).
// Loads whose per-lane offset lies beyond the range return zero (a direct
// load to LDS writes zero for those lanes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    // every operand here is wave-uniform; say so, so the descriptor lives in SGPRs
    const uint64_t p = (uint64_t)(uintptr_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    void* q = (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(q, 0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                             0x00020000);
}

// 16 bytes per lane from global memory straight into LDS: lane L of the wave
// writes lds + 16 L (lds must be the same for the whole wave).  AUX is the
// cache policy; SC1 (device scope) misses the CU's vector L1 and reads the
// XCD's L2, for data another CU of the XCD wrote in this launch; CP_NT
// (non-temporal) streams data read once per call past the caches.
constexpr int SC1 = 16;
constexpr int CP_NT = 2;
template <int AUX = 0>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, int voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS_AS void*)lds, 16, voff, soff, 0, AUX);
}

// The same with 4 bytes per lane: lane L writes lds + 4 L.
template <int AUX = 0>
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint8_t* lds, int voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS_AS void*)lds, 4, voff, soff, 0, AUX);
}

// Row swizzle of the stage layout (see the header).
__device__ __forceinline__ int row_swz(int n) { return (n & 7) ^ ((n >> 3) & 1); }

// Chunk swizzle of the 64-byte MXFP4 weight rows of a stage: the 16-byte chunk
// c of row n sits at position c ^ swz4(n), so the 8-byte part reads of 32
// rows spread over the banks (two-way at most).
__device__ __forceinline__ int swz4(int n) { return (n >> 1) & 3; }

// ---------------------------------------------------------------------------
// Operand fragments.  The MFMA operand of one 32-row (A) or 32-column (B)
// slice for a 64-K half h: lane L = r + 32g holds row r, K bytes 64h + 32p +
// 16g + [0,16) for p = 0, 1 (A and B alike, so each MFMA sums exactly the
// products of its half).
// ---------------------------------------------------------------------------
__device__ __forceinline__ v8i read_frag(const uint8_t* region, int s, int h) {
    const int L = threadIdx.x & 63;
    const int r = L & 31, g = L >> 5;
    const uint8_t* row = region + (32 * s + r) * 128;
    const int f = row_swz(r);
    const v4i q0 = *reinterpret_cast<const v4i*>(row + 16 * ((4 * h + g) ^ f));
    const v4i q1 = *reinterpret_cast<const v4i*>(row + 16 * ((4 * h + 2 + g) ^ f));
    return v8i{q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
}

// Both 64-K halves of slice s: dwords 0-7 half 0, dwords 8-15 half 1.
struct Frag {
    v8i h[2];
};

__device__ __forceinline__ Frag read_frag2(const uint8_t* region, int s) {
    return Frag{read_frag(region, s, 0), read_frag(region, s, 1)};
}

// Eight FP8 values (dwords 2q, 2q+1 of a half fragment) as one 16-K F16
// operand.  A and B convert alike, so the four F16 MFMAs of a half still sum
// all 64 of its products.
__device__ __forceinline__ v8h f16_part(const v8i& f, int q) {
    const int d0 = f[2 * q], d1 = f[2 * q + 1];
    const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, false);
    const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, true);
    const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, false);
    const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, true);
    return v8h{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// The raw 16 bytes of parts 2m and 2m + 1 (p = 4h + q) of slice (or column
// group) s: one LDS read.  K bytes 16m + [0,16) of the row for the lane's
// half, in the chunk order read_frag uses.
__device__ __forceinline__ v4i frag_pair_raw(const uint8_t* region, int s, int m) {
    const int L = threadIdx.x & 63;
    const int r = L & 31, g = L >> 5;
    const uint8_t* row = region + (32 * s + r) * 128;
    const int chunk = (4 * (m >> 1) + 2 * (m & 1) + g) ^ row_swz(r);
    return *reinterpret_cast<const v4i*>(row + 16 * chunk);
}

// Dwords 2h, 2h + 1 of a raw pair (part 2m + h) as one 16-K F16 operand.
__device__ __forceinline__ v8h f16_of_pair(const v4i& raw, int h) {
    const int d0 = raw[2 * h], d1 = raw[2 * h + 1];
    const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, false);
    const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, true);
    const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, false);
    const v2h e = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, true);
    return v8h{a[0], a[1], b[0], b[1], c[0], c[1], e[0], e[1]};
}

// One column group times NJ slices (0 .. NJ-1) of a stage: the group's B
// operand is already converted (b16, one v8h per 16-K part); the slices' MFMA
// chains run interleaved part by part, so consecutive MFMAs are independent,
// and each slice's raw A pair m + 1 is read while pair m is converted.
template <int NJ>
__device__ __forceinline__ void slice_chains(const uint8_t* stg, const v8h (&b16)[8], v16f (&d)[NJ]) {
    const v16f zero = v16f{};
    v4i ra[2][NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) ra[0][j] = frag_pair_raw(stg, j, 0);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        if (m < 3) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) ra[(m + 1) & 1][j] = frag_pair_raw(stg, j, m + 1);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int p = 2 * m + h;
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                d[j] = mfma_f16(b16[p], f16_of_pair(ra[m & 1][j], h), p == 0 ? zero : d[j]);
        }
    }
}

// MXFP4 weight rows in a stage: 64 bytes (128 E2M1 codes) per row.  The
// 8 bytes that pair m (16-K parts 2m, 2m + 1) of lane half g needs: codes
// K = 32m + 16g + [0, 16), the same K the FP8 activation parts carry.  Read
// as an integer vector, like every read of a stage (see lane_row_scale).
typedef int v2i __attribute__((ext_vector_type(2)));
__device__ __forceinline__ v2i fp4_pair_raw(const uint8_t* region, int s, int m) {
    const int L = threadIdx.x & 63;
    const int r = L & 31, g = L >> 5;
    const uint8_t* row = region + (32 * s + r) * 64;
    return *reinterpret_cast<const v2i*>(row + 16 * (m ^ swz4(r)) + 8 * g);
}

// 16 bytes (32 codes, K = 64hh + 32g + [0, 32)) of 64-K half hh for the
// scaled FP4 x FP8 MFMA: one 32-wide K block, the lane's own scale block.
__device__ __forceinline__ v4i fp4_half_raw(const uint8_t* region, int s, int hh) {
    const int L = threadIdx.x & 63;
    const int r = L & 31, g = L >> 5;
    const uint8_t* row = region + (32 * s + r) * 64;
    return *reinterpret_cast<const v4i*>(row + 16 * ((2 * hh + g) ^ swz4(r)));
}

// Eight E2M1 codes (one dword, low nibble first) times `scale` as one F16
// operand.  Exact for scale = 2^x, -23 <= x <= 13 (every product is then an
// F16 value, subnormals included).
__device__ __forceinline__ v8h f16_of_fp4(uint32_t d, float scale) {
    const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, scale, 0);
    const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, scale, 1);
    const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, scale, 2);
    const v2h e = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, scale, 3);
    return v8h{a[0], a[1], b[0], b[1], c[0], c[1], e[0], e[1]};
}

// UE8M0 byte i of w as the float 2^(e - 127) (e = 0 gives 0, e = 255 infinity:
// both fall outside the exact range and are reported).
__device__ __forceinline__ float e8_scale(uint32_t w, int i) {
    return __builtin_bit_cast(float, ((w >> (8 * i)) & 0xFFu) << 23);
}

// The scale dword (four UE8M0 bytes, the step's 32-K blocks) of stored weight
// row 32 s + lane % 32, read as an integer like the fragments: from the
// step's stage (row_bytes 4) or from a four-step block (row_bytes 16, wsc_rows
// already offset to the step's dword).
template <int ROW_BYTES = 4>
__device__ __forceinline__ uint32_t lane_wsc(const uint8_t* wsc_rows, int s) {
    return (uint32_t)*reinterpret_cast<const int*>(wsc_rows + ROW_BYTES * (32 * s + (threadIdx.x & 31)));
}

// The scale of this lane's row of a 32-row slice (result blocks are
// transposed: a lane holds one activation row).  Every read of a stage is an
// integer read, reinterpreted where needed: the compiler treats a float- or
// struct-typed LDS read of a stage as possibly aliasing the direct loads
// still in flight into the other stages and would drain all of them
// (vmcnt(0)) before it, while the k loop's wait and barrier already order
// these reads.  (Issuing them as inline assembly instead is unsafe: the
// compiler then cannot insert the wait states between an MFMA still reading
// a register and the LDS read that overwrites it.)
__device__ __forceinline__ float lane_row_scale(const uint8_t* sf_rows, int slice) {
    const int r = 32 * slice + (threadIdx.x & 31);
    return __builtin_bit_cast(float, *reinterpret_cast<const int*>(sf_rows + 4 * r));
}

// Two floats as packed BF16 (lo in bits 0-15), rounded to nearest even, NaN
// kept as a quiet NaN: one v_cvt_pk_bf16_f32 (measured on MI355X identical
// to integer round-to-nearest-even of the bit pattern for every class of
// input, subnormals and ties included).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// silu(g) * u of one output: the optional activation clamp of both values
// ("MegaMoE SM90 Implementation Design (Final)" 10.1 step 3; +inf leaves
// every finite value unchanged), then g / (1 + e^-g), with the accurate expf
// and an IEEE division, or with the hardware exp2 and reciprocal (a few
// float32 ulps) when FAST.
template <bool FAST>
__device__ __forceinline__ float silu_up(float g, float u, float clamp) {
    g = fminf(fmaxf(g, -clamp), clamp);
    u = fminf(fmaxf(u, -clamp), clamp);
    if constexpr (FAST) {
        const float ex = __builtin_amdgcn_exp2f(-g * 1.44269504088896340736f);
        return g * __builtin_amdgcn_rcpf(1.0f + ex) * u;
    } else {
        return g / (1.0f + expf(-g)) * u;
    }
}

// The value of another lane by a DPP move (CTRL: a quad_perm pattern).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// One instance per tile shape and weight format: BLOCK_M = 32 MS pool rows x
// BN output columns (128 or 256; 128 for MXFP4 weights).  A tile has BN/32
// waves, one per 32-column group.
template <int MS, int BNT, int WF = W_FP8>
struct Cfg {
    static constexpr bool MX = WF == W_MXFP4;
    static constexpr int PBM = 32 * MS;                   // pool rows per pool block
    // 128-row FP8 tiles on 128 columns hold one more 32-row slice: an expert's
    // last pool block, when it has at most 32 rows, joins the tile of the
    // block before it, so that its weights stream once (the LDS of this
    // configuration has room for the slice; the others do not)
    static constexpr int XS = merge_tail_for(MX, 32 * MS, BNT) ? 1 : 0;
    static constexpr int SL = MS + XS;                    // 32-row slices per tile
    static constexpr int BM = 32 * SL;                    // tile rows (at most)
    static constexpr int BN = BNT;                        // output columns per tile
    static constexpr int NW = BN / 32;                    // waves per workgroup
    static constexpr int NT = 64 * NW;                    // threads per workgroup
    static constexpr int NSB = BN / 128;                  // 128-row weight scale blocks per tile
    static constexpr int B_ROW = MX ? BK / 2 : BK;        // weight bytes per row per step
    static constexpr int A_BYTES = BM * BK;               // activation rows of a stage
    static constexpr int B_BYTES = BN * B_ROW;            // weight rows of a stage
    // UE8M0 scales of the weight rows: in the stage (one dword per row and
    // step), or, on tiles below 128 rows, in blocks of four steps (16 bytes
    // per row, double buffered outside the stages)
    static constexpr bool WSC_BLOCK = MX && MS <= 2;
    static constexpr int WSC_BYTES = MX && !WSC_BLOCK ? BN * 4 : 0;
    static constexpr int SF_BYTES = 2 * BM * 4;           // per-row scales of a step (2 halves in L2)
    static constexpr int OFF_B = A_BYTES;
    static constexpr int OFF_WSC = OFF_B + B_BYTES;
    static constexpr int OFF_SF = OFF_WSC + WSC_BYTES;
    static constexpr int STAGE = OFF_SF + SF_BYTES;
    // 128-column tiles: two workgroups share a CU (each SIMD runs one wave of
    // each) with half of the 160 KB of LDS each: 3 stages at 32- and 64-row
    // tiles, 2 at 128-row tiles (MXFP4 weights, half the bytes: 4 and 3).
    // 256-column tiles: one eight-wave workgroup per CU (two waves per SIMD)
    // with 3 stages.  While one workgroup (or wave) fills or drains its
    // pipeline at a tile boundary, or waits for an L1 tile, the other keeps
    // loading.
    static constexpr int WPC = BN == 128 ? 2 : 1;
    // Cache policy of the weight rows.  On the 32- and 64-row tiers (few
    // routes per expert) every weight byte is read once per call, in whole
    // 128-byte lines: non-temporal loads, measured on MI355X 8% faster on the
    // 128-token decode batch (a plain streaming read of 940 MB this way runs
    // at 6.9 TB/s, against 6.0 TB/s with the default policy).  Not for the
    // 128-row tier, where the tiles of a group share weight blocks through the
    // L2 (5-7% slower there), nor for MXFP4 rows, whose 64 bytes per step read
    // each line in two halves a step apart (19% slower).
    static constexpr int AUX_W = !MX && MS <= 2 ? CP_NT : 0;
    static constexpr int S = MX ? (MS == 4 ? 3 : 4) : (BN == 128 && MS == 4 ? 2 : 3);
    static constexpr int A_BLK = A_BYTES / 1024;          // 1 KB load blocks of activation rows
    static constexpr int B_BLK = B_BYTES / 1024;          // ... and of weight rows
    static constexpr int B_RPB = 1024 / B_ROW;            // weight rows per block
    static constexpr int PT = (A_BLK + B_BLK) / NW;       // 1 KB blocks per wave per step
    static constexpr int A_J = A_BLK / NW;                // of which activation rows
    static constexpr int LPS = PT + 1 + (MX ? 1 : 0);     // load instructions per wave per step
    static constexpr int WAIT = (S - 2) * LPS;            // loads younger than the current step
    static constexpr int OFF_WSB = S * STAGE;             // scale blocks [2][BN][16 bytes]
    static constexpr int OFF_DUMMY = OFF_WSB + (WSC_BLOCK ? 2 * BN * 16 : 0);  // 16 bytes per wave
    static constexpr int OFF_TILE = OFF_DUMMY + (WSC_BLOCK ? 64 * NW / 4 : 0);  // per-tile area
    static constexpr int HS = BN / 2 + 4;                 // L1 epilogue h row stride (floats)
    // L2 epilogue BF16 row stride (elements): 16 bytes past a multiple of the
    // 256 bytes that span the 64 LDS banks, so the 8-byte writes of one
    // column group's 32 rows (and the two lane halves) fall on distinct banks
    static constexpr int YS = BN + 8;
    static constexpr int LDS_BYTES = OFF_TILE + MAX_W_SF * NSB * 4 + BM * 4 + 16 + 2 * BM * 4;
    static_assert((A_BLK + B_BLK) % NW == 0 && A_BLK % NW == 0, "row blocks per wave");
    static_assert(!MX || BN == 128, "MXFP4 weights use 128-column tiles");
    static_assert(WAIT < 64, "vmcnt range");
    // the extra slice's loads are skipped on tiles without it, so the number
    // of loads per step varies: only the full wait of a two-stage ring allows that
    static_assert(XS == 0 || S == 2, "extra slice needs the two-stage ring");
    static_assert(WPC * LDS_BYTES <= 160 * 1024, "LDS per CU");
    static_assert(BM * YS * 2 <= S * STAGE && BM * HS * 4 <= S * STAGE, "epilogue buffers");
};

template <int MS, int BNT, int WF = W_FP8>
struct Lds {
    using C = Cfg<MS, BNT, WF>;
    uint8_t* base;
    __device__ uint8_t* stage(int i) const { return base + i * C::STAGE; }
    __device__ uint8_t* wsb(int buf) const { return base + C::OFF_WSB + buf * C::BN * 16; }
    __device__ uint8_t* dummy() const { return base + C::OFF_DUMMY; }
    // weight scales of the tile (FP8 weights): [NSB][KB]
    __device__ float* w_sf() const { return reinterpret_cast<float*>(base + C::OFF_TILE); }
    __device__ float* row_w() const { return w_sf() + MAX_W_SF * C::NSB; }   // top-k weight per row (L1)
    // [0] the dequeued tile, [1] the XCD whose queue it came from, [3] 1 for
    // an L1 tile, [4, 4 + BM) the L1 tile's x rows or the L2 tile's routes
    // (-1 past its valid rows), [4 + BM, 4 + 2 BM) 1 for the L1 rows whose
    // row_w holds the top-k weight times 2^64 (a tiny weight), else 0
    __device__ int* tile() const { return reinterpret_cast<int*>(row_w() + C::BM); }
    __device__ int* row_tiny() const { return tile() + 4 + C::BM; }
};

// Issues the direct loads of one step.  Wave w fills the 1 KB blocks
// b = NW j + w of the stage: activation rows first (8 rows of 128 bytes per
// block), then weight rows (8 FP8 rows of 128 bytes, or 16 MXFP4 rows of 64
// bytes): lane q takes row q / (chunks per row) of its block and the chunk
// whose swizzled position is q % (chunks per row).  Each wave then loads a
// quarter of the step's per-row activation scales (L1 tiles: one float per
// tile row, from that route's row of x_sf; L2 tiles: the two 64-K halves of
// l2_sf, in the pool-minor layout) and, with MXFP4 weights, the UE8M0 scales
// of its 32 weight rows: the step's dword (four 32-K blocks) of every row, or
// on tiles below 128 rows 16 bytes per row (four steps) every fourth step.
// A step past the end (real = false) still issues the same number of
// instructions, from lane 0 only, so every wave's count of outstanding loads
// is the same at every step.
template <int MS, int BNT, int HALVES, int WF = W_FP8>
struct Loader {
    using C = Cfg<MS, BNT, WF>;
    // L2 tiles read the activations and scales their L1 tiles just wrote
    static constexpr int AUX_ACT = HALVES == 2 ? SC1 : 0;
    static constexpr int AUX_W = C::AUX_W;
    static constexpr int PT = C::PT;
    static constexpr int Q = 4 * HALVES * C::BM / C::NW;  // scale bytes per wave
    __amdgpu_buffer_rsrc_t ra, rb, rs, rw;
    int voff[C::A_J];   // the wave's activation blocks
    int voff_b;         // its first weight block; block A_J + i lies i * bstep bytes further
    int bstep;
    int sf_voff;
    int wsc_voff;
    int w;
    int sf_step;     // bytes between the scale groups of consecutive steps
    bool xs_on;      // the tile has rows in its extra slice (more than PBM rows)

    // ra: activation rows (row_a bytes each), rb: weight rows (row_b bytes),
    // rs: activation scales, rw: UE8M0 scale rows of the weight rows (row_w
    // bytes; MXFP4 only).  L1 tiles (HALVES 1) gather: arow[n] is the row of
    // x that tile row n reads, or a row past the end of ra for the padding
    // rows, which then load as zeros; their scales are one float per row:
    // on 128-row tiles from the dispatch's pool-ordered copy (rs starts at
    // the tile's first pool row, row stride 4 bytes, step kb at byte 4 P kb),
    // else gathered from x_sf like the rows (row stride row_s bytes, step kb
    // at byte 4 kb).  L2 tiles read the pool in order (arow unused) and its
    // pool-minor scales (row stride P).
    // rows: the tile's rows; the activation rows of the extra slice load only
    // when it has some (a tile of at most PBM rows issues what a PBM-row
    // configuration would)
    __device__ Loader(__amdgpu_buffer_rsrc_t ra_, __amdgpu_buffer_rsrc_t rb_, int row_a, int row_b,
                      __amdgpu_buffer_rsrc_t rs_, int P, __amdgpu_buffer_rsrc_t rw_, int row_w, int rows,
                      const int* arow = nullptr, int row_s = 0)
        : ra(ra_), rb(rb_), rs(rs_), rw(rw_), xs_on(rows > C::PBM) {
        const int lane = threadIdx.x & 63;
        w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        // (consecutive weight blocks of a wave are NW blocks, 32 FP8 or 64
        // MXFP4 rows, apart, with the same swizzle: one offset and a stride)
#pragma unroll
        for (int j = 0; j < C::A_J; ++j) {
            const int n = 8 * (C::NW * j + w) + (lane >> 3);           // activation row
            int src_row = n;
            if constexpr (HALVES == 1) src_row = arow[n];
            voff[j] = src_row * row_a + 16 * ((lane & 7) ^ row_swz(n));
        }
        if constexpr (C::MX) {
            const int n = 16 * w + (lane >> 2);                        // MXFP4 weight row
            voff_b = n * row_b + 16 * ((lane & 3) ^ swz4(n));
            bstep = 16 * C::NW * row_b;
        } else {
            const int n = 8 * w + (lane >> 3);                         // FP8 weight row
            voff_b = n * row_b + 16 * ((lane & 7) ^ row_swz(n));
            bstep = 8 * C::NW * row_b;
        }
        if constexpr (HALVES == 1 && MS == 4) {
            // one scale per lane: rows [w*BM/NW, (w+1)*BM/NW) of the tile, from
            // the dispatch's pool-ordered copy (one contiguous run per step)
            const int n = w * (C::BM / C::NW) + min(lane, C::BM / C::NW - 1);
            sf_voff = n * 4;
            sf_step = P * 4;
        } else if constexpr (HALVES == 1) {
            // one scale per lane: rows [w*BM/NW, (w+1)*BM/NW) of the tile
            const int n = w * (C::BM / C::NW) + min(lane, C::BM / C::NW - 1);
            sf_voff = arow[n] * row_s;
            sf_step = 4;
        } else {
            // scale bytes [w*Q, w*Q + Q) of the step's 2*BM*4-byte scale area
            const int off = w * Q + 16 * lane;
            const int half = off / (C::BM * 4);
            sf_voff = half * P * 4 + (off - half * C::BM * 4);
            sf_step = HALVES * P * 4;
        }
        wsc_voff = (32 * w + (lane & 31)) * row_w;
    }

    // lds_base: the workgroup's LDS (for the scale blocks and the dummy slot)
    __device__ __forceinline__ void issue(uint8_t* stage, int kb, bool real, uint8_t* lds_base) const {
        const int lane = threadIdx.x & 63;
        const int soff_a = real ? kb * BK : 0;
        const int soff_b = real ? kb * C::B_ROW : 0;
#pragma unroll
        for (int j = 0; j < PT; ++j) {
            if (real || lane == 0) {
                if (j < C::A_J) {
                    if (j < C::A_J - C::XS || xs_on)
                        dma16<AUX_ACT>(ra, stage + (C::NW * j + w) * 1024, voff[j], soff_a);
                } else {
                    dma16<AUX_W>(rb, stage + (C::NW * j + w) * 1024, voff_b, soff_b + (j - C::A_J) * bstep);
                }
            }
        }
        if constexpr (HALVES == 1) {
            if (lane < C::BM / C::NW && (real || lane == 0))
                dma4(rs, stage + C::OFF_SF + 4 * w * (C::BM / C::NW), sf_voff, real ? kb * sf_step : 0);
        } else {
            if (lane < Q / 16 && (real || lane == 0))
                dma16<AUX_ACT>(rs, stage + C::OFF_SF + w * Q, sf_voff, real ? kb * sf_step : 0);
        }
        if constexpr (C::WSC_BLOCK) {
            // every fourth step: steps kb .. kb + 3 of the wave's 32 rows, 16
            // bytes each, into buffer (kb / 4) % 2; other steps issue one
            // lane into the wave's dummy slot so the count stays the same
            if (real && (kb & 3) == 0) {
                if (lane < 32)
                    dma16(rw, lds_base + C::OFF_WSB + ((kb >> 2) & 1) * C::BN * 16 + 512 * w, wsc_voff,
                          4 * kb);
            } else if (lane == 0) {
                dma16(rw, lds_base + C::OFF_DUMMY + 16 * w, 0, 0);
            }
        } else if constexpr (C::MX) {
            if (lane < 32 && (real || lane == 0))
                dma4(rw, stage + C::OFF_WSC + 128 * w, wsc_voff, real ? kb * 4 : 0);
        }
    }
};

// Waits for this wave's loads older than the last N, then for every wave.
template <int N>
__device__ __forceinline__ void wait_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// K loop over KB steps; compute(stage, kb) reads only stage.
template <int MS, int BNT, int HALVES, int WF, typename Compute>
__device__ __forceinline__ void k_loop(const Loader<MS, BNT, HALVES, WF>& ld, const Lds<MS, BNT, WF>& lds,
                                       int KB, Compute&& compute) {
    using C = Cfg<MS, BNT, WF>;
    constexpr int S = C::S;
#pragma unroll
    for (int d = 0; d < S - 1; ++d) ld.issue(lds.stage(d), d, d < KB, lds.base);
    int cur = 0;
    for (int kb = 0; kb < KB; ++kb) {
        wait_barrier<C::WAIT>();
        const int nk = kb + S - 1;
        ld.issue(lds.stage(cur == 0 ? S - 1 : cur - 1), nk, nk < KB, lds.base);
        compute(lds.stage(cur), kb);
        cur = cur == S - 1 ? 0 : cur + 1;
    }
    // the trailing loads (past the end) land in stages the epilogue reuses
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
}

// Wave layout of a tile with ACT active 32-row slices.  A full 128-row tile
// is split 2 slices x 2 column groups per wave, so a slice's A operand and a
// column group's B operand are read and converted once for two output
// blocks; any other tile gives wave w column group w over all active slices,
// so no wave idles on a ragged tile.  A 160-row tile (ACT 5) is the 128-row
// grid plus slice 4, which each wave computes for its first column group
// g(0): the upper waves take their two groups in the other order, so that
// the four waves' first groups are the four groups of the tile.
template <int MS, int BNT, int ACT>
struct Lay {
    static constexpr bool GRID = MS == 4 && ACT >= 4;
    static constexpr int NJ = GRID ? 2 : ACT;     // 32-row slices per wave (grid part)
    static constexpr int NG = GRID ? 2 : 1;       // 32-column groups per wave
    static constexpr int XJ = GRID ? ACT - 4 : 0; // extra slices (slice 4, group g(0))
    static constexpr int WC = Cfg<MS, BNT>::NW / 2;   // column-group pairs (GRID)
    int s0, g0, flip;
    __device__ Lay() {
        const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        s0 = GRID ? 2 * (w / WC) : 0;
        g0 = GRID ? 2 * (w % WC) : w;
        flip = XJ > 0 ? (w / WC) & 1 : 0;
    }
    // the wave's column group q (0 .. NG-1)
    __device__ int g(int q) const { return g0 + (q ^ flip); }
    // the 128-row weight scale block of this wave's column groups
    __device__ int sblock() const { return g0 >> 2; }
};

template <int N>
struct IntTag {
    static constexpr int value = N;
};

// Runs fn(IntTag<act>) for the active slice count (1..SL).
template <int SL, typename Fn>
__device__ __forceinline__ void dispatch_act(int act, Fn&& fn) {
    if constexpr (SL >= 5) {
        if (act == 5) { fn(IntTag<5>{}); return; }
    }
    if constexpr (SL >= 4) {
        if (act == 4) { fn(IntTag<4>{}); return; }
        if (act == 3) { fn(IntTag<3>{}); return; }
    }
    if constexpr (SL >= 2) {
        if (act == 2) { fn(IntTag<2>{}); return; }
    }
    fn(IntTag<1>{});
}

// ---------------------------------------------------------------------------
// L1 tile: pool rows [row0, row0 + valid) of expert e, W1 N block nb.
// ---------------------------------------------------------------------------
template <int MS, int BNT, int WF>
__device__ __forceinline__ void l1_tile(const MoeArgs& a, const Lds<MS, BNT, WF>& lds, int e, int pb,
                                        int row0, int valid, int nb) {
    using C = Cfg<MS, BNT, WF>;
    constexpr int BM = C::BM, BN = C::BN, NT = C::NT;
    const int H = a.H;
    const int KB = H / BK;
    const size_t P = a.P_cap;
    const int act = min(C::SL, (valid + 31) / 32);
    const size_t wrow0 = (size_t)e * (2 * a.I) + (size_t)nb * BN;     // first stored W1 row

    if constexpr (!C::MX) {
        // the tile's NSB weight scale rows of W1_sf [E, 2I/128, H/128], contiguous
        const float* wsf = a.w1_sf + ((size_t)e * a.nb1 + nb) * C::NSB * KB;
        for (int i = threadIdx.x; i < C::NSB * KB; i += NT) lds.w_sf()[i] = wsf[i];
    }
    // the tile's rows come straight from x: tile row r < valid is route
    // src[row0 + r] = t*k + j, which reads row t of x and x_sf and takes the
    // top-k weight topk_w[t*k + j] (from the dispatch's copy of it per pool
    // row); padding rows point one row past the end of x, where the buffer
    // loads return zeros
    // A top-k weight below 2^-60 (an underflowed softmax) is kept as
    // w * 2^64: h = silu(g) * u * w would otherwise fall below float32's
    // normal range and lose the bits its codes need; the factor comes back
    // out of the row's scales, exactly, in the quantisation below.
    for (int r = threadIdx.x; r < BM; r += NT) {
        // (every row below valid is a routed row; its weight comes from the
        // dispatch's per-row copy, so the two loads go out together)
        const int f = r < valid ? a.src[row0 + r] : -1;
        const float wt = r < valid ? a.pool_w[row0 + r] : 0.0f;
        const bool tiny = fabsf(wt) < 0x1p-60f;
        lds.row_w()[r] = tiny ? wt * 0x1p64f : wt;
        lds.row_tiny()[r] = tiny ? 1 : 0;
        lds.tile()[4 + r] = f >= 0 ? f / a.k : a.T;
    }
    __syncthreads();
    const int row_b = C::MX ? H / 2 : H;
    const Loader<MS, BNT, 1, WF> ld(
        make_rsrc(a.x, (uint32_t)((size_t)a.T * H)),
        make_rsrc(a.w1 + wrow0 * row_b, (uint32_t)(BN * row_b)), H, row_b,
        MS == 4 ? make_rsrc(a.l1_sf + row0, (uint32_t)(((size_t)(KB - 1) * P + valid) * 4))
                : make_rsrc(a.x_sf, (uint32_t)((size_t)a.T * KB * 4)),
        (int)P,
        make_rsrc(C::MX ? a.w1_e8 + wrow0 * (H / 32) : nullptr, C::MX ? (uint32_t)(BN * (H / 32)) : 0u),
        H / 32, valid, lds.tile() + 4, KB * 4);
    // MXFP4: smallest and largest block scale this lane converted (reported
    // when outside 2^-23 .. 2^13, where the F16 conversion stops being exact)
    float sc_lo = 1.0f, sc_hi = 1.0f;

    const v16f zero = v16f{};
    // ---- epilogue buffer: h of the tile, written from the accumulators ----
    // Each lane forms SwiGLU from a gate and an up accumulator it holds itself
    // (the layout is spelled out at write_h below) and writes h to LDS; then
    // one thread per 16 outputs of a row takes the row amax over its quad of
    // threads (DPP), the exactly rounded scale amax / 448, and writes 16 codes
    // (h * (1 / sf)) as one store.
    constexpr int HS = C::HS;                                           // h row stride (floats)
    float* hbuf = reinterpret_cast<float*>(lds.stage(0));              // [BM][HS]

    dispatch_act<C::SL>(act, [&](auto tag) {
        constexpr int ACT = decltype(tag)::value;
        using LY = Lay<MS, BNT, ACT>;
        const LY ly;
        v16f acc[LY::NJ][LY::NG];
#pragma unroll
        for (int j = 0; j < LY::NJ; ++j)
#pragma unroll
            for (int q = 0; q < LY::NG; ++q) acc[j][q] = v16f{};
        v16f accx = v16f{};   // slice 4 of a 160-row tile, column group g(0)
        // FP8 weights on the 2 x 2 wave grid: the raw products of the previous
        // step and their scales, folded into acc at the start of the next step
        // (zero before the first, so that fold adds nothing)
        v16f dp[LY::NJ][LY::NG];
        float svp[LY::NJ];
#pragma unroll
        for (int j = 0; j < LY::NJ; ++j) {
            svp[j] = 0.0f;
#pragma unroll
            for (int q = 0; q < LY::NG; ++q) dp[j][q] = v16f{};
        }

        k_loop(ld, lds, KB, [&](const uint8_t* stg, int kb) {
            const uint8_t* sfa = stg + C::OFF_SF;
            if constexpr (C::MX) {
                // MXFP4 weights: each pair m of 16-K parts is one 32-K scale
                // block; the codes convert to F16 with the block scale folded
                // in, then the same F16 MFMA chains as FP8 weights
                uint32_t wsc[LY::NG];
#pragma unroll
                for (int q = 0; q < LY::NG; ++q) {
                    if constexpr (C::WSC_BLOCK)
                        wsc[q] = lane_wsc<16>(lds.wsb((kb >> 2) & 1) + 4 * (kb & 3), ly.g(q));
                    else
                        wsc[q] = lane_wsc(stg + C::OFF_WSC, ly.g(q));
                }
                v16f d[LY::NJ][LY::NG];
                if constexpr (LY::GRID) {
                    v2i rb[2][LY::NG];
                    v4i ra[2][LY::NJ];
                    auto read_pair = [&](int buf, int m) {
#pragma unroll
                        for (int q = 0; q < LY::NG; ++q) rb[buf][q] = fp4_pair_raw(stg + C::OFF_B, ly.g(q), m);
#pragma unroll
                        for (int j = 0; j < LY::NJ; ++j) ra[buf][j] = frag_pair_raw(stg, ly.s0 + j, m);
                    };
                    read_pair(0, 0);
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        if (m < 3) read_pair((m + 1) & 1, m + 1);
                        float sc[LY::NG];
#pragma unroll
                        for (int q = 0; q < LY::NG; ++q) {
                            sc[q] = e8_scale(wsc[q], m);
                            sc_lo = fminf(sc_lo, sc[q]);
                            sc_hi = fmaxf(sc_hi, sc[q]);
                        }
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const bool first = m == 0 && h == 0;
                            v8h b16[LY::NG];
#pragma unroll
                            for (int q = 0; q < LY::NG; ++q)
                                b16[q] = f16_of_fp4((uint32_t)rb[m & 1][q][h], sc[q]);
#pragma unroll
                            for (int j = 0; j < LY::NJ; ++j) {
                                const v8h a16 = f16_of_pair(ra[m & 1][j], h);
#pragma unroll
                                for (int q = 0; q < LY::NG; ++q)
                                    d[j][q] = mfma_f16(b16[q], a16, first ? zero : d[j][q]);
                            }
                        }
                    }
                } else {
                    v8h b16[8];
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const v2i raw = fp4_pair_raw(stg + C::OFF_B, ly.g0, m);
                        const float sc = e8_scale(wsc[0], m);
                        sc_lo = fminf(sc_lo, sc);
                        sc_hi = fmaxf(sc_hi, sc);
                        b16[2 * m] = f16_of_fp4((uint32_t)raw[0], sc);
                        b16[2 * m + 1] = f16_of_fp4((uint32_t)raw[1], sc);
                    }
                    v16f dj[LY::NJ];
                    slice_chains<LY::NJ>(stg, b16, dj);
#pragma unroll
                    for (int j = 0; j < LY::NJ; ++j) d[j][0] = dj[j];
                }
                // no weight scale left to apply: promote by the row's x_sf
#pragma unroll
                for (int j = 0; j < LY::NJ; ++j) {
                    const float sa = lane_row_scale(sfa, ly.s0 + j);
#pragma unroll
                    for (int q = 0; q < LY::NG; ++q)
                        acc[j][q] = __builtin_elementwise_fma(d[j][q], v16f(sa), acc[j][q]);
                }
                return;
            }
            const float sw = lds.w_sf()[ly.sblock() * KB + kb];
            if constexpr (LY::GRID) {
                // eight 16-K parts in four pairs; the raw fragments of pair
                // m + 1 (two column groups, two slices) are read while pair m
                // is converted and fed to four independent MFMA chains, so
                // the LDS latency overlaps the matrix work
                static_assert(LY::NG + LY::NJ == 4, "2 x 2 wave blocks");
                if constexpr (LY::XJ > 0) {
                    // slice 4 times column group g(0) first, as its own chain
                    // over the eight parts (the order of every other chain),
                    // folded before the grid's four chains start: at most
                    // four chains are live at a time
                    // (all its fragment pairs read first, so that one LDS
                    // latency precedes the chain instead of one per pair)
                    v4i xb[4], xa[4];
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        xb[m] = frag_pair_raw(stg + C::OFF_B, ly.g(0), m);
                        xa[m] = frag_pair_raw(stg, 4, m);
                    }
                    v16f dx;
#pragma unroll
                    for (int m = 0; m < 4; ++m)
#pragma unroll
                        for (int h = 0; h < 2; ++h)
                            dx = mfma_f16(f16_of_pair(xb[m], h), f16_of_pair(xa[m], h), m == 0 && h == 0 ? zero : dx);
                    accx = __builtin_elementwise_fma(dx, v16f(lane_row_scale(sfa, 4) * sw), accx);
                    // (kept apart from the grid below, whose reads the
                    // scheduler would otherwise hoist into this chain)
                    __builtin_amdgcn_sched_barrier(0);
                }
                // this step's scales, for the fold at the start of the next step
                float svw[LY::NJ];
#pragma unroll
                for (int j = 0; j < LY::NJ; ++j) svw[j] = lane_row_scale(sfa, ly.s0 + j) * sw;
                v4i raw[2][4];
                auto read_pair = [&](v4i* dst, int m) {
#pragma unroll
                    for (int q = 0; q < LY::NG; ++q) dst[q] = frag_pair_raw(stg + C::OFF_B, ly.g(q), m);
#pragma unroll
                    for (int j = 0; j < LY::NJ; ++j) dst[LY::NG + j] = frag_pair_raw(stg, ly.s0 + j, m);
                };
                read_pair(raw[0], 0);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int cb = m & 1;
                    if (m < 3) read_pair(raw[(m + 1) & 1], m + 1);
                    // (the look-ahead reads stay ahead of this pair's work)
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const bool first = m == 0 && h == 0;
                        v8h b16[LY::NG];
#pragma unroll
                        for (int q = 0; q < LY::NG; ++q) b16[q] = f16_of_pair(raw[cb][q], h);
#pragma unroll
                        for (int j = 0; j < LY::NJ; ++j) {
                            const v8h a16 = f16_of_pair(raw[cb][LY::NG + j], h);
#pragma unroll
                            for (int q = 0; q < LY::NG; ++q) {
                                // the previous step's product of this chain is
                                // folded just before the chain restarts, so the
                                // adds overlap this step's LDS reads and first
                                // products instead of trailing the last ones
                                if (first)
                                    acc[j][q] = __builtin_elementwise_fma(dp[j][q], v16f(svp[j]), acc[j][q]);
                                dp[j][q] = mfma_f16(b16[q], a16, first ? zero : dp[j][q]);
                            }
                        }
                    }
                }
#pragma unroll
                for (int j = 0; j < LY::NJ; ++j) svp[j] = svw[j];

            } else {
                // one column group: its B operand converted once per step,
                // then one MFMA chain per active slice, interleaved
                const Frag fb = read_frag2(stg + C::OFF_B, ly.g0);
                v8h b16[8];
#pragma unroll
                for (int p = 0; p < 8; ++p) b16[p] = f16_part(fb.h[p >> 2], p & 3);
                v16f dj[LY::NJ];
                slice_chains<LY::NJ>(stg, b16, dj);
#pragma unroll
                for (int j = 0; j < LY::NJ; ++j) {
                    const float svw = lane_row_scale(sfa, j) * sw;
                    acc[j][0] = __builtin_elementwise_fma(dj[j], v16f(svw), acc[j][0]);
                }
            }
        });

        if constexpr (!C::MX && LY::GRID) {
            // the last step's products
#pragma unroll
            for (int j = 0; j < LY::NJ; ++j)
#pragma unroll
                for (int q = 0; q < LY::NG; ++q)
                    acc[j][q] = __builtin_elementwise_fma(dp[j][q], v16f(svp[j]), acc[j][q]);
        }
        // the k loop ended with a barrier, so the stages are free for h.  In a
        // transposed block, register v of lane l holds stored W1 row
        // 8(v/4) + 4(l/32) + v%4 of the column group for activation row l%32:
        // registers v and v + 4 (v%8 < 4) are the gate and up rows of output
        // 16g + 8(v/8) + 4(l/32) + v%4, so SwiGLU needs no data from another
        // lane, and each lane writes 4 consecutive outputs at a time.
        auto write_h = [&](auto fast) {
            constexpr bool FAST = decltype(fast)::value != 0;
            // the 32 x 32 block r of slice s, column group g
            auto put = [&](const v16f& r, int s, int g) {
                // (the lane's row offset is formed here, not kept in a register
                // from the kernel's start: this kernel uses all 256)
                int lane = threadIdx.x & 31;
                asm volatile("" : "+v"(lane));
                const int row = 32 * s + lane;
                const float wt = lds.row_w()[row];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    float hv[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        hv[v] = silu_up<FAST>(r[8 * half + v], r[8 * half + 4 + v], a.act_clamp) * wt;
                    const int col = 16 * g + 8 * half + 4 * ((threadIdx.x >> 5) & 1);
                    *reinterpret_cast<float4*>(hbuf + row * HS + col) = float4{hv[0], hv[1], hv[2], hv[3]};
                }
            };
#pragma unroll
            for (int j = 0; j < LY::NJ; ++j)
#pragma unroll
                for (int q = 0; q < LY::NG; ++q) put(acc[j][q], ly.s0 + j, ly.g(q));
            if constexpr (LY::XJ > 0) put(accx, 4, ly.g(0));
        };
        if (a.fast_math) write_h(IntTag<1>{});
        else write_h(IntTag<0>{});
    });
    if constexpr (C::MX) {
        if (!(sc_lo >= 0x1p-23f && sc_hi <= 0x1p13f))
            atomicOr(&a.ctrl->error, MEGA_MOE_DEVERR_SCALE_RANGE);
    }

    __syncthreads();
    // BN/32 threads per row, 16 outputs each; the 4 of one 64-output scale
    // group are consecutive lanes (NT and BN/32 are multiples of 4)
    constexpr int PPR = BN / 32;
    for (int t = threadIdx.x; t < PPR * 32 * act; t += NT) {
        const int r = t / PPR, part = t % PPR;
        const float4* src4 = reinterpret_cast<const float4*>(hbuf + r * HS + 16 * part);
        float hv[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 t = src4[q];
            hv[4 * q] = t.x; hv[4 * q + 1] = t.y; hv[4 * q + 2] = t.z; hv[4 * q + 3] = t.w;
        }
        float m = 0.0f;
#pragma unroll
        for (int q = 0; q < 16; ++q) m = fmaxf(m, fabsf(hv[q]));
        m = fmaxf(m, dpp_move<0xB1>(m));                                // quad_perm [1,0,3,2]
        m = fmaxf(m, dpp_move<0x4E>(m));                                // quad_perm [2,3,0,1]
        // codes = h / sf as (h * hsc) * (1 / (sf * ssc)), hsc and ssc powers
        // of two that keep the reciprocal finite and exact in range.  A row
        // whose h carries 2^64 (tiny top-k weight): sf = (amax / 448) * 2^-64
        // rounded once to float32 (via float64), and h / sf = h' / (sf *
        // 2^64).  Otherwise sf = amax / 448 in float32; below 2^-100 (tiny
        // SwiGLU outputs) h and sf are scaled by 2^100 first.  sf = 0 (amax
        // = 0, or amax / 448 below the smallest float) gives codes of zero.
        float sf, hsc, ssc;
        if (lds.row_tiny()[r]) {
            sf = (float)((double)m / 448.0 * 0x1p-64);
            hsc = 1.0f;
            ssc = 0x1p64f;
        } else {
            sf = m / 448.0f;
            hsc = ssc = sf < 0x1p-100f ? 0x1p100f : 1.0f;
        }
        const float inv = sf > 0.0f ? __builtin_amdgcn_rcpf(sf * ssc) : 0.0f;
#pragma unroll
        for (int q = 0; q < 16; ++q) hv[q] *= hsc;
        uint32_t code[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float v0 = fminf(fmaxf(hv[4 * q] * inv, -448.0f), 448.0f);
            float v1 = fminf(fmaxf(hv[4 * q + 1] * inv, -448.0f), 448.0f);
            float v2 = fminf(fmaxf(hv[4 * q + 2] * inv, -448.0f), 448.0f);
            float v3 = fminf(fmaxf(hv[4 * q + 3] * inv, -448.0f), 448.0f);
            int d = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
            code[q] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, d, true);
        }
        if (r < valid) {
            *reinterpret_cast<uint4*>(a.l2_acts + (size_t)(row0 + r) * a.I + nb * (BN / 2) +
                                      part * 16) = uint4{code[0], code[1], code[2], code[3]};
            if ((part & 3) == 0) a.l2_sf[(size_t)(nb * C::NSB + (part >> 2)) * P + row0 + r] = sf;
        }
    }
    // publish: the vector L1 writes through, so once every thread's stores are
    // acknowledged they sit in this XCD's L2, where this XCD's L2 tiles read
    // them.  The last L1 tile of the pool block also writes this XCD's L2 back
    // (an agent-scope release) and then sets READY_PUBLISHED, so that an L2
    // tile taken by a workgroup of another XCD can read the block from memory.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t done =
            __hip_atomic_fetch_add(&a.ready[pb], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
        if (((a.phase == 0 && a.steal) || a.phase >= PHASE_XCD_SPLIT) && done == (uint32_t)a.nb1) {
            // the write-back must be complete before the mark is set: the
            // compiler's own wait after the fence's write-back can be merged
            // away (it was, here), so it is written out
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __hip_atomic_fetch_or(&a.ready[pb], READY_PUBLISHED, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// NB matrix products, each folded into an accumulator with a per-lane scale:
// acc(i) += scale(i) * prod(i), i = 0 .. NB-1.  Product i + 1 is issued
// before the adds of product i (two result buffers), so the vector ALU works
// on one product while the matrix core computes the next; written as plain
// "product, then its adds", the compiler gives every product the same
// result registers and the adds wait out each product's whole latency.
template <int NB, typename Prod, typename Fold>
__device__ __forceinline__ void prod_fold_pipeline(Prod&& prod, Fold&& fold) {
    v16f d[2];
    d[0] = prod(0);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        if (i + 1 < NB) d[(i + 1) & 1] = prod(i + 1);
        fold(i, d[i & 1]);
    }
}

// The same, but the adds of the last product are left to the caller, who gets
// that product back and folds it at the start of the next step: fold_prev
// (the previous step's last product) runs once product 0 is issued, so those
// adds overlap the matrix core instead of waiting out the last product.
template <int NB, typename Prod, typename Fold, typename FoldPrev>
__device__ __forceinline__ v16f prod_fold_carry(Prod&& prod, Fold&& fold, FoldPrev&& fold_prev) {
    v16f d[2];
    d[0] = prod(0);
    fold_prev();
#pragma unroll
    for (int i = 0; i + 1 < NB; ++i) {
        d[(i + 1) & 1] = prod(i + 1);
        fold(i, d[i & 1]);
    }
    return d[(NB - 1) & 1];
}

// ---------------------------------------------------------------------------
// L2 tile: pool rows [row0, row0 + valid) of expert e, W2 N block nb.
// ---------------------------------------------------------------------------
template <int MS, int BNT, int WF>
__device__ __forceinline__ void l2_tile(const MoeArgs& a, const Lds<MS, BNT, WF>& lds, int e, int pb,
                                        int row0, int valid, int nb, bool foreign) {
    using C = Cfg<MS, BNT, WF>;
    constexpr int BM = C::BM, BN = C::BN, NT = C::NT;
    const int I = a.I;
    const int KB = I / BK;
    const size_t P = a.P_cap;
    const int act = min(C::SL, (valid + 31) / 32);

    const size_t wrow0 = (size_t)e * a.H + (size_t)nb * BN;         // first W2 row
    if constexpr (!C::MX) {
        // the tile's NSB weight scale rows of W2_sf [E, H/128, I/128], contiguous
        const float* wsf = a.w2_sf + ((size_t)e * a.nb2 + nb) * C::NSB * KB;
        for (int i = threadIdx.x; i < C::NSB * KB; i += NT) lds.w_sf()[i] = wsf[i];
    }
    // each row's route (-1 past the valid rows), for the epilogue's stores: read
    // now, alongside the scales, instead of one dependent load per store round
    for (int r = threadIdx.x; r < BM; r += NT) lds.tile()[4 + r] = r < valid ? a.src[row0 + r] : -1;
    // wait until every L1 tile of this pool block has published.  A tile of
    // this XCD's own range reads the block from this XCD's L2, where its L1
    // tiles left it.  A tile taken from another XCD's queue waits for the
    // block's write-back (READY_PUBLISHED, polled with atomics, which every XCD
    // sees alike), then invalidates this XCD's L2 (an agent-scope acquire) so
    // that no stale line of an earlier call is read.
    if (threadIdx.x == 0) {
        uint32_t spins = 0;
        for (;;) {
            const uint32_t r =
                foreign ? __hip_atomic_fetch_add(&a.ready[pb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                        : __hip_atomic_load(&a.ready[pb], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (foreign ? (r & READY_PUBLISHED) != 0u : (r & ~READY_PUBLISHED) >= (uint32_t)a.nb1) break;
            if (++spins > a.wait_spin_limit) {
                atomicOr(&a.ctrl->error, MEGA_MOE_DEVERR_WAIT_TIMEOUT);
                break;
            }
            __builtin_amdgcn_s_sleep(4);
        }
        if (foreign) {
            // the invalidation must be complete before the other waves,
            // released by the barrier below, issue their loads
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
    }
    __syncthreads();

    const int row_b = C::MX ? I / 2 : I;
    const Loader<MS, BNT, 2, WF> ld(
        make_rsrc(a.l2_acts + (size_t)row0 * I, (uint32_t)valid * I),
        make_rsrc(a.w2 + wrow0 * row_b, (uint32_t)(BN * row_b)), I, row_b,
        make_rsrc(a.l2_sf + row0, (uint32_t)(((2 * KB - 1) * P + valid) * 4)), (int)P,
        make_rsrc(C::MX ? a.w2_e8 + wrow0 * (I / 32) : nullptr, C::MX ? (uint32_t)(BN * (I / 32)) : 0u),
        I / 32, valid);

    const v16f zero = v16f{};
    constexpr int YS = C::YS;
    uint16_t* stage = reinterpret_cast<uint16_t*>(lds.stage(0));  // BF16 [BM][YS] after the k loop

    dispatch_act<C::SL>(act, [&](auto tag) {
        constexpr int ACT = decltype(tag)::value;
        using LY = Lay<MS, BNT, ACT>;
        const LY ly;
        v16f acc[LY::NJ][LY::NG];
#pragma unroll
        for (int j = 0; j < LY::NJ; ++j)
#pragma unroll
            for (int q = 0; q < LY::NG; ++q) acc[j][q] = v16f{};
        v16f accx = v16f{};   // slice 4 of a 160-row tile, column group g(0)
        // FP8 weights: the previous step's last product and its scale (zero
        // before the first step), and where it folds: slice 4 when the tile
        // has one, else the last slice and group, both in the second 64-K half
        v16f dl = v16f{};
        float sl = 0.0f;
        auto fold_last = [&]() {
            if constexpr (LY::XJ > 0)
                accx = __builtin_elementwise_fma(dl, v16f(sl), accx);
            else
                acc[LY::NJ - 1][LY::NG - 1] = __builtin_elementwise_fma(dl, v16f(sl), acc[LY::NJ - 1][LY::NG - 1]);
        };

        k_loop(ld, lds, KB, [&](const uint8_t* stg, int kb) {
            const uint8_t* sfa = stg + C::OFF_SF;
            if constexpr (C::MX) {
                // MXFP4 weights: the scaled MFMA applies each lane's 32-K block
                // scale (lane half g of 64-K half hh holds block 2hh + g)
                const int g = (threadIdx.x >> 5) & 1;
                uint32_t wsc[LY::NG];
                v4i fb[LY::NG][2];
#pragma unroll
                for (int q = 0; q < LY::NG; ++q) {
                    if constexpr (C::WSC_BLOCK)
                        wsc[q] = lane_wsc<16>(lds.wsb((kb >> 2) & 1) + 4 * (kb & 3), ly.g(q));
                    else
                        wsc[q] = lane_wsc(stg + C::OFF_WSC, ly.g(q));
                    fb[q][0] = fp4_half_raw(stg + C::OFF_B, ly.g(q), 0);
                    fb[q][1] = fp4_half_raw(stg + C::OFF_B, ly.g(q), 1);
                }
                Frag fa[LY::NJ];
                float sa[LY::NJ][2];
#pragma unroll
                for (int j = 0; j < LY::NJ; ++j) {
                    fa[j] = read_frag2(stg, ly.s0 + j);
                    sa[j][0] = lane_row_scale(sfa, ly.s0 + j);
                    sa[j][1] = lane_row_scale(sfa + 4 * BM, ly.s0 + j);
                }
                // product i: half i / (NJ NG), slice (i / NG) % NJ, group i % NG
                constexpr int NB = 2 * LY::NJ * LY::NG;
                prod_fold_pipeline<NB>(
                    [&](int i) {
                        const int hh = i / (LY::NJ * LY::NG), j = (i / LY::NG) % LY::NJ, q = i % LY::NG;
                        const int e8 = (int)((wsc[q] >> (8 * (2 * hh + g))) & 0xFFu);
                        return mfma_mx(fb[q][hh], fa[j].h[hh], zero, e8);
                    },
                    [&](int i, const v16f& d) {
                        const int hh = i / (LY::NJ * LY::NG), j = (i / LY::NG) % LY::NJ, q = i % LY::NG;
                        acc[j][q] = __builtin_elementwise_fma(d, v16f(sa[j][hh]), acc[j][q]);
                    });
                return;
            }
            const float sw = lds.w_sf()[ly.sblock() * KB + kb];
            Frag fb[LY::NG];
#pragma unroll
            for (int q = 0; q < LY::NG; ++q) fb[q] = read_frag2(stg + C::OFF_B, ly.g(q));
            Frag fa[LY::NJ + LY::XJ];
            float svw[LY::NJ + LY::XJ][2];
#pragma unroll
            for (int j = 0; j < LY::NJ + LY::XJ; ++j) {
                const int sl = j < LY::NJ ? ly.s0 + j : 4;
                fa[j] = read_frag2(stg, sl);
                svw[j][0] = lane_row_scale(sfa, sl) * sw;
                svw[j][1] = lane_row_scale(sfa + 4 * BM, sl) * sw;
            }
            // product i < NB0: half i / (NJ NG), slice (i / NG) % NJ, group
            // i % NG; then slice 4 with group g(0), half i - NB0
            constexpr int NB0 = 2 * LY::NJ * LY::NG;
            constexpr int NB = NB0 + 2 * LY::XJ;
            dl = prod_fold_carry<NB>(
                [&](int i) {
                    if constexpr (LY::XJ > 0) {
                        if (i >= NB0) return mfma_f8(fb[0].h[i - NB0], fa[LY::NJ].h[i - NB0], zero);
                    }
                    const int hh = i / (LY::NJ * LY::NG), j = (i / LY::NG) % LY::NJ, q = i % LY::NG;
                    return mfma_f8(fb[q].h[hh], fa[j].h[hh], zero);
                },
                [&](int i, const v16f& d) {
                    if constexpr (LY::XJ > 0) {
                        if (i >= NB0) {
                            accx = __builtin_elementwise_fma(d, v16f(svw[LY::NJ][i - NB0]), accx);
                            return;
                        }
                    }
                    const int hh = i / (LY::NJ * LY::NG), j = (i / LY::NG) % LY::NJ, q = i % LY::NG;
                    acc[j][q] = __builtin_elementwise_fma(d, v16f(svw[j][hh]), acc[j][q]);
                },
                fold_last);
            sl = LY::XJ > 0 ? svw[LY::NJ + LY::XJ - 1][1] : svw[LY::NJ - 1][1];
        });
        if constexpr (!C::MX) fold_last();   // the last step's last product

        // ---- epilogue: BF16 partials, staged so each route row is stored whole ----
        // (transposed blocks: register v of lane l is column 8(v/4) + 4(l/32)
        // + v%4 of the group for row l%32; four registers = 8 bytes of a row)
        auto put = [&](const v16f& r, int s, int g) {
            const int row = 32 * s + (threadIdx.x & 31);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint2 w2{pack_bf16x2(r[4 * t], r[4 * t + 1]), pack_bf16x2(r[4 * t + 2], r[4 * t + 3])};
                const int col = 32 * g + 8 * t + 4 * ((threadIdx.x >> 5) & 1);
                *reinterpret_cast<uint2*>(stage + row * YS + col) = w2;
            }
        };
#pragma unroll
        for (int j = 0; j < LY::NJ; ++j)
#pragma unroll
            for (int q = 0; q < LY::NG; ++q) put(acc[j][q], ly.s0 + j, ly.g(q));
        if constexpr (LY::XJ > 0) put(accx, 4, ly.g(0));
    });
    __syncthreads();
    for (int q = threadIdx.x; q < 32 * act * (BN / 8); q += NT) {
        const int r = q / (BN / 8), part = q % (BN / 8);
        const int f = lds.tile()[4 + r];
        if (f >= 0) {
            const uint4 v = *reinterpret_cast<const uint4*>(stage + r * YS + part * 8);
            *reinterpret_cast<uint4*>(a.comb + (size_t)f * a.H + nb * BN + part * 8) = v;
        }
    }
}

// Two workgroups of four waves per CU, one wave of each per SIMD; the launch
// puts num_cus * 2 of them in flight and they take tiles until their XCD's
// queue is empty.
template <int MS, int BNT, int WF>
__global__ void __launch_bounds__((Cfg<MS, BNT, WF>::NT)) __attribute__((amdgpu_waves_per_eu(2)))
moe_expert_ffn(MoeArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[Cfg<MS, BNT, WF>::LDS_BYTES];
    const Lds<MS, BNT, WF> lds{smem};
    // XCC_ID hardware register, bits [3:0]
    const int xcd = (__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 0xf) % a.n_xcd;
    const int G = a.xcd_group;
    // Each XCD keeps two queues over its range of pool blocks: its L1 tiles
    // and its L2 tiles.  A workgroup drains its own XCD's L1 queue, then its
    // L2 queue (phase 1 only the former, phase 2 only the latter); in the
    // fused kernel (phase 0) it then takes the L2 tiles still queued on the
    // other XCDs, so that XCDs that finish early share the work of the slower
    // ones.  Thread 0 keeps the queue state: 0 own L1, 1 own L2, 2 .. n_xcd
    // the XCD (xcd + q - 1) % n_xcd, past that done.  With the phases on
    // disjoint XCD sets (phase 3 + n) an L1 XCD's workgroups take its own L1
    // queue only, and an L2 XCD's the L2 queues of the n L1 XCDs in turn
    // (state q >= 1: the XCD (xcd + q - 1) % n).
    const int nx1 = a.phase - PHASE_XCD_SPLIT;
    const bool l2_side = a.phase == 2 || (a.phase >= PHASE_XCD_SPLIT && xcd >= nx1);
    int q = l2_side ? 1 : 0;
    const int q_end = a.phase >= PHASE_XCD_SPLIT ? (l2_side ? 1 + nx1 : 1)
                                                 : (a.phase == 0 && a.steal ? 1 + a.n_xcd : 2);
    // this XCD's range of pool blocks (fixed for the call)
    const int own_first = __builtin_amdgcn_readfirstlane(a.xcd_info[2 * xcd]);
    const int own_cnt = __builtin_amdgcn_readfirstlane(a.xcd_info[2 * xcd + 1]);
    for (;;) {
        if (threadIdx.x == 0) {
            int u = -1, v = xcd, l1 = 0;
            while (q < q_end) {
                if (q == 0) {
                    const int t = atomicAdd(&a.ctrl->next_tile[xcd], 1);
                    if (t < own_cnt * a.nb1) { u = t; l1 = 1; break; }
                    q = a.phase == 0 ? 1 : q_end;
                } else {
                    v = (xcd + q - 1) % (a.phase >= PHASE_XCD_SPLIT ? nx1 : a.n_xcd);
                    const int t = atomicAdd(&a.ctrl->next_tile_l2[v], 1);
                    if (t < a.xcd_info[2 * v + 1] * a.nb2) { u = t; break; }
                    ++q;
                }
            }
            lds.tile()[0] = u;
            lds.tile()[1] = v;
            lds.tile()[3] = l1;
        }
        // one barrier per tile here: every wave has finished the previous tile
        // (whose LDS the next one overwrites), and the dequeued tile is
        // visible.  Thread 0 writes it again only after the tile's own first
        // barrier (or the one below for a tile with no rows), which every wave
        // reaches after reading it.
        __syncthreads();
        const int u = __builtin_amdgcn_readfirstlane(lds.tile()[0]);
        const int v = __builtin_amdgcn_readfirstlane(lds.tile()[1]);
        const bool is_l1 = __builtin_amdgcn_readfirstlane(lds.tile()[3]) != 0;
        if (u < 0) break;
        // the tile from its pool block's record (expert, first pool row, rows,
        // N-major group), written by the dispatch
        const int first = v == xcd ? own_first : __builtin_amdgcn_readfirstlane(a.xcd_info[2 * v]);
        const int nbs = is_l1 ? a.nb1 : a.nb2;
        const int pq = first + u / nbs;
        int g0 = pq, gs = 1;
        if (a.n_major && G > 1) {
            const int grp = __builtin_amdgcn_readfirstlane(a.pb_rec[4 * pq + 3]);
            g0 = grp >> 8;
            gs = grp & 255;
        }
        int pb, nb;
        tile_in_group(u, first, nbs, g0, gs, pb, nb);
        const int e = __builtin_amdgcn_readfirstlane(a.pb_rec[4 * pb]);
        const int row0 = __builtin_amdgcn_readfirstlane(a.pb_rec[4 * pb + 1]);
        const int valid = __builtin_amdgcn_readfirstlane(a.pb_rec[4 * pb + 2]);
        if (valid > 0) {
            if (is_l1) l1_tile(a, lds, e, pb, row0, valid, nb);
            else l2_tile(a, lds, e, pb, row0, valid, nb, v != xcd);
        } else {
            __syncthreads();   // (a block taken by the tile before it)
        }
    }
}

template <int MS, int BNT, int WF = W_FP8>
static int launch_one(const MoeArgs& a, int num_cus, hipStream_t stream) {
    constexpr int NT = Cfg<MS, BNT, WF>::NT;
    static int per_cu = 0;   // occupancy of this instance (same on every call)
    if (per_cu == 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, moe_expert_ffn<MS, BNT, WF>, NT, 0) !=
                hipSuccess || n < 1)
            n = 1;
        per_cu = n;
    }
    hipLaunchKernelGGL((moe_expert_ffn<MS, BNT, WF>), dim3(num_cus * per_cu), dim3(NT), 0, stream, a);
    return num_cus * per_cu;
}

// Every workgroup sets bit XCC_ID of *word: the XCD ids the device's
// workgroups run on (checked once when a handle is created).
__global__ void __launch_bounds__(64) moe_xcd_probe(uint32_t* word) {
    if (threadIdx.x == 0)
        atomicOr(word, 1u << (__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 0xf));
}

// Runs the probe over 4 workgroups per compute unit (workgroups are dealt to
// the XCDs in turn, so every XCD gets some) and returns the mask in *seen.
hipError_t probe_xcds(uint32_t* word, int num_cus, uint32_t* seen) {
    hipError_t e = hipMemset(word, 0, sizeof(uint32_t));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(moe_xcd_probe, dim3(4 * num_cus), dim3(64), 0, nullptr, word);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return hipMemcpy(seen, word, sizeof(uint32_t), hipMemcpyDeviceToHost);
}

int launch_expert_ffn(const MoeArgs& a, int num_cus, hipStream_t stream) {
    if (a.w_fmt == W_MXFP4) {
        switch (a.block_m) {
            case 32: return launch_one<1, 128, W_MXFP4>(a, num_cus, stream);
            case 64: return launch_one<2, 128, W_MXFP4>(a, num_cus, stream);
            default: return launch_one<4, 128, W_MXFP4>(a, num_cus, stream);
        }
    }
    if (a.block_n == 256) {
        if (a.block_m == 64) return launch_one<2, 256>(a, num_cus, stream);
        return launch_one<4, 256>(a, num_cus, stream);
    }
    switch (a.block_m) {
        case 32: return launch_one<1, 128>(a, num_cus, stream);
        case 64: return launch_one<2, 128>(a, num_cus, stream);
        default: return launch_one<4, 128>(a, num_cus, stream);
    }
}

}  // namespace mega_moe
