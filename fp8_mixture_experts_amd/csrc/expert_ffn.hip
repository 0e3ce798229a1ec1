// The expert path of the layer in one persistent kernel: L1 FP8 grouped GEMM
// (gate/up interleaved) with per-128 float scales, SwiGLU times the top-k
// weight, per-row per-64 amax and FP8 re-quantisation, then the L2 FP8
// grouped GEMM with per-64 activation scales and the BF16 partial of every
// route ("MegaMoE SM90 Implementation Design (Final)" 3.3 phases 2-3, 5.1-5.4,
// 10.1, 11.1, 12).
//
// Work is a queue of tiles of BLOCK_M pool rows x 128 output columns: first
// every L1 tile (pool block pb, 128 interleaved W1 rows = 64 outputs = one
// per-64 scale group), then every L2 tile (pool block pb, 128 columns of H).
// Workgroups take tiles in queue order with one atomic each.  An L2 tile of pb
// waits until all 2I/128 L1 tiles of pb have published their output through
// an arrival counter (the role of the L2 arrival mask of 14.3).  L1 tiles
// never wait and every L2 tile depends only on tiles that precede it in the
// queue, which running workgroups already own, so the wait always ends,
// whatever the number of co-resident workgroups; it is still bounded by a
// spin limit that raises MEGA_MOE_DEVERR_WAIT_TIMEOUT.
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
// Each wave streams its own operand fragments straight from global memory
// into registers (one 128-K step ahead), so the K loop has no LDS traffic and
// no workgroup barrier; LDS is used only by the epilogues.
#include <hip/hip_runtime.h>

#include "moe_args.h"
#include "mega_moe.h"

namespace mega_moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v16f mfma_f8(const v8i& a, const v8i& b, const v16f& c) {
    // scale operands 0 select the plain (unscaled) FP8 x FP8 instruction
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v16f mfma_f16(const v8h& a, const v8h& b, const v16f& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Operand fragment of one 32-row (A) or 32-column (B) slice for one 128-K
// step: half h holds K bytes [64h, 64h+64).  Lane l owns row l%32; its group
// g = l/32 takes bytes 64h + 16g + [0,16) and 64h + 32 + 16g + [0,16) of the
// half.  A and B use the same K placement, so each MFMA sums exactly the 64
// products of its half.
struct Frag {
    v8i h[2];
};

__device__ __forceinline__ void load_frag(Frag& f, const uint8_t* row, bool valid) {
    if (valid) {
        const int g = (threadIdx.x >> 5) & 1;
        const uint4* p = reinterpret_cast<const uint4*>(row) + g;
        const uint4 q0 = p[0], q1 = p[2], q2 = p[4], q3 = p[6];
        f.h[0] = v8i{(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w, (int)q1.x, (int)q1.y, (int)q1.z, (int)q1.w};
        f.h[1] = v8i{(int)q2.x, (int)q2.y, (int)q2.z, (int)q2.w, (int)q3.x, (int)q3.y, (int)q3.z, (int)q3.w};
    } else {
        f.h[0] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
        f.h[1] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    }
}

// The 64 FP8 values a lane holds for one 128-K step, as 8 groups of 8 F16
// (one 16-K F16 MFMA operand each).  Which K goes to which group does not
// matter as long as A and B convert alike: each group of 8 MFMAs still sums
// all 128 products of the step.
struct HFrag {
    v8h q[8];
};

__device__ __forceinline__ void to_f16(HFrag& o, const Frag& f) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int d0 = f.h[q >> 2][(q & 3) * 2];
        const int d1 = f.h[q >> 2][(q & 3) * 2 + 1];
        const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, false);
        const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, true);
        const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, false);
        const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, true);
        o.q[q] = v8h{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    }
}

// Accumulator layout of the 32x32 MFMA: register v of lane l holds row
// 8*(v/4) + 4*(l/32) + v%4 and column l%32.  A lane's 16 rows come in four
// runs of four consecutive rows, so per-row vectors load as four float4.
__device__ __forceinline__ int acc_row(int v) {
    return 8 * (v >> 2) + 4 * ((threadIdx.x >> 5) & 1) + (v & 3);
}

__device__ __forceinline__ void load_row_vec(float (&out)[16], const float* base) {
    const int g4 = 4 * ((threadIdx.x >> 5) & 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 s = *reinterpret_cast<const float4*>(base + 8 * q + g4);
        out[4 * q + 0] = s.x;
        out[4 * q + 1] = s.y;
        out[4 * q + 2] = s.z;
        out[4 * q + 3] = s.w;
    }
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// OCP E4M3 code of v (|v| <= 448 after the clamp), round to nearest even.
__device__ __forceinline__ uint8_t e4m3_code(float v) {
    v = fminf(fmaxf(v, -448.0f), 448.0f);
    return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(v, v, 0, false) & 0xff);
}

constexpr int BN = 128;         // output columns per tile
constexpr int BK = 128;         // K bytes per step

template <int BM, int NWM>
struct TileCfg {
    static constexpr int kWaves = NWM * 2;            // 2 waves across the 128 columns
    static constexpr int kThreads = kWaves * 64;
    static constexpr int kMS = BM / (32 * NWM);       // 32-row slices per wave
    static_assert(kMS >= 1 && kMS * 32 * NWM == BM, "bad tile");
};

template <int BM, int NWM>
struct Smem {
    union {
        struct {
            float amax[2][BM];
            uint8_t codes[BM][64];
        } l1;
        uint16_t l2_stage[BM][BN];
    };
    int tile;
};

// ---------------------------------------------------------------------------
// L1 tile: pool rows [row0, row0 + valid) of expert e, W1 N block nb.
// ---------------------------------------------------------------------------
template <int BM, int NWM>
__device__ void l1_tile(const MoeArgs& a, Smem<BM, NWM>& sm, int e, int pb, int row0,
                        int valid, int nb) {
    using C = TileCfg<BM, NWM>;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / 2, wn = wave % 2;
    const int c = lane & 31;
    const int H = a.H;
    const int KB = H / BK;
    const size_t P = a.P_cap;

    // A rows of this lane, one per 32-row slice
    const uint8_t* arow[C::kMS];
    bool avalid[C::kMS];
    int slice0[C::kMS];
#pragma unroll
    for (int i = 0; i < C::kMS; ++i) {
        slice0[i] = (wm * C::kMS + i) * 32;
        const int r = slice0[i] + c;
        avalid[i] = r < valid;
        arow[i] = a.l1_acts + (size_t)(row0 + r) * H;
    }
    // B rows: slice 0 = gate rows, slice 1 = up rows of outputs 32*wn + c
    const uint8_t* w1e = a.w1 + (size_t)e * (2 * a.I) * H;
    const uint8_t* brow[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int n = nb * BN + wn * 64 + 16 * (c >> 3) + 8 * s + (c & 7);
        brow[s] = w1e + (size_t)n * H;
    }
    const float* sw_base = a.w1_sf + ((size_t)e * a.nb1 + nb) * KB;

    v16f acc[C::kMS][2];
#pragma unroll
    for (int i = 0; i < C::kMS; ++i)
#pragma unroll
        for (int s = 0; s < 2; ++s) acc[i][s] = v16f{};
    const v16f zero = v16f{};

    Frag fa[C::kMS], fb[2];
#pragma unroll
    for (int i = 0; i < C::kMS; ++i) load_frag(fa[i], arow[i], avalid[i]);
#pragma unroll
    for (int s = 0; s < 2; ++s) load_frag(fb[s], brow[s], true);

    for (int kb = 0; kb < KB; ++kb) {
        Frag na[C::kMS], nbf[2];
        const bool more = kb + 1 < KB;
        if (more) {
#pragma unroll
            for (int i = 0; i < C::kMS; ++i) load_frag(na[i], arow[i] + (kb + 1) * BK, avalid[i]);
#pragma unroll
            for (int s = 0; s < 2; ++s) load_frag(nbf[s], brow[s] + (kb + 1) * BK, true);
        }
        const float sw = sw_base[kb];
        HFrag hb[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) to_f16(hb[s], fb[s]);
#pragma unroll
        for (int i = 0; i < C::kMS; ++i) {
            float sa[16];
            load_row_vec(sa, a.l1_sf + (size_t)kb * P + row0 + slice0[i]);
#pragma unroll
            for (int v = 0; v < 16; ++v) sa[v] *= sw;
            HFrag ha;
            to_f16(ha, fa[i]);
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                v16f d = mfma_f16(ha.q[0], hb[s].q[0], zero);
#pragma unroll
                for (int q = 1; q < 8; ++q) d = mfma_f16(ha.q[q], hb[s].q[q], d);
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][s][v] = fmaf(d[v], sa[v], acc[i][s][v]);
            }
        }
        if (more) {
#pragma unroll
            for (int i = 0; i < C::kMS; ++i) fa[i] = na[i];
#pragma unroll
            for (int s = 0; s < 2; ++s) fb[s] = nbf[s];
        }
    }

    // ---- epilogue: SwiGLU x top-k weight, row amax over the 64 outputs ----
    float h[C::kMS][16];
#pragma unroll
    for (int i = 0; i < C::kMS; ++i) {
        float w[16];
        load_row_vec(w, a.l1_w + row0 + slice0[i]);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float g = acc[i][0][v];
            const float u = acc[i][1][v];
            const float silu = g / (1.0f + expf(-g));
            h[i][v] = silu * u * w[v];
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            float m = fabsf(h[i][v]);
#pragma unroll
            for (int d = 1; d < 32; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
            if (c == 0) sm.l1.amax[wn][slice0[i] + acc_row(v)] = m;
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < C::kMS; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = slice0[i] + acc_row(v);
            const float amax = fmaxf(sm.l1.amax[0][r], sm.l1.amax[1][r]);
            const float sf = amax / 448.0f;
            const float q = sf > 0.0f ? h[i][v] / sf : 0.0f;
            sm.l1.codes[r][wn * 32 + c] = e4m3_code(q);
            if (wn == 0 && c == 0 && r < valid) a.l2_sf[(size_t)nb * P + row0 + r] = sf;
        }
    }
    __syncthreads();
    // coalesced store of the BM x 64 FP8 block (16 bytes per thread)
    for (int q = tid; q < BM * 4; q += C::kThreads) {
        const int r = q >> 2, part = q & 3;
        if (r < valid) {
            const uint4 v = *reinterpret_cast<const uint4*>(&sm.l1.codes[r][part * 16]);
            *reinterpret_cast<uint4*>(a.l2_acts + (size_t)(row0 + r) * a.I + nb * 64 + part * 16) = v;
        }
    }
    // publish: every thread's stores reach the device coherence point before
    // the arrival counter of this pool block moves
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (tid == 0) __hip_atomic_fetch_add(&a.ready[pb], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// L2 tile: pool rows [row0, row0 + valid) of expert e, W2 N block nb.
// ---------------------------------------------------------------------------
template <int BM, int NWM>
__device__ void l2_tile(const MoeArgs& a, Smem<BM, NWM>& sm, int e, int pb, int row0,
                        int valid, int nb) {
    using C = TileCfg<BM, NWM>;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / 2, wn = wave % 2;
    const int c = lane & 31;
    const int I = a.I;
    const int KB = I / BK;
    const size_t P = a.P_cap;

    // wait until every L1 tile of this pool block has published
    if (tid == 0) {
        uint32_t spins = 0;
        while (__hip_atomic_load(&a.ready[pb], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
               (uint32_t)a.nb1) {
            if (++spins > a.wait_spin_limit) {
                atomicOr(&a.ctrl->error, MEGA_MOE_DEVERR_WAIT_TIMEOUT);
                break;
            }
            __builtin_amdgcn_s_sleep(4);
        }
    }
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

    const uint8_t* arow[C::kMS];
    bool avalid[C::kMS];
    int slice0[C::kMS];
#pragma unroll
    for (int i = 0; i < C::kMS; ++i) {
        slice0[i] = (wm * C::kMS + i) * 32;
        const int r = slice0[i] + c;
        avalid[i] = r < valid;
        arow[i] = a.l2_acts + (size_t)(row0 + r) * I;
    }
    const uint8_t* w2e = a.w2 + (size_t)e * a.H * I;
    const uint8_t* brow[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) brow[s] = w2e + (size_t)(nb * BN + wn * 64 + s * 32 + c) * I;
    const float* sw_base = a.w2_sf + ((size_t)e * a.nb2 + nb) * KB;

    v16f acc[C::kMS][2];
#pragma unroll
    for (int i = 0; i < C::kMS; ++i)
#pragma unroll
        for (int s = 0; s < 2; ++s) acc[i][s] = v16f{};
    const v16f zero = v16f{};

    Frag fa[C::kMS], fb[2];
#pragma unroll
    for (int i = 0; i < C::kMS; ++i) load_frag(fa[i], arow[i], avalid[i]);
#pragma unroll
    for (int s = 0; s < 2; ++s) load_frag(fb[s], brow[s], true);

    for (int kb = 0; kb < KB; ++kb) {
        Frag na[C::kMS], nbf[2];
        const bool more = kb + 1 < KB;
        if (more) {
#pragma unroll
            for (int i = 0; i < C::kMS; ++i) load_frag(na[i], arow[i] + (kb + 1) * BK, avalid[i]);
#pragma unroll
            for (int s = 0; s < 2; ++s) load_frag(nbf[s], brow[s] + (kb + 1) * BK, true);
        }
        const float sw = sw_base[kb];
#pragma unroll
        for (int i = 0; i < C::kMS; ++i) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                float sa[16];
                load_row_vec(sa, a.l2_sf + (size_t)(2 * kb + hh) * P + row0 + slice0[i]);
#pragma unroll
                for (int v = 0; v < 16; ++v) sa[v] *= sw;
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const v16f d = mfma_f8(fa[i].h[hh], fb[s].h[hh], zero);
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[i][s][v] = fmaf(d[v], sa[v], acc[i][s][v]);
                }
            }
        }
        if (more) {
#pragma unroll
            for (int i = 0; i < C::kMS; ++i) fa[i] = na[i];
#pragma unroll
            for (int s = 0; s < 2; ++s) fb[s] = nbf[s];
        }
    }

    // ---- epilogue: BF16 partials, staged so each route row is stored whole ----
#pragma unroll
    for (int i = 0; i < C::kMS; ++i)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                sm.l2_stage[slice0[i] + acc_row(v)][wn * 64 + s * 32 + c] = bf16_rne(acc[i][s][v]);
    __syncthreads();
    for (int q = tid; q < BM * 16; q += C::kThreads) {
        const int r = q >> 4, part = q & 15;
        if (r < valid) {
            const int f = a.src[row0 + r];
            if (f >= 0) {
                const uint4 v = *reinterpret_cast<const uint4*>(&sm.l2_stage[r][part * 8]);
                *reinterpret_cast<uint4*>(a.comb + (size_t)f * a.H + nb * BN + part * 8) = v;
            }
        }
    }
}

template <int BM, int NWM>
__global__ void __launch_bounds__(NWM * 128)
moe_expert_ffn(MoeArgs a) {
    __shared__ Smem<BM, NWM> sm;
    const int total_mb = a.ctrl->total_mb;
    const int l1_tiles = total_mb * a.nb1;
    const int total = l1_tiles + total_mb * a.nb2;
    for (;;) {
        if (threadIdx.x == 0) sm.tile = atomicAdd(&a.ctrl->next_tile, 1);
        __syncthreads();
        const int u = sm.tile;
        __syncthreads();
        if (u >= total) break;
        int pb, nb;
        const bool is_l1 = u < l1_tiles;
        if (is_l1) {
            pb = u / a.nb1;
            nb = u - pb * a.nb1;
        } else {
            const int u2 = u - l1_tiles;
            if (a.n_major) {
                // tiles of one expert ordered W2 block by W2 block
                int lo = 0, hi = a.E - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (a.mb_start[mid] * a.nb2 <= u2) lo = mid; else hi = mid - 1;
                }
                const int mb0 = a.mb_start[lo];
                const int mbe = a.mb_start[lo + 1] - mb0;
                const int local = u2 - mb0 * a.nb2;
                nb = local / mbe;
                pb = mb0 + (local - nb * mbe);
            } else {
                pb = u2 / a.nb2;
                nb = u2 - pb * a.nb2;
            }
        }
        const int e = a.pb_expert[pb];
        const int m_local = pb - a.mb_start[e];
        const int row0 = a.offsets[e] + m_local * BM;
        const int valid = min(BM, a.counts[e] - m_local * BM);
        if (is_l1) l1_tile<BM, NWM>(a, sm, e, pb, row0, valid, nb);
        else l2_tile<BM, NWM>(a, sm, e, pb, row0, valid, nb);
        __syncthreads();
    }
}

template <int BM, int NWM>
static int launch_one(const MoeArgs& a, int num_cus, hipStream_t stream) {
    using C = TileCfg<BM, NWM>;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, moe_expert_ffn<BM, NWM>,
                                                     C::kThreads, 0) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    hipLaunchKernelGGL((moe_expert_ffn<BM, NWM>), dim3(num_cus * per_cu), dim3(C::kThreads), 0,
                       stream, a);
    return num_cus * per_cu;
}

int launch_expert_ffn(const MoeArgs& a, int num_cus, hipStream_t stream) {
    switch (a.block_m) {
        case 32: return launch_one<32, 1>(a, num_cus, stream);
        case 64: return launch_one<64, 2>(a, num_cus, stream);
        default: return launch_one<128, 2>(a, num_cus, stream);
    }
}

}  // namespace mega_moe
