// Top-k combine: y[t, n] = bf16( sum over active slots j, ascending, of
// float32(partial[t*k + j, n]) ), a float32 running sum from +0 ("MegaMoE SM90
// Implementation Design (Final)" 11.2; "PR357 Green-Context Split MegaMoE
// code review" 6.3).  A slot is active when 0 <= topk_idx < E.
//
// HBM-bound: each thread owns 8 consecutive columns (16-byte loads and
// stores) of one token and walks its k partial rows in slot order; a row of
// H columns is covered by H/8 threads, so every load instruction of a wave
// reads 1 KB of one contiguous partial row.  The partials are read once, so
// their loads are non-temporal (measured on MI355X: 12% less time on the
// 8192-token batch, no change on the small ones).
#include <hip/hip_runtime.h>

#include "moe_args.h"

namespace mega_moe {

constexpr int COMBINE_THREADS = 128;
constexpr int COMBINE_COLS = COMBINE_THREADS * 8;   // columns per workgroup

// Two floats as packed BF16 (lo in bits 0-15), rounded to nearest even, NaN
// kept as a quiet NaN (one v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__global__ void __launch_bounds__(COMBINE_THREADS)
moe_combine(MoeArgs a) {
    if (a.err_move && blockIdx.x == 0 && threadIdx.x == 0) {
        // every kernel that can raise an error bit of this call ran before
        // this one on the stream
        const uint32_t e = __hip_atomic_exchange(&a.ctrl->error, 0u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
        if (e && a.err_out) atomicOr(a.err_out, e);
    }
    const int col_blocks = (a.H + COMBINE_COLS - 1) / COMBINE_COLS;
    const int t = blockIdx.x / col_blocks;
    const int col = (blockIdx.x - t * col_blocks) * COMBINE_COLS + threadIdx.x * 8;
    if (col >= a.H) return;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    // slots in groups of 8: all expert ids of the group, then all active
    // partial loads in flight together, then the adds in slot order.  An
    // inactive slot contributes +0, which leaves the sum unchanged: it starts
    // at +0, so it is never -0.
    const int* idx = a.topk_idx + (size_t)t * a.k;
    const uint16_t* part = a.comb + (size_t)t * a.k * a.H + col;
    for (int j0 = 0; j0 < a.k; j0 += 8) {
        const int n = min(8, a.k - j0);
        u32x4 p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            p[j] = u32x4{0u, 0u, 0u, 0u};
            if (j < n) {
                const int e = idx[j0 + j];
                if (e >= 0 && e < a.E)
                    p[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(part + (size_t)(j0 + j) * a.H));
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j >= n) break;
            const uint32_t w[4] = {p[j][0], p[j][1], p[j][2], p[j][3]};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] += __uint_as_float(w[i] << 16);
                acc[2 * i + 1] += __uint_as_float(w[i] & 0xffff0000u);
            }
        }
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(a.y + (size_t)t * a.H + col) = o;
}

void launch_combine(const MoeArgs& a, hipStream_t stream) {
    const int col_blocks = (a.H + COMBINE_COLS - 1) / COMBINE_COLS;
    dim3 grid(col_blocks * a.T);
    hipLaunchKernelGGL(moe_combine, grid, dim3(COMBINE_THREADS), 0, stream, a);
}

}  // namespace mega_moe
