// Gate/up interleave of W1 ("MegaMoE SM90 Implementation Design (Final)"
// 15.1) from the plain layout (all I gate rows, then all I up rows, one
// float32 scale per 128x128 block of that tensor) into the stored layout the
// layer takes (stored row 16g + r is gate row 8g + r for r < 8, up row
// 8g + r - 8 otherwise; one scale per 128x128 block of the stored tensor,
// 15.2).  Stored block n holds 64 gate rows of source block n/2 and 64 up
// rows of source block I/128 + n/2, so it takes the larger of the two
// scales, and the codes of rows whose source scale is smaller are re-rounded
// at the ratio of the two (in float64, round to nearest even).
//
// Memory bound: one read and one write of W1 (0.94 GB at 32 x 4096 x 7168),
// 8 bytes per thread per iteration.  It runs once when weights are loaded,
// not per forward call.
#include <hip/hip_runtime.h>
#include <math.h>

#include "moe_args.h"

namespace mega_moe {

// Value of an OCP E4M3 ("fn") code: sign, 4 exponent bits with bias 7, 3
// mantissa bits; exponent 0 is subnormal; S.1111.111 is NaN.
__device__ __forceinline__ double e4m3_value(uint32_t c) {
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    double mag;
    if (e == 15u && m == 7u) return __longlong_as_double(0x7ff8000000000000ll);
    if (e == 0u) mag = ldexp((double)m, -9);
    else mag = ldexp((double)(8u + m), (int)e - 10);
    return (c & 0x80u) ? -mag : mag;
}

// Nearest E4M3 code of a float64 value, ties to even, finite magnitudes
// above 448 saturate to 448, NaN -> 0x7F, the sign of zero kept.  All the
// steps are exact in float64: scaling by powers of two and rint.
__device__ __forceinline__ uint32_t e4m3_rne(double v) {
    if (isnan(v)) return 0x7Fu;
    const bool neg = signbit(v);
    const double a = fmin(fabs(v), 448.0);
    int ex;
    frexp(a, &ex);                              // a = f * 2^ex, f in [0.5, 1)
    const int e = max(ex - 1, -6);              // binade of a (subnormals: -6)
    const double q = ldexp(1.0, e - 3);         // spacing of codes in it
    const double r = rint(a / q) * q;           // nearest representable value
    uint32_t code;
    if (r < ldexp(1.0, -6)) {
        code = (uint32_t)rint(r * 512.0);       // subnormal: m x 2^-9
    } else {
        int rex;
        frexp(r, &rex);
        const int re = rex - 1;
        code = ((uint32_t)(re + 7) << 3) | (uint32_t)rint((ldexp(r, -re) - 1.0) * 8.0);
    }
    return neg ? (code | 0x80u) : code;
}

__global__ void __launch_bounds__(256)
moe_transform_w1(const uint8_t* __restrict__ w1, const float* __restrict__ sf,
                 uint8_t* __restrict__ out, float* __restrict__ out_sf, int E, int N, int H) {
    const int I = N / 2, KB = H / 128, NB = N / 128, cpr = H / 8;
    const size_t chunks = (size_t)E * N * cpr;
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < chunks;
         idx += (size_t)gridDim.x * blockDim.x) {
        const size_t row = idx / cpr;            // e * N + stored row
        const int col = (int)(idx - row * cpr) * 8;
        const int e = (int)(row / N), r = (int)(row - (size_t)e * N);
        const int g = r >> 4, o = r & 15;
        const bool up = o >= 8;
        const int src = up ? I + 8 * g + o - 8 : 8 * g + o;
        const int n = r / 128, kb = col / 128;
        const float s_gate = sf[((size_t)e * NB + (64 * n) / 128) * KB + kb];
        const float s_up = sf[((size_t)e * NB + (I + 64 * n) / 128) * KB + kb];
        const float s_new = fmaxf(s_gate, s_up);
        if ((r & 127) == 0 && (col & 127) == 0) out_sf[((size_t)e * NB + n) * KB + kb] = s_new;
        const double ratio = s_new > 0.0f ? (double)(up ? s_up : s_gate) / (double)s_new : 0.0;
        const uint2 d = *reinterpret_cast<const uint2*>(w1 + ((size_t)e * N + src) * H + col);
        uint32_t w[2] = {d.x, d.y}, o2[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint32_t packed = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint32_t c = (w[h] >> (8 * b)) & 0xFFu;
                const uint32_t c2 = s_new > 0.0f ? e4m3_rne(e4m3_value(c) * ratio) : 0u;
                packed |= c2 << (8 * b);
            }
            o2[h] = packed;
        }
        *reinterpret_cast<uint2*>(out + row * H + col) = uint2{o2[0], o2[1]};
    }
}

void launch_transform_w1(const uint8_t* w1, const float* sf, uint8_t* out, float* out_sf, int E,
                         int N, int H, hipStream_t stream) {
    const size_t chunks = (size_t)E * N * (H / 8);
    size_t blocks = (chunks + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    hipLaunchKernelGGL(moe_transform_w1, dim3((unsigned)blocks), dim3(256), 0, stream, w1, sf,
                       out, out_sf, E, N, H);
}

}  // namespace mega_moe
