// Probability-weighted combine of the expert outputs back into the tokens ("MLX Nucleus-Image",
// "Conversion notes": each expert picks its top-C tokens and the results are scattered back).
//
// out[t, :] = bf16( sum over experts e in ascending order that took t of w[e, c] * z[e*C + c, :] ), fp32,
// starting from +0.0f, one rounding at the end; tokens taken by no expert get +0.  Deterministic: one
// workgroup per token, no atomics, so the sum order is fixed.
//
// Each wave reads the slot map entries of up to 64 experts in one vector load (lane = expert), ballots the
// experts that took the token, and walks that mask from the lowest expert up.
#include "device_common.h"
#include "kernels.h"

namespace crk {
namespace {

template <int CH>  // 16-byte chunks (8 bf16) per thread
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ z, const int32_t* __restrict__ slotmap,
                                                      const float* __restrict__ wt, int T, int E, int C, int d,
                                                      uint16_t* __restrict__ out) {
    const int t = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int nch = d >> 3;
    float acc[CH][8];
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[j][q] = 0.0f;

    for (int e0 = 0; e0 < E; e0 += 64) {
        const int e = e0 + lane;
        const int c = (e < E) ? slotmap[(int64_t)e * T + t] : -1;
        const float w = (c >= 0) ? wt[(int64_t)e * C + c] : 0.0f;
        uint64_t taken = __ballot(c >= 0);
        while (taken) {
            const int l = __ffsll((unsigned long long)taken) - 1;
            taken &= taken - 1;
            const int cs = __shfl(c, l);
            const float ws = __shfl(w, l);
            const uint16_t* zr = z + ((int64_t)(e0 + l) * C + cs) * d;
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const int ch = threadIdx.x + 256 * j;
                if (ch < nch) {
                    const uint4 raw = *reinterpret_cast<const uint4*>(zr + 8 * ch);
                    const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float z0 = bf16_to_float(wv[q] & 0xffffu);
                        const float z1 = bf16_to_float(wv[q] >> 16);
                        const float p0 = ws * z0;
                        const float p1 = ws * z1;
                        acc[j][2 * q] = acc[j][2 * q] + p0;
                        acc[j][2 * q + 1] = acc[j][2 * q + 1] + p1;
                    }
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int ch = threadIdx.x + 256 * j;
        if (ch < nch) {
            uint4 o;
            o.x = float_to_bf16(acc[j][0]) | (float_to_bf16(acc[j][1]) << 16);
            o.y = float_to_bf16(acc[j][2]) | (float_to_bf16(acc[j][3]) << 16);
            o.z = float_to_bf16(acc[j][4]) | (float_to_bf16(acc[j][5]) << 16);
            o.w = float_to_bf16(acc[j][6]) | (float_to_bf16(acc[j][7]) << 16);
            *reinterpret_cast<uint4*>(out + (int64_t)t * d + 8 * ch) = o;
        }
    }
}

}  // namespace

hipError_t launch_combine(const uint16_t* z, const int32_t* slotmap, const float* wt, int T, int E, int C, int d,
                          uint16_t* out, hipStream_t st) {
    if (T == 0) return hipSuccess;
    const int ch = (d / 8 + 255) / 256;
    const dim3 grid(T), block(256);
    if (ch <= 1) combine_kernel<1><<<grid, block, 0, st>>>(z, slotmap, wt, T, E, C, d, out);
    else if (ch <= 2) combine_kernel<2><<<grid, block, 0, st>>>(z, slotmap, wt, T, E, C, d, out);
    else if (ch <= 4) combine_kernel<4><<<grid, block, 0, st>>>(z, slotmap, wt, T, E, C, d, out);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace crk
