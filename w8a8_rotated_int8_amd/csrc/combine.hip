// Probability-weighted combine of the expert outputs back into the tokens ("MLX Nucleus-Image",
// "Conversion notes": each expert picks its top-C tokens and the results are scattered back).
//
// out[t, :] = bf16( sum over experts e in ascending order that took t of w[e, c] * z[e*C + c, :] ), fp32,
// starting from +0.0f, one rounding at the end; tokens taken by no expert get +0.  Deterministic: every output
// element is summed by one lane, no atomics, so the sum order is fixed.
//
// A token's row is split over wavefronts of 64 chunks of 16 bytes (more, shorter wavefronts measured faster
// than one per token).  In each, lane e reads the slot-table entry of expert e (the token's entries for 64
// experts are contiguous: one coalesced load), a ballot gives the taking experts, and their rows are summed
// from the lowest expert up.  Two dependent loads per expert row (slot, then row and weight).
// The row loads of up to kBatch experts are all issued before any of them is summed, so a token costs one
// memory latency per kBatch experts rather than one per expert.  Lane l owns the chunks l, l + 64, ... of its wavefront's
// part of the row.
#include "device_common.h"
#include "kernels.h"

namespace crk {
namespace {

constexpr int kBatch = 4;
constexpr int kMaxChunks = 1;  // 16-byte chunks per lane: a d = 2048 row is split over 4 wavefronts

template <int CH>  // 16-byte chunks (8 bf16) per lane
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ z, const int32_t* __restrict__ slots,
                                                      const float* __restrict__ wt, int T, int E, int C, int d,
                                                      int split, uint16_t* __restrict__ out) {
    const int wv = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int t = wv / split;  // `split` wavefronts per token, each over 64 CH consecutive chunks
    if (t >= T) return;        // wave-uniform
    const int part = wv - t * split;
    const int lane = threadIdx.x & 63;
    const int nch = d >> 3;
    const int ch0 = part * 64 * CH;
    float acc[CH][8];
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[j][q] = 0.0f;

    for (int e0 = 0; e0 < E; e0 += 64) {
        const int e = e0 + lane;
        const int c = e < E ? slots[(int64_t)t * E + e] : -1;
        const float w = (c >= 0) ? wt[(int64_t)e * C + c] : 0.0f;
        uint64_t taken = __ballot(c >= 0);
        while (taken) {
            // the next (up to) kBatch experts, lowest first
            int cnt = 0;
            uint4 raw[kBatch][CH];
            float wb[kBatch];
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                if (taken) {
                    const int l = __ffsll((unsigned long long)taken) - 1;
                    taken &= taken - 1;
                    const int cs = __builtin_amdgcn_readlane(c, l);
                    wb[b] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), l));
                    const uint16_t* zr = z + ((int64_t)(e0 + l) * C + cs) * d;
#pragma unroll
                    for (int j = 0; j < CH; ++j) {
                        const int ch = ch0 + lane + 64 * j;
                        raw[b][j] = ch < nch ? *reinterpret_cast<const uint4*>(zr + 8 * ch) : make_uint4(0u, 0u, 0u, 0u);
                    }
                    cnt = b + 1;
                }
            }
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                if (b < cnt) {
#pragma unroll
                    for (int j = 0; j < CH; ++j) {
                        const uint32_t wv[4] = {raw[b][j].x, raw[b][j].y, raw[b][j].z, raw[b][j].w};
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float z0 = bf16_to_float(wv[q] & 0xffffu);
                            const float z1 = __uint_as_float(wv[q] & 0xffff0000u);
                            const float p0 = wb[b] * z0;
                            const float p1 = wb[b] * z1;
                            acc[j][2 * q] = acc[j][2 * q] + p0;
                            acc[j][2 * q + 1] = acc[j][2 * q + 1] + p1;
                        }
                    }
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int ch = ch0 + lane + 64 * j;
        if (ch < nch) {
            uint4 o;
            o.x = pack_bf16x2(acc[j][0], acc[j][1]);
            o.y = pack_bf16x2(acc[j][2], acc[j][3]);
            o.z = pack_bf16x2(acc[j][4], acc[j][5]);
            o.w = pack_bf16x2(acc[j][6], acc[j][7]);
            *reinterpret_cast<uint4*>(out + (int64_t)t * d + 8 * ch) = o;
        }
    }
}

}  // namespace

hipError_t launch_combine(const uint16_t* z, const int32_t* slots, const float* wt, int T, int E, int C, int d,
                          uint16_t* out, hipStream_t st) {
    if (T == 0) return hipSuccess;
    // chunks per lane with one wavefront per token, then split over wavefronts to at most kMaxChunks each
    const int ch_one = (d / 8 + 63) / 64;
    const int split = (ch_one + kMaxChunks - 1) / kMaxChunks;
    const int ch = (ch_one + split - 1) / split;
    const dim3 grid((unsigned)(((int64_t)T * split + 3) / 4)), block(256);
    if (ch <= 1) combine_kernel<1><<<grid, block, 0, st>>>(z, slots, wt, T, E, C, d, split, out);
    else if (ch <= 2) combine_kernel<2><<<grid, block, 0, st>>>(z, slots, wt, T, E, C, d, split, out);
    else if (ch <= 4) combine_kernel<4><<<grid, block, 0, st>>>(z, slots, wt, T, E, C, d, split, out);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace crk
