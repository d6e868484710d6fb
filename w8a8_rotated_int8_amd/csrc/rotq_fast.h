// Rotate + quantise of activation rows, fast path (K a multiple of 8 g): the per-row device routine, shared
// by the stand-alone kernel and the launch that runs it beside the router softmax.
#pragma once

#include "device_common.h"

namespace crk {
namespace {

// ---- activation rows, fast path: K a multiple of 8 g ------------------------------------------------------
// Lane l holds, in each of R = K / (8 g) rounds, the contiguous run of E = g / 8 elements
// [round * 8g + l * E, + E): every g-block sits on 8 consecutive lanes, so the transform runs its stages
// h < E inside the lane and only h = E, 2E, 4E across lanes (partner lane l ^ 1, ^ 2 via DPP quad
// permutations, ^ 4 via a swizzle).  Every stage still forms the pairs (a + b, a - b) of the ascending-h
// transform, so the fp32 values are those of the plain loop.
//
// The transform's sums v are 2^k times the rotated values r = v 2^-k (k = log2(g) / 2, an exact power of
// two).  With sc = amax|v| / qmax, the row's scale is sc 2^-k and its codes rint(v / sc): while sc >= 2^-96
// every scaled quantity stays normal, so r / scale and v / sc are the same quotient bit for bit (a v whose
// r would be subnormal quantises to 0 either way), and the per-element scaling is skipped.  Smaller rows
// scale each value as defined and take the IEEE division.
//
// Quantiser division: with y = 1 / sc rounded to nearest (one IEEE division per row), the quotient q0 = v y,
// its exact remainder e = fma(-q0, sc, v) and q = fma(e, y, q0) give the correctly rounded v / sc
// (Markstein's theorem; it needs the remainder to be exact, which holds while sc >= 2^-96 -- checked
// exhaustively on random and half-integer quotients over the whole fp32 range).

__device__ __forceinline__ float dpp_xor1(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));  // quad_perm 1,0,3,2
}
__device__ __forceinline__ float dpp_xor2(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));  // quad_perm 2,3,0,1
}
__device__ __forceinline__ float swz_xor4(float v) {
    // ds_swizzle bit-mask mode: and 0x1f, or 0, xor 4 (within 32 lanes)
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x101F));
}

// Code byte of a quotient t with |t| <= 127.5: clamp to [-127, 127], then adding 1.5 * 2^23 rounds to the
// nearest integer (ties to even, as rint) and leaves it in the low mantissa bits, whose low byte is the code
// in two's complement.
__device__ __forceinline__ uint32_t code_bits(float t) {
    return __float_as_uint(__builtin_amdgcn_fmed3f(t, -127.0f, 127.0f) + 12582912.0f);
}
// The same for |t| < 127.5, with no clamp.  The fast path's quotients are in range: |v| <= amax and
// sc = amax / 127 rounded to nearest, so |v / sc| <= 127 / (1 - 2^-24) < 127.00001.
__device__ __forceinline__ uint32_t code_bits_in_range(float t) { return __float_as_uint(t + 12582912.0f); }
// Low bytes of four such words, packed in order.
__device__ __forceinline__ uint32_t pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);  // bytes: a0, b0, 0, 0
    const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x04000c0cu);  // bytes: 0, 0, c0, d0
    return ab | cd;
}

// The bf16 bits of this lane's part of a row: R rounds of E = g / 8 elements, 16 bytes per uint4.
template <int G, int R>
struct RotqRaw {
    uint4 d[R][G / 64];
};

template <int G, int R>
__device__ __forceinline__ void rotq_fast_load(const uint16_t* __restrict__ x, int64_t row, bool valid, int K, int part,
                                               RotqRaw<G, R>& raw) {
    constexpr int E = G / 8;
    const int lane = threadIdx.x & 63;
    const uint16_t* src = x + row * (int64_t)K + (int64_t)part * R * 8 * G + lane * E;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < E / 8; ++c)
            raw.d[r][c] = valid ? *reinterpret_cast<const uint4*>(src + r * 8 * G + 8 * c) : make_uint4(0u, 0u, 0u, 0u);
}

// Rotate + quantise of a row part already loaded by rotq_fast_load.
template <int G, int R, int WPR>
__device__ __forceinline__ void rotq_fast_finish(const RotqRaw<G, R>& raw_in, int64_t row, bool valid, int K, int part,
                                                 int8_t* __restrict__ q, float* __restrict__ s, float* xch) {
    constexpr int E = G / 8;  // elements per lane per round
    const int lane = threadIdx.x & 63;
    const int64_t off0 = row * (int64_t)K + (int64_t)part * R * 8 * G + lane * E;
    float v[R][E];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < E / 8; ++c) {
            const uint4 raw = raw_in.d[r][c];
            const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[r][8 * c + 2 * e] = bf16_to_float(w[e] & 0xffffu);
                v[r][8 * c + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
            }
        }
    constexpr float kNorm = (G == 256) ? 0.0625f : 0.125f;  // 2^-(log2 g)/2, exact
    // Across lanes the pair (a + b, a - b) is other + sgn * mine: the lower lane of a pair adds, the upper
    // lane subtracts its own value from its partner's (multiplying by +-1 is exact, the fma rounds once).
    const float sg1 = (lane & 1) ? -1.0f : 1.0f, sg2 = (lane & 2) ? -1.0f : 1.0f, sg4 = (lane & 4) ? -1.0f : 1.0f;
    float amax = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int h = 1; h < E; h *= 2)
#pragma unroll
            for (int e = 0; e < E; ++e)
                if ((e & h) == 0) {
                    const float a = v[r][e], b = v[r][e + h];
                    v[r][e] = a + b;
                    v[r][e + h] = a - b;
                }
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float mine = v[r][e];
            mine = __builtin_fmaf(sg1, mine, dpp_xor1(mine));
            mine = __builtin_fmaf(sg2, mine, dpp_xor2(mine));
            mine = __builtin_fmaf(sg4, mine, swz_xor4(mine));
            v[r][e] = mine;  // 2^k times the rotated value
            amax = fmaxf(amax, fabsf(mine));
        }
    }
    amax = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_max(amax))));  // wave-uniform
    if constexpr (WPR > 1) {
        const int w = threadIdx.x >> 6, w0 = w - part;
        if (lane == 0) xch[w] = amax;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < WPR; ++i) amax = fmaxf(amax, xch[w0 + i]);
    }
    if (!valid) return;  // wave-uniform, after the barrier
    const float sc = amax / 127.0f;
    int8_t* dst = q + off0;
    auto store_round = [&](int r, const uint32_t (&packed)[E / 4]) {
        if constexpr (E == 8) {
            *reinterpret_cast<uint2*>(dst + r * 8 * G) = make_uint2(packed[0], packed[1]);
        } else {
#pragma unroll
            for (int c = 0; c < E / 16; ++c)
                *reinterpret_cast<uint4*>(dst + r * 8 * G + 16 * c) =
                    make_uint4(packed[4 * c], packed[4 * c + 1], packed[4 * c + 2], packed[4 * c + 3]);
        }
    };
    float scale;
    if (sc >= 0x1p-96f) {
        scale = sc * kNorm;  // exact
        const float y = 1.0f / sc;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            uint32_t packed[E / 4];
#pragma unroll
            for (int e = 0; e < E; e += 4) {
                uint32_t b[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float q0 = v[r][e + u] * y;
                    const float rem = __builtin_fmaf(-q0, sc, v[r][e + u]);
                    b[u] = code_bits_in_range(__builtin_fmaf(rem, y, q0));
                }
                packed[e / 4] = pack4(b[0], b[1], b[2], b[3]);
            }
            store_round(r, packed);
        }
    } else {
        scale = (amax * kNorm) / 127.0f;  // the largest scaled value is the scaled largest value
#pragma unroll
        for (int r = 0; r < R; ++r) {
            uint32_t packed[E / 4];
#pragma unroll
            for (int e = 0; e < E; e += 4) {
                uint32_t b[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) b[u] = code_bits(scale == 0.0f ? 0.0f : (v[r][e + u] * kNorm) / scale);
                packed[e / 4] = pack4(b[0], b[1], b[2], b[3]);
            }
            store_round(r, packed);
        }
    }
    if (lane == 0 && part == 0) s[row] = scale;
}

// Rounds [part R, part R + R) of one row by this wavefront; WPR wavefronts of the workgroup (consecutive, this
// one among them) share the row and exchange their maxima through xch (WPR floats from the group's first
// wavefront on) behind a workgroup barrier, which every wavefront reaches (valid = false: a row past the end,
// nothing read or written).  WPR = 1: one row per wavefront, no exchange.
template <int G, int R, int WPR>
__device__ __forceinline__ void rotq_fast_part(const uint16_t* __restrict__ x, int64_t row, bool valid, int K, int part,
                                               int8_t* __restrict__ q, float* __restrict__ s, float* xch) {
    RotqRaw<G, R> raw;
    rotq_fast_load<G, R>(x, row, valid, K, part, raw);
    rotq_fast_finish<G, R, WPR>(raw, row, valid, K, part, q, s, xch);
}

// One row per wavefront (row < rows is the caller's check).
template <int G, int R>
__device__ __forceinline__ void rotq_fast_row(const uint16_t* __restrict__ x, int64_t row, int K,
                                              int8_t* __restrict__ q, float* __restrict__ s) {
    rotq_fast_part<G, R, 1>(x, row, true, K, 0, q, s, nullptr);
}

}  // namespace
}  // namespace crk
