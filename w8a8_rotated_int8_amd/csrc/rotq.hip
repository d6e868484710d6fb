// Fused block-Hadamard rotation + per-row symmetric quantisation (activations and the offline weight
// converter), and quantisation of already-rotated fp32 rows.
//
// ConvRot as used by the Nucleus-Image INT8 Convrot model card ("Quantization") and NitroFusion2 for
// ComfyUI ("How they were made"): each row is rotated by the block-diagonal normalised Hadamard matrix
// (contiguous blocks of g = 64 or 256 along K), then quantised symmetrically with one fp32 scale per row
// (max|r| / qmax) and nearest rounding, ties to even.
//
// One wavefront per row.  Lane l holds the 8-element vectors i = l + 64 j (elements 8i .. 8i+7), so a
// g-block is g/8 consecutive lanes of one j.  The fast transform runs stages h = 1, 2, 4 inside each
// lane's vector and stages h = 8, 16, ... across lanes (partner lane l ^ (h/8)); every stage forms exactly
// the pairs (a + b, a - b) of the textbook ascending-h transform, so the fp32 results are those of the
// plain loop.  The row maximum is a wave reduction, the codes use IEEE division and rint.
#include "device_common.h"
#include "kernels.h"
#include "rotq_fast.h"

namespace crk {
namespace {

struct Vec8 {
    float v[8];
};

template <int G>
__device__ __forceinline__ void fwht_vec_inlane(Vec8& x) {
#pragma unroll
    for (int h = 1; h < 8 && h < G; h *= 2)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if ((e & h) == 0) {
                float a = x.v[e], b = x.v[e + h];
                x.v[e] = a + b;
                x.v[e + h] = a - b;
            }
}

// Stages h = 8m for m = 1, 2, ..., g/16: the partner of element (lane, e) is (lane ^ m, e); the lane
// holding the lower index keeps a + b, the other keeps a - b.
template <int G>
__device__ __forceinline__ void fwht_vec_crosslane(Vec8& x, int lane) {
#pragma unroll
    for (int m = 1; m < G / 8; m *= 2) {
        const bool upper = (lane & m) != 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float mine = x.v[e];
            float other = __shfl_xor(mine, m);
            x.v[e] = upper ? (other - mine) : (mine + other);
        }
    }
}

// One quantised code: clamp(rint(r / scale), -qmax, qmax), or 0 if scale == 0.
template <int QMAX>
__device__ __forceinline__ int quant_code(float r, float scale) {
    if (scale == 0.0f) return 0;
    float c = rintf(r / scale);
    c = fminf(fmaxf(c, -(float)QMAX), (float)QMAX);
    return (int)c;
}

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
    return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
           ((uint32_t)(d & 0xff) << 24);
}

// Byte offset of the 8 codes k = 8i .. 8i+7 of row n (of one expert) in the MFMA-tiled layout: every
// (32-row block, K-block) tile is 1 KiB.  int8 tiles span 32 k: 16-byte entry r + 32*((k%32)/16) holds 16
// consecutive k of row r.  int4 tiles span 64 k: 8-byte entry 64*(r/16) + 16*((k%64)/16) + r%16 holds 16
// consecutive k of row r, so the 64 lanes of a 16-row fragment read 512 contiguous bytes.
template <bool INT4>
__device__ __forceinline__ int64_t tiled_offset(int n, int k, int K) {
    const int r = n & 31;
    if constexpr (!INT4) {
        return ((int64_t)(n >> 5) * (K >> 5) + (k >> 5)) * 1024 + (r + 32 * ((k & 31) >> 4)) * 16 + (k & 15);
    } else {
        return ((int64_t)(n >> 5) * (K >> 6) + (k >> 6)) * 1024 + (64 * (r >> 4) + 16 * ((k & 63) >> 4) + (r & 15)) * 8 +
               ((k & 15) >> 1);
    }
}

// Output modes of the codes.
enum class Out : int { kRowI8 = 0, kRowI4 = 1, kTiledI8 = 2, kTiledI4 = 3 };

// G: rotation group (0 = no rotation, fp32 input); NV: vectors per lane (K <= 512 NV);
// QMAX: 127 or 7; OUT: code layout; CHECK: flag non-finite rows with a NaN scale.
// Row-major modes process `rows` rows.  Tiled modes process E * NB * 32 rows, where NB = ceil(N / 32) and
// `rows` = E * N: launch row R is row n = R % (NB*32) of expert e = R / (NB*32); rows n >= N only write
// zero codes (the padding of the last row block).
template <int G, int NV, int QMAX, Out OUT, bool CHECK>
__global__ __launch_bounds__(256) void rotq_rows_kernel(const void* __restrict__ xin, int64_t rows, int K, int N,
                                                        void* __restrict__ qout, float* __restrict__ sout,
                                                        float* __restrict__ rot_out) {
    constexpr bool kTiled = (OUT == Out::kTiledI8 || OUT == Out::kTiledI4);
    const int lane = threadIdx.x & 63;
    const int64_t lrow = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    int64_t row = lrow;          // source row (and scale index)
    int64_t expert = 0;
    int n = 0;
    bool pad = false;
    if constexpr (kTiled) {
        const int nbr = ((N + 31) >> 5) << 5;  // rows per expert incl. padding
        expert = lrow / nbr;
        n = (int)(lrow - expert * nbr);
        if (expert * N >= rows) return;  // wave-uniform
        pad = n >= N;
        row = expert * N + n;
    } else {
        if (row >= rows) return;  // wave-uniform
    }
    const int nvec = K >> 3;

    Vec8 x[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int i = lane + 64 * j;
        if (i < nvec && !pad) {
            if constexpr (G > 0) {
                const uint4 raw = *reinterpret_cast<const uint4*>(
                    static_cast<const uint16_t*>(xin) + row * (int64_t)K + 8 * i);
                const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[j].v[2 * e] = bf16_to_float(w[e] & 0xffffu);
                    x[j].v[2 * e + 1] = bf16_to_float(w[e] >> 16);
                }
            } else {
                const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(xin) +
                                                                  row * (int64_t)K + 8 * i);
                const float4 a = p[0], b = p[1];
                x[j].v[0] = a.x; x[j].v[1] = a.y; x[j].v[2] = a.z; x[j].v[3] = a.w;
                x[j].v[4] = b.x; x[j].v[5] = b.y; x[j].v[6] = b.z; x[j].v[7] = b.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[j].v[e] = 0.0f;
        }
    }

    if constexpr (G > 0) {
        constexpr float kNorm = (G == 256) ? 0.0625f : 0.125f;  // 2^-(log2 g)/2, exact
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            fwht_vec_inlane<G>(x[j]);
            fwht_vec_crosslane<G>(x[j], lane);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[j].v[e] = x[j].v[e] * kNorm;
        }
    }

    float amax = 0.0f;
    int bad = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float a = fabsf(x[j].v[e]);
            amax = fmaxf(amax, a);
            if constexpr (CHECK) bad |= !(a <= 3.40282347e38f);
        }
    amax = wave_max(amax);
    float scale = amax / (float)QMAX;
    if constexpr (CHECK) {
        if (wave_or(bad)) scale = __uint_as_float(0x7fc00000u);
    }

#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int i = lane + 64 * j;
        if (i >= nvec) continue;
        int c[8];
        if (CHECK && scale != scale) {
#pragma unroll
            for (int e = 0; e < 8; ++e) c[e] = 0;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) c[e] = quant_code<QMAX>(x[j].v[e], scale);
        }
        if constexpr (OUT == Out::kRowI4 || OUT == Out::kTiledI4) {
            // row-major: code e in nibble e (even k low); tiled: codes 0-3 in the low nibbles of bytes 0-3 and
            // codes 4-7 in their high nibbles, so the GEMM widens a word with two masks
            uint32_t packed = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                packed |= (uint32_t)(c[e] & 0xf) << (OUT == Out::kTiledI4 ? 8 * (e & 3) + 4 * (e >> 2) : 4 * e);
            const int64_t off = (OUT == Out::kRowI4)
                                    ? row * (int64_t)(K / 2) + 4 * i
                                    : expert * (int64_t)(((N + 31) >> 5) << 5) * (K / 2) + tiled_offset<true>(n, 8 * i, K);
            *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(qout) + off) = packed;
        } else {
            uint2 o;
            o.x = pack4_i8(c[0], c[1], c[2], c[3]);
            o.y = pack4_i8(c[4], c[5], c[6], c[7]);
            const int64_t off = (OUT == Out::kRowI8)
                                    ? row * (int64_t)K + 8 * i
                                    : expert * (int64_t)(((N + 31) >> 5) << 5) * K + tiled_offset<false>(n, 8 * i, K);
            *reinterpret_cast<uint2*>(static_cast<int8_t*>(qout) + off) = o;
        }
        if (pad) continue;
        if (rot_out) {
            float4* r = reinterpret_cast<float4*>(rot_out + row * (int64_t)K + 8 * i);
            r[0] = make_float4(x[j].v[0], x[j].v[1], x[j].v[2], x[j].v[3]);
            r[1] = make_float4(x[j].v[4], x[j].v[5], x[j].v[6], x[j].v[7]);
        }
    }
    if (lane == 0 && !pad) sout[row] = scale;
}

template <int G, int R>
__global__ __launch_bounds__(256) void rotq_act_fast_kernel(const uint16_t* __restrict__ x, int64_t rows, int K,
                                                            int8_t* __restrict__ q, float* __restrict__ s) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;  // wave-uniform
    rotq_fast_row<G, R>(x, row, K, q, s);
}

// Long rows (R = K / 8g above 1 for g = 256, above 4 for g = 64): WPR wavefronts share a row, RW rounds each, and
// take its maximum from one another through LDS.  One round of g = 256 per lane holds 54 VGPRs where four hold
// 217, so the split runs 8 wavefronts per SIMD instead of 2.
template <int G, int RW, int WPR>
__global__ __launch_bounds__(256) void rotq_act_split_kernel(const uint16_t* __restrict__ x, int64_t rows, int K,
                                                             int8_t* __restrict__ q, float* __restrict__ s) {
    __shared__ float xch[4];
    const int w = threadIdx.x >> 6;
    const int64_t row = (int64_t)blockIdx.x * (4 / WPR) + w / WPR;
    rotq_fast_part<G, RW, WPR>(x, row, row < rows, K, w % WPR, q, s, xch);
}

// ---- LoRA patch of quantised weights, re-quantised with random rounding ----------------------------------
// NitroFusion2 page ("Why a step-1 file"): a LoRA applied to a quantised file is re-quantised with fresh
// scales and random rounding; XB loader page ("Inputs that matter"): a stochastic LoRA mode bakes LoRAs in at
// load with random-rounding deltas.  Per row n of expert e, in the rotated basis:
//   R = (float)q * s;  D[k] = alpha * sum_j B[n, j] * A[j, k] (ascending j from +0, separate mul and add);
//   V = R + rotate_g(D);  scale = max|V| / 127;  t = V / scale;
//   code = clamp(floor(t) + (u < t - floor(t)), -127, 127), u = top 24 bits of a Philox4x64-10 word times 2^-24
//   (counter ((e N + n) K/4 + k/4, 0, 0, 0), key (seed, 0), word k % 4).

// Philox4x64 with 10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3",
// SC 2011): each round takes the full 128-bit products of counter words 0 and 2 with the two multipliers;
// the key advances by the two Weyl constants before every round but the first.
__device__ __forceinline__ void philox4x64_10(uint64_t (&c)[4], uint64_t k0, uint64_t k1) {
    constexpr uint64_t kM0 = 0xD2E7470EE14C6C93ull, kM1 = 0xCA5A826395121157ull;
    constexpr uint64_t kW0 = 0x9E3779B97F4A7C15ull, kW1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += kW0;
            k1 += kW1;
        }
        const uint64_t lo0 = kM0 * c[0], hi0 = __umul64hi(kM0, c[0]);
        const uint64_t lo1 = kM1 * c[2], hi1 = __umul64hi(kM1, c[2]);
        const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = lo1;
        c[2] = n2;
        c[3] = lo0;
    }
}

// One wavefront per row (rows in the launch order of rotq_rows_kernel: tiled modes include the padding rows of
// the last 32-row block, which get zero codes).  Lane l holds the vectors i = l + 64 j (elements 8i .. 8i+7).
template <int G, int NV, Out OUT>
__global__ __launch_bounds__(256) void lora_requant_kernel(const int8_t* __restrict__ qin, const float* __restrict__ sin,
                                                           int64_t rows, int K, int N,
                                                           const uint16_t* __restrict__ lb,
                                                           const uint16_t* __restrict__ la, int rank, float alpha,
                                                           uint64_t seed, int nearest, int8_t* __restrict__ qout,
                                                           float* __restrict__ sout) {
    constexpr bool kTiled = OUT == Out::kTiledI8;
    const int lane = threadIdx.x & 63;
    const int64_t lrow = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    int64_t row = lrow, expert = 0;
    int n = 0;
    bool pad = false;
    if constexpr (kTiled) {
        const int nbr = ((N + 31) >> 5) << 5;
        expert = lrow / nbr;
        n = (int)(lrow - expert * nbr);
        if (expert * N >= rows) return;  // wave-uniform
        pad = n >= N;
        row = expert * N + n;
    } else {
        if (row >= rows) return;  // wave-uniform
        expert = row / N;
    }
    const int nvec = K >> 3;

    // delta row, then rotated
    Vec8 d[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) d[j].v[e] = 0.0f;
    if (!pad) {
        for (int r = 0; r < rank; ++r) {
            const float b = bf16_to_float(lb[row * rank + r]);
            const uint16_t* arow = la + (expert * rank + r) * (int64_t)K;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const int i = lane + 64 * j;
                if (i >= nvec) continue;
                const uint4 raw = *reinterpret_cast<const uint4*>(arow + 8 * i);
                const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p0 = b * bf16_to_float(w[e] & 0xffffu);
                    const float p1 = b * bf16_to_float(w[e] >> 16);
                    d[j].v[2 * e] = d[j].v[2 * e] + p0;
                    d[j].v[2 * e + 1] = d[j].v[2 * e + 1] + p1;
                }
            }
        }
    }
    constexpr float kNorm = (G == 256) ? 0.0625f : 0.125f;  // 2^-(log2 g)/2, exact
#pragma unroll
    for (int j = 0; j < NV; ++j) {
#pragma unroll
        for (int e = 0; e < 8; ++e) d[j].v[e] = alpha * d[j].v[e];
        fwht_vec_inlane<G>(d[j]);
        fwht_vec_crosslane<G>(d[j], lane);
#pragma unroll
        for (int e = 0; e < 8; ++e) d[j].v[e] = d[j].v[e] * kNorm;
    }

    // patched rotated row and its maximum
    const float s0 = pad ? 0.0f : sin[row];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int i = lane + 64 * j;
        int8_t c8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (i < nvec && !pad) {
            const uint2 raw = *reinterpret_cast<const uint2*>(qin + row * (int64_t)K + 8 * i);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                c8[e] = (int8_t)(raw.x >> (8 * e));
                c8[4 + e] = (int8_t)(raw.y >> (8 * e));
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float r = (float)c8[e] * s0;
            d[j].v[e] = (i < nvec) ? r + d[j].v[e] : 0.0f;
            amax = fmaxf(amax, fabsf(d[j].v[e]));
        }
    }
    amax = wave_max(amax);
    const float scale = amax / 127.0f;

    const int64_t flat0 = row * (int64_t)(K / 4);  // Philox counter of this row's first 4 elements
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int i = lane + 64 * j;
        if (i >= nvec) continue;
        int c[8];
        if (nearest) {  // wave-uniform: the re-quantising mode, the weight quantiser on the patched values
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float code = 0.0f;
                if (scale != 0.0f) code = fminf(fmaxf(rintf(d[j].v[e] / scale), -127.0f), 127.0f);
                c[e] = pad ? 0 : (int)code;
            }
        }
#pragma unroll
        for (int h = 0; h < 2 && !nearest; ++h) {
            uint64_t ctr[4] = {(uint64_t)(flat0 + 2 * i + h), 0, 0, 0};
            philox4x64_10(ctr, seed, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float u = (float)(ctr[e] >> 40) * 0x1p-24f;
                float code = 0.0f;
                if (scale != 0.0f) {
                    const float t = d[j].v[4 * h + e] / scale;
                    const float fl = floorf(t);
                    code = fl + (u < t - fl ? 1.0f : 0.0f);
                    code = fminf(fmaxf(code, -127.0f), 127.0f);
                }
                c[4 * h + e] = pad ? 0 : (int)code;
            }
        }
        uint2 o;
        o.x = pack4_i8(c[0], c[1], c[2], c[3]);
        o.y = pack4_i8(c[4], c[5], c[6], c[7]);
        const int64_t off = kTiled ? expert * (int64_t)(((N + 31) >> 5) << 5) * K + tiled_offset<false>(n, 8 * i, K)
                                   : row * (int64_t)K + 8 * i;
        *reinterpret_cast<uint2*>(qout + off) = o;
    }
    if (lane == 0 && !pad) sout[row] = scale;
}

// rows: source rows (E * N for weights); N: rows per expert (tiled modes only).
template <int G, int QMAX, Out OUT, bool CHECK>
hipError_t launch_nv(const void* x, int64_t rows, int K, int N, void* q, float* s, float* rot, hipStream_t st) {
    const int nv = (K / 8 + 63) / 64;
    int64_t launch_rows = rows;
    if (OUT == Out::kTiledI8 || OUT == Out::kTiledI4) launch_rows = rows / N * (((N + 31) >> 5) << 5);
    const dim3 grid((unsigned)((launch_rows + 3) / 4)), block(256);
#define CRK_NV_CASE(NVC)                                                                                 \
    if (nv <= NVC) {                                                                                     \
        rotq_rows_kernel<G, NVC, QMAX, OUT, CHECK><<<grid, block, 0, st>>>(x, rows, K, N, q, s, rot);    \
        return hipGetLastError();                                                                        \
    }
    CRK_NV_CASE(1)
    CRK_NV_CASE(2)
    CRK_NV_CASE(3)
    CRK_NV_CASE(4)
    CRK_NV_CASE(6)
    CRK_NV_CASE(8)
    CRK_NV_CASE(12)
    CRK_NV_CASE(16)
#undef CRK_NV_CASE
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_rotq_act(const uint16_t* x, int64_t rows, int K, int group, int8_t* q, float* s, float* rot,
                           hipStream_t st) {
    if (rows == 0) return hipSuccess;
    if (rot == nullptr && K % (8 * group) == 0) {
        const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
        const int R = K / (8 * group);
#define CRK_FAST(G, RR)                                                                          \
    if (group == G && R == RR) {                                                                 \
        rotq_act_fast_kernel<G, RR><<<grid, block, 0, st>>>(x, rows, K, q, s);                   \
        return hipGetLastError();                                                                \
    }
#define CRK_SPLIT(G, RR, RW, WPR)                                                                          \
    if (group == G && R == RR) {                                                                           \
        const dim3 sgrid((unsigned)((rows + 4 / WPR - 1) / (4 / WPR)));                                    \
        rotq_act_split_kernel<G, RW, WPR><<<sgrid, block, 0, st>>>(x, rows, K, q, s);                      \
        return hipGetLastError();                                                                          \
    }
        CRK_FAST(256, 1)
        CRK_SPLIT(256, 2, 1, 2)
        CRK_SPLIT(256, 4, 1, 4)
        CRK_FAST(64, 1)
        CRK_FAST(64, 2)
        CRK_FAST(64, 3)
        CRK_FAST(64, 4)
        CRK_SPLIT(64, 6, 3, 2)
        CRK_SPLIT(64, 8, 2, 4)
#undef CRK_SPLIT
#undef CRK_FAST
    }
    if (group == 256) return launch_nv<256, 127, Out::kRowI8, false>(x, rows, K, 0, q, s, rot, st);
    return launch_nv<64, 127, Out::kRowI8, false>(x, rows, K, 0, q, s, rot, st);
}

hipError_t launch_requantize_lora(const int8_t* qin, const float* sin, int E, int N, int K, int group,
                                  const uint16_t* lb, const uint16_t* la, int rank, float alpha, uint64_t seed,
                                  bool nearest, bool tiled, int8_t* qout, float* sout, hipStream_t st) {
    const int64_t rows = (int64_t)E * N;
    if (rows == 0) return hipSuccess;
    const int nv = (K / 8 + 63) / 64;
    const int64_t launch_rows = tiled ? (int64_t)E * (((N + 31) >> 5) << 5) : rows;
    const dim3 grid((unsigned)((launch_rows + 3) / 4)), block(256);
#define CRK_LR(GG, NVC)                                                                                       \
    if (group == GG && nv <= NVC) {                                                                           \
        if (tiled)                                                                                            \
            lora_requant_kernel<GG, NVC, Out::kTiledI8><<<grid, block, 0, st>>>(qin, sin, rows, K, N, lb, la, \
                                                                                 rank, alpha, seed, nearest,    \
                                                                                 qout, sout);                   \
        else                                                                                                  \
            lora_requant_kernel<GG, NVC, Out::kRowI8><<<grid, block, 0, st>>>(qin, sin, rows, K, N, lb, la,   \
                                                                               rank, alpha, seed, nearest,      \
                                                                               qout, sout);                     \
        return hipGetLastError();                                                                             \
    }
    CRK_LR(256, 4)
    CRK_LR(256, 8)
    CRK_LR(256, 16)
    CRK_LR(64, 1)
    CRK_LR(64, 2)
    CRK_LR(64, 4)
    CRK_LR(64, 8)
    CRK_LR(64, 16)
#undef CRK_LR
    return hipErrorInvalidValue;
}

hipError_t launch_rotq_weights(const uint16_t* w, int E, int N, int K, int group, int bits, bool tiled, void* q,
                               float* s, hipStream_t st) {
    const int64_t rows = (int64_t)E * N;
    if (rows == 0) return hipSuccess;
#define CRK_W(G, QMAX, OUTM) return launch_nv<G, QMAX, OUTM, true>(w, rows, K, N, q, s, nullptr, st)
    if (bits == 8) {
        if (tiled) {
            if (group == 256) CRK_W(256, 127, Out::kTiledI8);
            CRK_W(64, 127, Out::kTiledI8);
        }
        if (group == 256) CRK_W(256, 127, Out::kRowI8);
        CRK_W(64, 127, Out::kRowI8);
    }
    if (tiled) {
        if (group == 256) CRK_W(256, 7, Out::kTiledI4);
        CRK_W(64, 7, Out::kTiledI4);
    }
    if (group == 256) CRK_W(256, 7, Out::kRowI4);
    CRK_W(64, 7, Out::kRowI4);
#undef CRK_W
}

hipError_t launch_quantize_prerotated(const float* r, int64_t rows, int K, int bits, int8_t* q, float* s,
                                      hipStream_t st) {
    if (rows == 0) return hipSuccess;
    if (bits == 8) return launch_nv<0, 127, Out::kRowI8, false>(r, rows, K, 0, q, s, nullptr, st);
    return launch_nv<0, 7, Out::kRowI8, false>(r, rows, K, 0, q, s, nullptr, st);
}

}  // namespace crk
