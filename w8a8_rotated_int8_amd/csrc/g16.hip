// W6A8 / W4A8 linears: 6- or 4-bit weight codes in the rotated basis with an FP8 scale per group of 16
// ("NitroFusion2 for ComfyUI: int8, W6A8, W4A8", "How they were made"), 8-bit activations.
//
// Format (the library's reading of the page, as in include/convrot.h):
//   - rotation: the same block Hadamard as the int8 format, in fp32;
//   - codes: symmetric integers, qmax = 31 (6 bits) or 7 (4 bits), nearest rounding, ties to even;
//   - FP8 = E4M3 (bias 7, 3 mantissa bits, subnormals, largest 448), one per 16 consecutive k, relative to one
//     fp32 scale per row: s_row = amax / (qmax * 448), f = E4M3((amax_group / amax) * 448), the group's scale
//     s_row * f, code = clamp(rint(r / (s_row * f)), +-qmax);
//   - packing: 4-bit as two's-complement nibbles, even k low; 6-bit codes 4j..4j+3 in the little-endian
//     24-bit word j (code 4j+i in bits 6i..6i+5).
//
// The GEMM multiplies in fp16 on the matrix cores: an int8 activation code and a decoded weight code * f are
// both exact in fp16 (at most 9 significant bits, within its range), so every product is exact in the fp32
// accumulator; y = bf16((acc * s_x) * s_row) (+ bias).
#include <cstddef>
#include <cstdint>

#include "device_common.h"
#include "kernels.h"

namespace crk {
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// ---- E4M3 -------------------------------------------------------------------------------------------------
// Non-negative fp32 -> E4M3 byte, nearest value with ties to the even mantissa; 448 and above give 448.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
    if (!(x > 0.0f)) return 0u;
    if (x >= 448.0f) return 0x7eu;
    int E = (int)(__float_as_uint(x) >> 23) - 127;  // x in [2^E, 2^(E+1)) (fp32 subnormals round to 0 below)
    if (E < -6) E = -6;                             // the subnormal spacing 2^-9 continues below 2^-6
    int n = (int)rintf(ldexpf(x, 3 - E));           // x in units of the spacing 2^(E-3)
    if (E == -6 && n < 8) return (uint32_t)n;
    if (n == 16) {
        E += 1;
        n = 8;
    }
    return (uint32_t)(((E + 7) << 3) | (n - 8));
}
// E4M3 byte (no NaN code) -> value.
__device__ __forceinline__ float e4m3_decode(uint32_t b) {
    const int e = (int)((b >> 3) & 15u), m = (int)(b & 7u);
    const float v = e == 0 ? ldexpf((float)m, -9) : ldexpf((float)(8 + m), e - 10);
    return (b & 0x80u) ? -v : v;
}

// ---- converter: one workgroup per row ---------------------------------------------------------------------
// The row is rotated in LDS by the fast transform, stage by stage (h = 1, 2, ..., g/2, pairs (i, i + h) with
// bit h of i's offset clear becoming (a + b, a - b)), then scaled by 2^-(log2 g)/2; then each group of 16 is
// quantised by one thread.
constexpr int kConvThreads = 256;

template <int BITS>
__global__ __launch_bounds__(kConvThreads) void quantize_g16_kernel(const uint16_t* __restrict__ w, int K, int g,
                                                                    uint8_t* __restrict__ q, uint8_t* __restrict__ f8,
                                                                    float* __restrict__ s_row) {
    constexpr int kQmax = BITS == 6 ? 31 : 7;
    extern __shared__ float row[];
    __shared__ float red[kConvThreads / 64];
    const int tid = threadIdx.x;
    const int64_t n = blockIdx.x;
    for (int k = tid; k < K; k += kConvThreads) row[k] = bf16_to_float(w[n * K + k]);
    __syncthreads();
    const int half = g / 2;
    for (int h = 1; h < g; h *= 2) {
        for (int p = tid; p < K / 2; p += kConvThreads) {
            const int blk = p / half, j = p % half;
            const int i0 = blk * g + (j / h) * 2 * h + (j % h);
            const float a = row[i0], b = row[i0 + h];
            row[i0] = a + b;
            row[i0 + h] = a - b;
        }
        __syncthreads();
    }
    const float norm = g == 256 ? 0.0625f : 0.125f;  // 2^-(log2 g)/2, exact
    float amax = 0.0f;
    for (int k = tid; k < K; k += kConvThreads) {
        const float v = row[k] * norm;
        row[k] = v;
        amax = fmaxf(amax, fabsf(v));
    }
    amax = wave_max(amax);
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float sr = amax / (float)(kQmax * 448);
    if (tid == 0) s_row[n] = sr;
    const int groups = K / 16;
    for (int j = tid; j < groups; j += kConvThreads) {
        const float* v = row + 16 * j;
        float aj = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) aj = fmaxf(aj, fabsf(v[i]));
        uint32_t f = 0u;
        if (amax > 0.0f) {
            const float ratio = aj / amax;
            f = e4m3_encode(ratio * 448.0f);
        }
        f8[n * groups + j] = (uint8_t)f;
        const float S = sr * e4m3_decode(f);
        int c[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float t = 0.0f;
            if (S != 0.0f) t = fminf(fmaxf(rintf(v[i] / S), -(float)kQmax), (float)kQmax);
            c[i] = (int)t;
        }
        if constexpr (BITS == 4) {
            uint8_t* o = q + n * (K / 2) + 8 * j;
#pragma unroll
            for (int b = 0; b < 8; ++b) o[b] = (uint8_t)((c[2 * b] & 15) | ((c[2 * b + 1] & 15) << 4));
        } else {
            uint8_t* o = q + n * (K / 4 * 3) + 12 * j;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                uint32_t wd = 0u;
#pragma unroll
                for (int i = 0; i < 4; ++i) wd |= ((uint32_t)c[4 * u + i] & 63u) << (6 * i);
                o[3 * u] = (uint8_t)wd;
                o[3 * u + 1] = (uint8_t)(wd >> 8);
                o[3 * u + 2] = (uint8_t)(wd >> 16);
            }
        }
    }
}

// ---- GEMM + dequant ---------------------------------------------------------------------------------------
// Workgroup tile 256 tokens x 256 weight rows, 8 wavefronts of 64 tokens x 128 rows (2 x 4 blocks of 32 x 32),
// K in steps of 64 (four groups).  Each step is staged in LDS already decoded to fp16 (tokens: code; weights:
// code * f), double-buffered (144 KiB): the step after the current one is decoded into the other buffer while
// the current one is multiplied, and the global loads of the step after that are in flight.  The 256 x 256 tile measured 18 % faster than 128 x 128 (half the decode and a third less LDS
// traffic per multiply-add), and K steps of 64 faster than 32.
constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kGemmThreads = 512;
constexpr int kWN = 4;  // 32-row weight blocks per wavefront (wavefront tile 64 tokens x 128 rows)
constexpr int kGPT = kBK / 32;        // groups of 16 per thread per step (two threads per row)
constexpr int kRowHalves = kBK + 8;  // LDS row pitch: the 16-byte pad spreads the fragment reads over the banks

template <int BITS>
struct StageRegs {
    uint4 a[kGPT];                        // 16 token codes per group
    uint32_t b[kGPT][BITS == 6 ? 3 : 2];  // 16 packed weight codes per group
    uint32_t f[kGPT];                     // their E4M3 scales
};

template <int BITS>
__device__ __forceinline__ void stage_load(StageRegs<BITS>& r, const int8_t* __restrict__ qx, int M, int K,
                                           const uint8_t* __restrict__ qw, const uint8_t* __restrict__ f8, int N,
                                           int m0, int n0, int k0) {
    const int t = threadIdx.x, row = t >> 1, hk = t & 1;
    const int m = min(m0 + row, M - 1), n = min(n0 + row, N - 1);  // rows past the end compute unused outputs
#pragma unroll
    for (int u = 0; u < kGPT; ++u) {
        const int grp = k0 / 16 + kGPT * hk + u;
        r.a[u] = *reinterpret_cast<const uint4*>(qx + (int64_t)m * K + 16 * grp);
        if constexpr (BITS == 4) {
            const uint2 v = *reinterpret_cast<const uint2*>(qw + (int64_t)n * (K / 2) + 8 * grp);
            r.b[u][0] = v.x;
            r.b[u][1] = v.y;
        } else {
            const uint32_t* p = reinterpret_cast<const uint32_t*>(qw + (int64_t)n * (K / 4 * 3) + 12 * grp);
            r.b[u][0] = p[0];
            r.b[u][1] = p[1];
            r.b[u][2] = p[2];
        }
        r.f[u] = f8[(int64_t)n * (K / 16) + grp];
    }
}

// Decoding to fp16 with integer operations: for a code c in [-2^(b-1), 2^(b-1)), the half whose bits are
// 0x6400 | (c + 2^(b-1)) is 1024 + c + 2^(b-1) exactly, so one packed fp16 subtraction of 1024 + 2^(b-1) gives
// c, two codes per 32-bit register (and c * f is exact too).  The two codes of a register are k and k + 4 of an
// 8-wide chunk, so a chunk is stored in the order k0, k4, k1, k5, k2, k6, k3, k7 -- for the tokens and the
// weights alike, which leaves every dot product unchanged.
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t h2_bits(h2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ h2 bits_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }

// Group u of this thread's token codes, decoded, into the stage's token rows.
template <int BITS>
__device__ __forceinline__ void stage_store_tokens(const StageRegs<BITS>& r, int u, _Float16* As) {
    const int t = threadIdx.x, row = t >> 1, hk = t & 1;
    uint32_t a[8];
    // bytes k and k + 4 of each 8-byte chunk into one register, sign bit flipped (x + 128 in 0..255)
    const uint32_t aw[4] = {r.a[u].x, r.a[u].y, r.a[u].z, r.a[u].w};
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t x = __builtin_amdgcn_perm(aw[2 * c + 1], aw[2 * c], 0x0c040c00u + (uint32_t)(i | (i << 16)));
            a[4 * c + i] = h2_bits(bits_h2(x ^ 0x64806480u) - h2{(_Float16)1152.0f, (_Float16)1152.0f});
        }
    uint32_t* ao = reinterpret_cast<uint32_t*>(As + row * kRowHalves + 16 * (kGPT * hk + u));
    *reinterpret_cast<uint4*>(ao) = make_uint4(a[0], a[1], a[2], a[3]);
    *reinterpret_cast<uint4*>(ao + 4) = make_uint4(a[4], a[5], a[6], a[7]);
}

// Group u of this thread's weight codes, decoded and scaled by the group's E4M3 factor, into the weight rows.
template <int BITS>
__device__ __forceinline__ void stage_store_weights(const StageRegs<BITS>& r, int u, _Float16* Bs) {
    const int t = threadIdx.x, row = t >> 1, hk = t & 1;
    uint32_t b[8];
    const _Float16 fh = (_Float16)e4m3_decode(r.f[u]);  // every E4M3 value is an fp16 value
    const h2 f2{fh, fh};
    if constexpr (BITS == 4) {
        // word c holds codes 8c..8c+7 as nibbles; (w >> 4i) & 0x000f000f puts codes i and i + 4 in the halves
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t x = (r.b[u][c] >> (4 * i)) & 0x000f000fu;
                b[4 * c + i] =
                    h2_bits((bits_h2(x ^ 0x64086408u) - h2{(_Float16)1032.0f, (_Float16)1032.0f}) * f2);
            }
    } else {
        // code j at bit 6 j of the 96-bit run; alignbit takes a field that straddles two words
        auto field = [&](int j) -> uint32_t {
            const int p = 6 * j, w = p >> 5;
            const uint32_t hi = w + 1 < 3 ? r.b[u][w + 1] : 0u;
            return __builtin_amdgcn_alignbit(hi, r.b[u][w], (uint32_t)(p & 31)) & 63u;
        };
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t x = field(8 * c + i) | (field(8 * c + i + 4) << 16);
                b[4 * c + i] =
                    h2_bits((bits_h2(x ^ 0x64206420u) - h2{(_Float16)1056.0f, (_Float16)1056.0f}) * f2);
            }
    }
    uint32_t* bo = reinterpret_cast<uint32_t*>(Bs + row * kRowHalves + 16 * (kGPT * hk + u));
    *reinterpret_cast<uint4*>(bo) = make_uint4(b[0], b[1], b[2], b[3]);
    *reinterpret_cast<uint4*>(bo + 4) = make_uint4(b[4], b[5], b[6], b[7]);
}

// Part p (0..3) of a stage's decode: tokens or weights (p % 2) of group p / 2.
template <int BITS>
__device__ __forceinline__ void stage_store_part(const StageRegs<BITS>& r, int p, _Float16* As, _Float16* Bs) {
    if (p & 1)
        stage_store_weights<BITS>(r, p >> 1, Bs);
    else
        stage_store_tokens<BITS>(r, p >> 1, As);
}

template <int BITS>
__device__ __forceinline__ void stage_store(const StageRegs<BITS>& r, _Float16* As, _Float16* Bs) {
#pragma unroll
    for (int p = 0; p < 2 * kGPT; ++p) stage_store_part<BITS>(r, p, As, Bs);
}

template <int BITS>
__global__ __launch_bounds__(kGemmThreads) void gemm_g16_kernel(const int8_t* __restrict__ qx,
                                                                const float* __restrict__ sx, int M, int K,
                                                                const uint8_t* __restrict__ qw,
                                                                const uint8_t* __restrict__ f8,
                                                                const float* __restrict__ s_row, int N,
                                                                const uint16_t* __restrict__ bias,
                                                                uint16_t* __restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) _Float16 g16_lds[];
    _Float16* const lds_base = g16_lds;
    auto Abuf = [&](int b) { return lds_base + b * (kBM * kRowHalves); };
    auto Bbuf = [&](int b) { return lds_base + 2 * kBM * kRowHalves + b * (kBN * kRowHalves); };
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;  // wm 0..3 (64 tokens), wn 0..1 (128 rows)
    const int n0 = blockIdx.x * kBN, m0 = blockIdx.y * kBM;
    const int nk = K / kBK;

    v16f acc[2][kWN];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < kWN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Stage kt is multiplied from LDS buffer kt % 2 while stage kt + 1, loaded into registers one step earlier,
    // is decoded into the other buffer, one quarter per 16-deep slice, so the decode's VALU work runs beside the
    // matrix work; the global loads of stage kt + 2 go to the second register set.  One barrier per step.
    StageRegs<BITS> ra, rb;
    stage_load<BITS>(ra, qx, M, K, qw, f8, N, m0, n0, 0);
    stage_store<BITS>(ra, Abuf(0), Bbuf(0));
    if (nk > 1) stage_load<BITS>(ra, qx, M, K, qw, f8, N, m0, n0, kBK);
    __syncthreads();
    // fragments of slice sl (16 deep): row lane % 32 of a 32-row block, halves 16 sl + 8 (lane / 32) .. + 8
    auto read_frags = [&](int buf, int sl, v8h (&af)[2], v8h (&bf)[kWN]) {
        const int col = 16 * sl + 8 * (lane >> 5);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            af[i] = *reinterpret_cast<const v8h*>(Abuf(buf) + (wm * 64 + 32 * i + (lane & 31)) * kRowHalves + col);
#pragma unroll
        for (int j = 0; j < kWN; ++j)
            bf[j] = *reinterpret_cast<const v8h*>(Bbuf(buf) + (wn * 128 + 32 * j + (lane & 31)) * kRowHalves + col);
    };
    auto step = [&](int kt, const StageRegs<BITS>& dec, StageRegs<BITS>& ld) {
        const int buf = kt & 1;
        if (kt + 2 < nk) stage_load<BITS>(ld, qx, M, K, qw, f8, N, m0, n0, (kt + 2) * kBK);
        // the next slice's fragments are read while the current slice multiplies
        v8h af[2][2], bf[2][kWN];
        read_frags(buf, 0, af[0], bf[0]);
#pragma unroll
        for (int sl = 0; sl < kBK / 16; ++sl) {
            if (sl + 1 < kBK / 16) read_frags(buf, sl + 1, af[(sl + 1) & 1], bf[(sl + 1) & 1]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < kWN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[sl & 1][j], af[sl & 1][i], acc[i][j], 0, 0, 0);
            // unconditional, to keep one scheduling region: on the last step it decodes stale registers into the
            // buffer no one reads any more (every read of it ended at the previous barrier)
            stage_store_part<BITS>(dec, sl, Abuf(buf ^ 1), Bbuf(buf ^ 1));
            // issue order: the next slice's fragment reads, then each MFMA followed by a few of the decode's
            // VALU instructions (they run while the MFMA does), then the decode's LDS stores
            __builtin_amdgcn_sched_group_barrier(0x100, 2 + kWN, 0);
#pragma unroll
            for (int m = 0; m < 2 * kWN; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);
        }
        __syncthreads();
    };
    for (int kt = 0; kt < nk; kt += 2) {
        step(kt, ra, rb);
        if (kt + 1 < nk) step(kt + 1, rb, ra);
    }

    // The weights are the MFMA's first operand: lane l holds token l % 32 of each 32 x 32 block and, in
    // register 4 q + i, weight row 8 q + 4 (l / 32) + i.
    const bool vec = (N & 3) == 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int m = m0 + wm * 64 + 32 * i + (lane & 31);
        if (m >= M) continue;
        const float sm = sx[m];
#pragma unroll
        for (int j = 0; j < kWN; ++j)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const int nb = n0 + wn * 128 + 32 * j + 8 * qd + 4 * (lane >> 5);
                uint32_t h[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int n = min(nb + e, N - 1);
                    float v = acc[i][j][4 * qd + e];
                    v = v * sm;
                    v = v * s_row[n];
                    if (bias) v = v + bf16_to_float(bias[n]);
                    h[e] = float_to_bf16(v);
                }
                uint16_t* out = y + (int64_t)m * N + nb;
                if (vec && nb + 3 < N) {
                    *reinterpret_cast<uint2*>(out) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (nb + e < N) out[e] = (uint16_t)h[e];
                }
            }
    }
}

}  // namespace

hipError_t launch_quantize_g16(const uint16_t* w, int N, int K, int group, int bits, uint8_t* q, uint8_t* f8,
                               float* s_row, hipStream_t st) {
    if (N == 0) return hipSuccess;
    const size_t lds = sizeof(float) * (size_t)K;  // the row, at most 32 KiB
    if (bits == 6)
        quantize_g16_kernel<6><<<dim3((unsigned)N), dim3(kConvThreads), lds, st>>>(w, K, group, q, f8, s_row);
    else
        quantize_g16_kernel<4><<<dim3((unsigned)N), dim3(kConvThreads), lds, st>>>(w, K, group, q, f8, s_row);
    return hipGetLastError();
}

hipError_t launch_gemm_g16(const int8_t* qx, const float* sx, int M, int K, const uint8_t* qw, const uint8_t* f8,
                           const float* s_row, int N, int bits, const uint16_t* bias, uint16_t* y, hipStream_t st) {
    const dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM)), block(kGemmThreads);
    constexpr size_t kLds = sizeof(_Float16) * 2 * (kBM + kBN) * kRowHalves;
    static const hipError_t a6 = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_g16_kernel<6>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
    static const hipError_t a4 = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_g16_kernel<4>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
    if (a6 != hipSuccess) return a6;
    if (a4 != hipSuccess) return a4;
    if (bits == 6)
        gemm_g16_kernel<6><<<grid, block, kLds, st>>>(qx, sx, M, K, qw, f8, s_row, N, bias, y);
    else
        gemm_g16_kernel<4><<<grid, block, kLds, st>>>(qx, sx, M, K, qw, f8, s_row, N, bias, y);
    return hipGetLastError();
}

}  // namespace crk
