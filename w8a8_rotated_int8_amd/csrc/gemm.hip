// Grouped INT8 x INT8 -> INT32 GEMM on gfx950 MFMA (v_mfma_i32_32x32x32_i8) with fused epilogues:
//   kI32    exact int32 accumulators (test export, plain GEMM)
//   kBf16   bf16( ((float)acc * s_act[row]) * s_w[n] ) [+ bias]      (single linear, expert down proj)
//   kSwiGLU gate and up of the same column in one workgroup, each dequantised to bf16, then
//           bf16( silu(gate) * up )                                   (expert gate/up proj)
//
// W8A8 ConvRot linear of the Nucleus-Image INT8 Convrot model card ("Quantization"; multiply in INT8 and
// dequantise on the fly as on the XB_UNetLoaderINTROCm page), inside the expert-choice MoE of
// "MLX Nucleus-Image" (SwiGLU convention silu(gate) * up, gate = first half of the fused projection).
//
// Work decomposition: one workgroup per (expert e, M-block, N-tile).  For the MoE the M-block covers all C
// slots of the expert when C <= 256, so every weight byte is read from HBM once per layer.  The activation
// rows of an expert are gathered through `a_rows` (row index per slot) directly in the global loads.
// Workgroup ids are remapped so that all N-tiles of an expert run on the same XCD and share its L2.
//
// Main loop: K-steps of 128 bytes (one full 128-byte line per row), double-buffered in LDS with register
// prefetch of the next step; each wave owns a (BM/WM) x (BN/WN) sub-tile of 32x32 MFMA blocks.  INT32
// accumulation is exact, so the result does not depend on the k order inside the MFMA.  4-bit weights are
// sign-extended to int8 in registers between the global load and the LDS store.
#include "device_common.h"
#include "kernels.h"

namespace crk {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kBK = 128;
constexpr int kLdsStride = kBK + 16;  // bytes per LDS row: 144 = 36 banks, conflict-free 16-byte reads

// Sign-extend the 8 nibbles of w (code 2j in the low nibble of byte j) into 8 int8 bytes, in k order.
__device__ __forceinline__ uint2 unpack_nibbles(uint32_t w) {
    uint32_t lo = w & 0x0f0f0f0fu;
    uint32_t hi = (w >> 4) & 0x0f0f0f0fu;
    lo |= (lo & 0x08080808u) * 0x1eu;  // 0x08 * 0x1e = 0xf0 per byte: fills the upper nibble with the sign
    hi |= (hi & 0x08080808u) * 0x1eu;
    uint2 r;
    r.x = (lo & 0xffu) | ((hi & 0xffu) << 8) | ((lo & 0xff00u) << 8) | ((hi & 0xff00u) << 16);
    r.y = ((lo >> 16) & 0xffu) | ((hi >> 8) & 0xff00u) | ((lo >> 8) & 0xff0000u) | (hi & 0xff000000u);
    return r;
}

template <int BM, int BN, int WM, int WN, Epi EPI, int WBITS>
__global__ __launch_bounds__(WM * WN * 64) void grouped_gemm_kernel(const GemmProblem p, int tiles_m,
                                                                     int tiles_n) {
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM / 32;
    constexpr int TN = BN / WN / 32;
    constexpr int KCH = kBK / 16;                 // 16-byte int8 chunks per row per K-step
    constexpr int A_CH = BM * KCH / NT;           // A chunks per thread
    constexpr int PB = (WBITS == 8) ? 16 : 32;    // codes per 16-byte global chunk of B
    constexpr int KCH_B = kBK / PB;               // global B chunks per row per K-step
    constexpr int B_CH = BN * KCH_B / NT;         // B chunks per thread
    static_assert(BM * KCH % NT == 0 && BN * KCH_B % NT == 0, "tile / thread mismatch");
    static_assert(EPI != Epi::kSwiGLU || TN % 2 == 0, "SwiGLU pairs gate and up fragments");

    extern __shared__ __attribute__((aligned(16))) int8_t smem[];

    const int total = p.E * tiles_m * tiles_n;
    const int tile = xcd_remap((int)blockIdx.x, total);
    const int nt = tile % tiles_n;
    const int mt = (tile / tiles_n) % tiles_m;
    const int e = tile / (tiles_n * tiles_m);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN;
    const int wn = wave % WN;
    const int M = p.M, N = p.N, K = p.K;
    const int I = N / 2;  // SwiGLU half width

    // ---- per-thread global source rows ----
    const int8_t* a_src[A_CH];
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
        const int c = tid + NT * i;
        const int r = c / KCH;
        int m = mt * BM + r;
        m = m < M ? m : M - 1;
        const int64_t slot = (int64_t)e * M + m;
        int64_t arow = p.a_rows ? (int64_t)p.a_rows[slot] : slot;
        arow = arow < 0 ? 0 : (arow < p.a_nrows ? arow : p.a_nrows - 1);
        a_src[i] = p.A + arow * K + (c % KCH) * 16;
    }
    const int8_t* b_src[B_CH];
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
        const int c = tid + NT * i;
        const int r = c / KCH_B;
        int n;
        if constexpr (EPI == Epi::kSwiGLU) {
            constexpr int H = BN / 2;
            if (r < H) {
                n = nt * H + r;
                n = n < I ? n : I - 1;
            } else {
                n = nt * H + (r - H);
                n = (n < I ? n : I - 1) + I;
            }
        } else {
            n = nt * BN + r;
            n = n < N ? n : N - 1;
        }
        const int64_t row_bytes = (WBITS == 8) ? K : K / 2;
        b_src[i] = static_cast<const int8_t*>(p.B) + ((int64_t)e * N + n) * row_bytes + (c % KCH_B) * 16;
    }

    v16i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    int4 ra[A_CH];
    int4 rb[B_CH];

    auto load_step = [&](int kt) {
        const int k0 = kt * kBK;
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int kk = k0 + ((tid + NT * i) % KCH) * 16;
            ra[i] = (kk < K) ? *reinterpret_cast<const int4*>(a_src[i] + k0) : make_int4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            const int kk = k0 + ((tid + NT * i) % KCH_B) * PB;
            const int off = (WBITS == 8) ? k0 : k0 / 2;
            rb[i] = (kk < K) ? *reinterpret_cast<const int4*>(b_src[i] + off) : make_int4(0, 0, 0, 0);
        }
    };

    auto store_step = [&](int buf) {
        int8_t* As = smem + buf * (BM + BN) * kLdsStride;
        int8_t* Bs = As + BM * kLdsStride;
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int c = tid + NT * i;
            *reinterpret_cast<int4*>(As + (c / KCH) * kLdsStride + (c % KCH) * 16) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            const int c = tid + NT * i;
            if constexpr (WBITS == 8) {
                *reinterpret_cast<int4*>(Bs + (c / KCH_B) * kLdsStride + (c % KCH_B) * 16) = rb[i];
            } else {
                const uint2 u0 = unpack_nibbles((uint32_t)rb[i].x), u1 = unpack_nibbles((uint32_t)rb[i].y);
                const uint2 u2 = unpack_nibbles((uint32_t)rb[i].z), u3 = unpack_nibbles((uint32_t)rb[i].w);
                int8_t* dst = Bs + (c / KCH_B) * kLdsStride + (c % KCH_B) * 32;
                *reinterpret_cast<int4*>(dst) = make_int4((int)u0.x, (int)u0.y, (int)u1.x, (int)u1.y);
                *reinterpret_cast<int4*>(dst + 16) = make_int4((int)u2.x, (int)u2.y, (int)u3.x, (int)u3.y);
            }
        }
    };

    auto b_tile_row = [&](int tn) -> int {
        if constexpr (EPI == Epi::kSwiGLU) {
            constexpr int HT = TN / 2;
            return tn < HT ? (wn * HT + tn) * 32 : BN / 2 + (wn * HT + tn - HT) * 32;
        } else {
            return (wn * TN + tn) * 32;
        }
    };

    auto compute_step = [&](int buf) {
        const int8_t* As = smem + buf * (BM + BN) * kLdsStride;
        const int8_t* Bs = As + BM * kLdsStride;
#pragma unroll
        for (int ks = 0; ks < kBK / 32; ++ks) {
            const int koff = ks * 32 + (lane >> 5) * 16;
            v4i af[TM], bfr[TN];
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
                af[tm] = *reinterpret_cast<const v4i*>(As + (wm * (BM / WM) + tm * 32 + (lane & 31)) * kLdsStride + koff);
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
                bfr[tn] = *reinterpret_cast<const v4i*>(Bs + (b_tile_row(tn) + (lane & 31)) * kLdsStride + koff);
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
                    acc[tm][tn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[tm], bfr[tn], acc[tm][tn], 0, 0, 0);
        }
    };

    const int nk = (K + kBK - 1) / kBK;
    load_step(0);
    store_step(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) load_step(kt + 1);
        compute_step(kt & 1);
        if (kt + 1 < nk) store_step((kt + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds column (lane & 31) and rows 8(r/4) + 4(lane/32) + r%4 of each 32x32 block ----
    const int col = lane & 31;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const int mbase = mt * BM + wm * (BM / WM) + tm * 32 + (lane >> 5) * 4;
        if constexpr (EPI == Epi::kI32) {
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                const int n = nt * BN + (wn * TN + tn) * 32 + col;
                if (n >= N) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = mbase + (r >> 2) * 8 + (r & 3);
                    if (m < M)
                        static_cast<int32_t*>(p.out)[((int64_t)e * M + m) * N + n] = acc[tm][tn][r];
                }
            }
        } else {
            float srow[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = mbase + (r >> 2) * 8 + (r & 3);
                const int mm = m < M ? m : M - 1;
                const int64_t slot = (int64_t)e * M + mm;
                int64_t arow = p.a_rows ? (int64_t)p.a_rows[slot] : slot;
                arow = arow < 0 ? 0 : (arow < p.a_nrows ? arow : p.a_nrows - 1);
                srow[r] = p.a_scale[arow];
            }
            if constexpr (EPI == Epi::kBf16) {
#pragma unroll
                for (int tn = 0; tn < TN; ++tn) {
                    const int n = nt * BN + (wn * TN + tn) * 32 + col;
                    if (n >= N) continue;
                    const float sw = p.b_scale[(int64_t)e * N + n];
                    const float bias = p.bias ? bf16_to_float(p.bias[n]) : 0.0f;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int m = mbase + (r >> 2) * 8 + (r & 3);
                        if (m >= M) continue;
                        float v = (float)acc[tm][tn][r];
                        v = v * srow[r];
                        v = v * sw;
                        if (p.bias) v = v + bias;
                        static_cast<uint16_t*>(p.out)[((int64_t)e * M + m) * N + n] = (uint16_t)float_to_bf16(v);
                    }
                }
            } else {
                constexpr int HT = TN / 2;
#pragma unroll
                for (int tn = 0; tn < HT; ++tn) {
                    const int j = nt * (BN / 2) + (wn * HT + tn) * 32 + col;
                    if (j >= I) continue;
                    const float sg = p.b_scale[(int64_t)e * N + j];
                    const float su = p.b_scale[(int64_t)e * N + I + j];
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int m = mbase + (r >> 2) * 8 + (r & 3);
                        if (m >= M) continue;
                        float g = (float)acc[tm][tn][r];
                        g = g * srow[r];
                        g = g * sg;
                        float u = (float)acc[tm][tn + HT][r];
                        u = u * srow[r];
                        u = u * su;
                        const float gb = bf16_to_float(float_to_bf16(g));
                        const float ub = bf16_to_float(float_to_bf16(u));
                        const float a = silu_fixed(gb) * ub;
                        static_cast<uint16_t*>(p.out)[((int64_t)e * M + m) * I + j] = (uint16_t)float_to_bf16(a);
                    }
                }
            }
        }
    }
}

template <int BM, int WM, int WN, Epi EPI, int WBITS>
hipError_t launch_cfg(const GemmProblem& p, hipStream_t st) {
    constexpr int BN = 128;
    const int tiles_m = (p.M + BM - 1) / BM;
    const int tiles_n = (EPI == Epi::kSwiGLU) ? (p.N / 2 + BN / 2 - 1) / (BN / 2) : (p.N + BN - 1) / BN;
    const size_t lds = 2 * (size_t)(BM + BN) * kLdsStride;
    auto kern = grouped_gemm_kernel<BM, BN, WM, WN, EPI, WBITS>;
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess) return attr;
    const int64_t total = (int64_t)p.E * tiles_m * tiles_n;
    if (total <= 0) return hipSuccess;
    if (total > 0x7fffffff) return hipErrorInvalidValue;
    kern<<<dim3((unsigned)total), dim3(WM * WN * 64), lds, st>>>(p, tiles_m, tiles_n);
    return hipGetLastError();
}

template <Epi EPI, int WBITS>
hipError_t launch_epi(const GemmProblem& p, hipStream_t st) {
    if (p.M <= 64) return launch_cfg<64, 2, 2, EPI, WBITS>(p, st);
    if (p.M <= 128) return launch_cfg<128, 2, 2, EPI, WBITS>(p, st);
    return launch_cfg<256, 2, 2, EPI, WBITS>(p, st);
}

}  // namespace

hipError_t launch_grouped_gemm(const GemmProblem& p, hipStream_t st) {
    if (p.wbits == 4) {
        switch (p.epi) {
            case Epi::kI32: return launch_epi<Epi::kI32, 4>(p, st);
            case Epi::kBf16: return launch_epi<Epi::kBf16, 4>(p, st);
            case Epi::kSwiGLU: return launch_epi<Epi::kSwiGLU, 4>(p, st);
        }
    }
    switch (p.epi) {
        case Epi::kI32: return launch_epi<Epi::kI32, 8>(p, st);
        case Epi::kBf16: return launch_epi<Epi::kBf16, 8>(p, st);
        case Epi::kSwiGLU: return launch_epi<Epi::kSwiGLU, 8>(p, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace crk
