// Grouped INT8 x INT8 -> INT32 GEMM on gfx950 MFMA (v_mfma_i32_32x32x32_i8) with fused epilogues:
//   kI32    exact int32 accumulators (test export, plain GEMM)
//   kBf16   bf16( ((float)acc * s_act[row]) * s_w[n] ) [+ bias]      (single linear, expert down proj)
//   kSwiGLU gate and up of the same column in one wavefront, each dequantised to bf16, then
//           bf16( silu(gate) * up )                                   (expert gate/up proj)
//
// W8A8 ConvRot linear of the Nucleus-Image INT8 Convrot model card ("Quantization"; multiply in INT8 and
// dequantise on the fly as on the XB_UNetLoaderINTROCm page), inside the expert-choice MoE of
// "MLX Nucleus-Image" (SwiGLU convention silu(gate) * up, gate = first half of the fused projection).
//
// Work decomposition.  One workgroup (4 wavefronts) per (expert e, N-tile of 256 output columns, M-block of
// BM <= 128 rows); two workgroups share a CU.  The M-blocks of one (expert, N-tile) are consecutive tiles, so
// the weight panel is streamed from HBM once and re-read from L2 by the other M-blocks.  Wavefront w owns all BM rows and two 32-column blocks (for SwiGLU: the
// gate block and the up block of the same 32 columns, so the epilogue pairs them in registers).  Workgroup
// ids are remapped so that the N-tiles of one expert run on one XCD and share its L2 for the activations.
//
// Main loop, K-steps of 64 (two 32-deep MFMA slices), S-stage software pipeline:
//   * activations (gathered token rows for gate/up, contiguous slot rows for down) go global -> LDS with
//     gfx950's global_load_lds_dwordx4 into an S-deep LDS ring; rows are 64 bytes, 16-byte chunks XOR-
//     swizzled by (row / 4) % 4 so the 16-byte fragment reads are bank-conflict free;
//   * weights take the same DMA path into a wavefront-private LDS region of each stage: the MFMA-tiled
//     layout makes every (32-row block, K-block) tile 1 KiB in B-operand lane order, so each DMA is one
//     coalesced 16-byte load per lane and the fragment read is a contiguous ds_read_b128;
//   * per K-step: wait for the oldest stage (explicit vmcnt; every load of the loop is a DMA, so the count
//     is exact and no register load stalls the MFMAs), one workgroup barrier, issue the loads of stage
//     kt+S-1, then TM x 2 x 2 MFMAs on stage kt.
// INT32 accumulation is exact, so the result does not depend on the k order inside the MFMA.  4-bit weights
// are sign-extended to int8 in registers right before the MFMA.
#include "device_common.h"
#include "kernels.h"

namespace crk {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBK = 64;    // K bytes per pipeline stage (two MFMA slices)
constexpr int kBN = 256;   // output columns per workgroup (4 wavefronts x 2 blocks of 32)
constexpr int kThreads = 256;
// Cache policy of the weight DMAs: non-temporal (each weight byte is used by one workgroup, or by the M-blocks
// of one N-tile right after each other); streaming with nt measured ~6.5 TB/s vs ~5.7 TB/s without.
constexpr int kNonTemporal = 2;

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

// LDS byte offset of 16-byte chunk c (0..3) of row r inside one activation stage.
__device__ __forceinline__ int a_lds_offset(int r, int c) { return r * kBK + ((c ^ ((r >> 2) & 3)) << 4); }

// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt[5:4] in bits 15:14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// OCC: wavefronts per SIMD the register budget must allow (2: two workgroups share a CU, so one workgroup's
// epilogue overlaps the other's MFMA loop).
template <int BM, int S, int OCC, Epi EPI, int WBITS, bool TILED>
__global__ __launch_bounds__(kThreads, OCC) void grouped_gemm_kernel(const GemmProblem p, int tiles_m, int tiles_n) {
    constexpr int TM = BM / 32;                 // 32-row blocks per wavefront
    constexpr int NA = BM / 64;                 // activation DMA instructions per thread per stage
    constexpr int NBT = (WBITS == 8) ? 4 : 2;   // 1 KiB weight tiles per wavefront per stage
    constexpr int A_BYTES = BM * kBK;
    constexpr int B_WAVE = NBT * 1024;
    constexpr int STAGE = A_BYTES + 4 * B_WAVE;
    static_assert(BM % 64 == 0 && S >= 2, "tile config");
    static_assert(TILED || WBITS == 8, "4-bit weights are only stored tiled");

    // LDS: S stages of [activations | weights] (reused to stage the output tile after the main loop), then
    // the BM activation-row scales.
    extern __shared__ __attribute__((aligned(16))) int8_t smem[];
    constexpr int OUT_COLS = (EPI == Epi::kSwiGLU) ? kBN / 2 : kBN;
    constexpr int OUT_STRIDE = OUT_COLS * 2 + 16;  // bytes per staged output row (padded against bank conflicts)
    constexpr int RING = (S * STAGE > BM * OUT_STRIDE) ? S * STAGE : BM * OUT_STRIDE;
    float* srow_lds = reinterpret_cast<float*>(smem + RING);

    const int total = p.E * tiles_m * tiles_n;
    const int tile = xcd_remap((int)blockIdx.x, total);
    // M-blocks fastest: the M-blocks of one N-tile stream the same weight panel back to back on one XCD, so
    // all but the first read it from L2.
    const int mt = tile % tiles_m;
    const int nt = (tile / tiles_m) % tiles_n;
    const int e = tile / (tiles_n * tiles_m);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int M = p.M, N = p.N, K = p.K;
    const int I = N >> 1;
    const int nk = (K + kBK - 1) / kBK;

    // ---- activation sources: DMA instruction j of this wavefront fills LDS chunk slot s = (4j + w)*64 + lane ----
    const int8_t* a_src[NA];
    int a_koff[NA];
#pragma unroll
    for (int j = 0; j < NA; ++j) {
        const int slot = (4 * j + wave) * 64 + lane;
        const int r = slot >> 2;                     // tile row
        const int c = (slot & 3) ^ ((r >> 2) & 3);   // logical 16-byte chunk held by that slot
        int m = mt * BM + r;
        m = m < M ? m : M - 1;
        const int64_t sl = (int64_t)e * M + m;
        int64_t arow = p.a_rows ? (int64_t)p.a_rows[sl] : sl;
        arow = arow < 0 ? 0 : (arow < p.a_nrows ? arow : p.a_nrows - 1);
        a_src[j] = p.A + arow * K;
        a_koff[j] = c * 16;
    }

    // ---- weight blocks of this wavefront: q = 0, 1 ----
    int nblk[2];
    if constexpr (EPI == Epi::kSwiGLU) {
        const int jb = nt * 4 + wave;             // 32-column block of the gate/up halves
        nblk[0] = jb;                             // gate rows jb*32 ..
        nblk[1] = (I >> 5) + jb;                  // up rows I + jb*32 ..
    } else {
        nblk[0] = nt * 8 + 2 * wave;
        nblk[1] = nt * 8 + 2 * wave + 1;
    }
    const int NBk = (N + 31) >> 5;                // row blocks per expert
    const int8_t* b_base[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int nb = nblk[q] < NBk ? nblk[q] : NBk - 1;  // out-of-range blocks compute unused columns
        if constexpr (TILED) {
            const int64_t expert_bytes = (int64_t)NBk * 32 * K * WBITS / 8;
            b_base[q] = static_cast<const int8_t*>(p.B) + e * expert_bytes + (int64_t)nb * 32 * K * WBITS / 8 +
                        lane * 16;
        } else {
            int n = nb * 32 + (lane & 31);
            n = n < N ? n : N - 1;
            b_base[q] = static_cast<const int8_t*>(p.B) + ((int64_t)e * N + n) * K + (lane >> 5) * 16;
        }
    }

    // Loads of one stage.  Tiled weights: every 1 KiB tile is DMA'd into this wavefront's private LDS region
    // in lane order (exactly the MFMA operand layout).  Row-major weights (test path): registers with zero
    // fill past K, then ds_write into the same place.
    auto issue = [&](int kt, int buf) {
        int8_t* st = smem + buf * STAGE;
        const int k0 = kt * kBK;
#pragma unroll
        for (int j = 0; j < NA; ++j) {
            int k = k0 + a_koff[j];
            k = k <= K - 16 ? k : K - 16;  // past K the weights are zero, any in-bounds bytes do
            __builtin_amdgcn_global_load_lds(static_cast<const void*>(a_src[j] + k),
                                             (lds_void*)(st + (4 * j + wave) * 1024), 16, 0, 0);
        }
        int8_t* bw = st + A_BYTES + wave * B_WAVE;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            if constexpr (TILED && WBITS == 8) {
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    __builtin_amdgcn_global_load_lds(static_cast<const void*>(b_base[q] + (int64_t)(2 * kt + s) * 1024),
                                                     (lds_void*)(bw + (2 * q + s) * 1024), 16, 0, kNonTemporal);
            } else if constexpr (TILED) {
                __builtin_amdgcn_global_load_lds(static_cast<const void*>(b_base[q] + (int64_t)kt * 1024),
                                                 (lds_void*)(bw + q * 1024), 16, 0, kNonTemporal);
            } else {
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int k = k0 + s * 32 + (lane >> 5) * 16;
                    const v4i v = (k + 16 <= K) ? *reinterpret_cast<const v4i*>(b_base[q] + k0 + s * 32)
                                                : v4i{0, 0, 0, 0};
                    *reinterpret_cast<v4i*>(bw + (2 * q + s) * 1024 + lane * 16) = v;
                }
            }
        }
    };

    v16i acc[TM][2];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][q][r] = 0;

    // All fragments of both slices are read first (20 ds_read_b128 for BM = 256), so the LDS latency of later
    // fragments hides under the MFMAs of earlier ones.
    auto compute = [&](int buf) {
        const int8_t* As = smem + buf * STAGE;
        const int8_t* bw = As + A_BYTES + wave * B_WAVE + lane * 16;
        v4i bf[2][2];
        v4i af[2][TM];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                if constexpr (WBITS == 8) {
                    bf[s][q] = *reinterpret_cast<const v4i*>(bw + (2 * q + s) * 1024);
                } else {
                    const uint2 w = *reinterpret_cast<const uint2*>(bw + q * 1024 + 8 * s);
                    const uint2 u0 = unpack_nibbles(w.x), u1 = unpack_nibbles(w.y);
                    bf[s][q] = v4i{(int)u0.x, (int)u0.y, (int)u1.x, (int)u1.y};
                }
            }
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
                af[s][tm] = *reinterpret_cast<const v4i*>(As + a_lds_offset(tm * 32 + (lane & 31), 2 * s + (lane >> 5)));
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int q = 0; q < 2; ++q)
                    acc[tm][q] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[s][tm], bf[s][q], acc[tm][q], 0, 0, 0);
        // Scheduling order: every LDS read of the stage, then the MFMAs (the waitcnt pass then waits only for
        // the fragments each MFMA needs).
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * (TM + 2), 0);  // DS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 4 * TM, 0);        // MFMAs
    };

    // Row scales of the tile (gathered like the activation rows) into LDS, column scales into registers;
    // issued before the pipeline so their latency hides under it.
    float csc[2] = {0.0f, 0.0f};
    if constexpr (EPI != Epi::kI32) {
        for (int r = tid; r < BM; r += kThreads) {
            int m = mt * BM + r;
            m = m < M ? m : M - 1;
            const int64_t sl = (int64_t)e * M + m;
            int64_t arow = p.a_rows ? (int64_t)p.a_rows[sl] : sl;
            arow = arow < 0 ? 0 : (arow < p.a_nrows ? arow : p.a_nrows - 1);
            srow_lds[r] = p.a_scale[arow];
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            int n = nblk[q] * 32 + (lane & 31);
            n = n < N ? n : N - 1;
            csc[q] = p.b_scale[(int64_t)e * N + n];
        }
    }

    // prologue: stages 0 .. S-2 in flight
    for (int u = 0; u < S - 1 && u < nk; ++u) issue(u, u);

    for (int kt = 0; kt < nk; ++kt) {
        // Every stage is NA + NBT DMA instructions per thread (in issue order); stages kt+1 .. kt+S-2 may
        // still be in flight.
        if (kt + S - 2 < nk)
            wait_vmcnt<(S - 2) * (NA + NBT)>();
        else
            wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();  // all stage-kt data landed; everyone is done with stage kt-1
        // keeps the LDS reads of stage kt below the barrier (costs an lgkmcnt wait, not a vmcnt one)
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        if (kt + S - 1 < nk) issue(kt + S - 1, (kt + S - 1) % S);
        compute(kt % S);
    }

    // ---- epilogue: lane holds column (lane & 31) and rows 8(r/4) + 4(lane/32) + r%4 of each 32x32 block ----
    const int col = lane & 31;
    if constexpr (EPI == Epi::kI32) {
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
            const int mbase = mt * BM + tm * 32 + (lane >> 5) * 4;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int n = nblk[q] * 32 + col;
                if (n >= N) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = mbase + (r >> 2) * 8 + (r & 3);
                    if (m < M) static_cast<int32_t*>(p.out)[((int64_t)e * M + m) * N + n] = acc[tm][q][r];
                }
            }
        }
        return;
    } else {
        // bf16 results go to an LDS copy of the output tile, then out with coalesced 16-byte stores.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();  // every wavefront is done with the ring
        int8_t* stage = smem;
        float bias[2] = {0.0f, 0.0f};
        if constexpr (EPI == Epi::kBf16) {
            if (p.bias) {
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    int n = nblk[q] * 32 + col;
                    n = n < N ? n : N - 1;
                    bias[q] = bf16_to_float(p.bias[n]);
                }
            }
        }
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = tm * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);  // row within the tile
                const float sr = srow_lds[lr];
                if constexpr (EPI == Epi::kBf16) {
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        float v = (float)acc[tm][q][r];
                        v = v * sr;
                        v = v * csc[q];
                        if (p.bias) v = v + bias[q];
                        const int lc = (2 * wave + q) * 32 + col;  // column within the tile
                        *reinterpret_cast<uint16_t*>(stage + lr * OUT_STRIDE + lc * 2) = (uint16_t)float_to_bf16(v);
                    }
                } else {
                    float g = (float)acc[tm][0][r];
                    g = g * sr;
                    g = g * csc[0];
                    float u = (float)acc[tm][1][r];
                    u = u * sr;
                    u = u * csc[1];
                    const float gb = bf16_to_float(float_to_bf16(g));
                    const float ub = bf16_to_float(float_to_bf16(u));
                    const float a = silu_fixed(gb) * ub;
                    const int lc = wave * 32 + col;
                    *reinterpret_cast<uint16_t*>(stage + lr * OUT_STRIDE + lc * 2) = (uint16_t)float_to_bf16(a);
                }
            }
        }
        __syncthreads();
        const int ldo = (EPI == Epi::kSwiGLU) ? I : N;                  // output row length (elements)
        const int col0 = (EPI == Epi::kSwiGLU) ? nt * (kBN / 2) : nt * kBN;
        const int ncols = (ldo - col0) < OUT_COLS ? (ldo - col0) : OUT_COLS;
        constexpr int CPR = OUT_COLS / 8;                                // 16-byte chunks per tile row
        uint16_t* out = static_cast<uint16_t*>(p.out);
        if ((ldo & 7) == 0) {
            for (int c = tid; c < BM * CPR; c += kThreads) {
                const int lr = c / CPR, ch = c % CPR;
                const int m = mt * BM + lr;
                if (m >= M || ch * 8 >= ncols) continue;
                const uint4 v = *reinterpret_cast<const uint4*>(stage + lr * OUT_STRIDE + ch * 16);
                *reinterpret_cast<uint4*>(out + ((int64_t)e * M + m) * ldo + col0 + ch * 8) = v;
            }
        } else {
            for (int c = tid; c < BM * OUT_COLS; c += kThreads) {
                const int lr = c / OUT_COLS, cc = c % OUT_COLS;
                const int m = mt * BM + lr;
                if (m >= M || cc >= ncols) continue;
                out[((int64_t)e * M + m) * ldo + col0 + cc] =
                    *reinterpret_cast<const uint16_t*>(stage + lr * OUT_STRIDE + cc * 2);
            }
        }
    }
}

template <int BM, int S, int OCC, Epi EPI, int WBITS, bool TILED>
hipError_t launch_cfg(const GemmProblem& p, hipStream_t st) {
    const int tiles_m = (p.M + BM - 1) / BM;
    const int tiles_n = (EPI == Epi::kSwiGLU) ? (p.N / 2 + kBN / 2 - 1) / (kBN / 2) : (p.N + kBN - 1) / kBN;
    constexpr int stage = BM * kBK + 4 * ((WBITS == 8) ? 4 : 2) * 1024;
    constexpr int out_stride = ((EPI == Epi::kSwiGLU) ? kBN / 2 : kBN) * 2 + 16;
    constexpr int ring = (S * stage > BM * out_stride) ? S * stage : BM * out_stride;
    const size_t lds = (size_t)ring + BM * sizeof(float);
    auto kern = grouped_gemm_kernel<BM, S, OCC, EPI, WBITS, TILED>;
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess) return attr;
    const int64_t total = (int64_t)p.E * tiles_m * tiles_n;
    if (total <= 0) return hipSuccess;
    if (total > 0x7fffffff) return hipErrorInvalidValue;
    kern<<<dim3((unsigned)total), dim3(kThreads), lds, st>>>(p, tiles_m, tiles_n);
    return hipGetLastError();
}

template <Epi EPI, int WBITS, bool TILED>
hipError_t launch_epi(const GemmProblem& p, hipStream_t st) {
    // Two workgroups per CU in both shapes (LDS: 60 KiB and 72.5 KiB per workgroup).
    if (p.M <= 64) return launch_cfg<64, 3, 2, EPI, WBITS, TILED>(p, st);
    return launch_cfg<128, 3, 2, EPI, WBITS, TILED>(p, st);
}

}  // namespace

hipError_t launch_grouped_gemm(const GemmProblem& p, hipStream_t st) {
    if (!p.b_tiled) {
        if (p.wbits != 8 || p.epi != Epi::kI32) return hipErrorInvalidValue;
        return launch_epi<Epi::kI32, 8, false>(p, st);
    }
    if (p.wbits == 4) {
        switch (p.epi) {
            case Epi::kBf16: return launch_epi<Epi::kBf16, 4, true>(p, st);
            case Epi::kSwiGLU: return launch_epi<Epi::kSwiGLU, 4, true>(p, st);
            default: return hipErrorInvalidValue;
        }
    }
    switch (p.epi) {
        case Epi::kBf16: return launch_epi<Epi::kBf16, 8, true>(p, st);
        case Epi::kSwiGLU: return launch_epi<Epi::kSwiGLU, 8, true>(p, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace crk
