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
// Work decomposition.  A tile is (expert e, N-tile of 256 weight rows, M-block of BM <= 256 rows).  For the
// MoE one M-block holds all C <= 256 slots of an expert, so every weight byte is streamed from HBM exactly
// once per layer.  The kernel is persistent: one workgroup of 8 wavefronts per CU (the LDS budget admits one)
// walks a sequence of tiles.  The tiles are split into 8 contiguous ranges, one per XCD (workgroup g runs on
// XCD g % 8), and the workgroups of an XCD take the tiles of its range round robin, so at any time they work
// on neighbouring N-tiles of the same experts and share the gathered activation rows in that XCD's L2.
//
// Wavefront w computes rows [(w / 4) * BM/2, +BM/2) of the tile against two 32-row weight blocks picked by
// w % 4 (for SwiGLU the gate block and the up block of the same 32 output columns, so the epilogue pairs
// them in registers).
//
// Main loop: K-steps of 64 bytes (two 32-deep MFMA slices), one pipeline running across all tiles of the
// workgroup, so the loads of the next tile's first stages overlap the current tile's last steps and its
// epilogue.
//   * Every operand moves global -> LDS with gfx950's global_load_lds (no register staging): the weights, the
//     gathered activation rows, the per-tile row indices, row scales and column scales.
//   * Weights are stored MFMA-tiled: each (32-row block, K-block) tile is 1 KiB in B-operand lane order, so a
//     DMA is one coalesced 16-byte load per lane (non-temporal: each byte is used once) and the fragment read
//     is one ds_read_b128.  Activation rows are 64 bytes per stage with the 16-byte chunks XOR-swizzled by
//     (row / 4) % 4, so the fragment reads are free of bank conflicts.
//   * Load roles: wavefronts 0-3 issue the weight DMAs into an SB-deep ring, wavefronts 4-7 the activation
//     DMAs into an SA-deep ring.  A wavefront's vector memory operations complete in issue order, so waiting
//     for vmcnt <= X, where X counts operations it issued after a stage, proves that the stage has landed.
//     Every wavefront counts the operations it issues (DMAs, and the epilogue's buffer stores, which are
//     always issued and drop out-of-range lanes in hardware) and waits with that exact X, so each ring keeps
//     its full depth in flight through tile boundaries and epilogues.  Operations left out of the count can
//     only make a wait stricter.
//   * Half steps: the MFMAs of a stage's first slice run while its second slice is read from LDS; then one
//     workgroup barrier publishes the next stage (and frees the slots of this one for the loads S stages
//     ahead), and the MFMAs of the second slice run while the first slice of the next stage is read.  The
//     matrix pipe never waits for a whole stage of fragment reads.
// INT32 accumulation is exact, so the result does not depend on the k order inside the MFMA.  4-bit weights
// are sign-extended to int8 in registers right before the MFMA.
#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace crk {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBK = 64;          // K bytes per pipeline stage (two MFMA slices)
constexpr int kBN = 256;         // weight rows per tile (8 blocks of 32)
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBufferFlags = 0x00020000;  // buffer resource word 3 for raw (untyped) gfx9 buffer access
constexpr int kOobOffset = 0x40000000;    // byte offset past every output range (the store is dropped)
// Cache policy of the weight DMAs: non-temporal; streaming with nt measured ~6.5 TB/s vs ~5.7 TB/s without.
constexpr int kNonTemporal = 2;

// SwiGLU gate activation silu(g) = g / (1 + E(-g)) for every bf16 bit pattern g (index = the bits), built on
// the host from the same definition.  The epilogue keeps the window of gate values with |g| in [2^-13, 2^5)
// (bf16 exponent fields 114..131, both signs: 4608 entries, 18 KiB) in LDS and evaluates E for the rest.
__device__ const uint32_t kSiluTable[65536] = {
#include "silu_table.inc"
};
constexpr uint32_t kSiluLo = 114u << 7;       // first (sign-less) bf16 pattern of the window
constexpr uint32_t kSiluSpan = 18u << 7;      // patterns per sign
constexpr int kSiluBytes = 2 * kSiluSpan * 4;

// Sign-extend the 8 nibbles of a tiled int4 word into 8 int8 bytes in k order: the low nibbles hold the first
// 4 k, the high nibbles the next 4.  Per byte, n ^ 0x88 = 0x80 + (v + 8) for the 4-bit two's complement v;
// subtracting 8 cannot borrow out of the byte, and xor 0x80 leaves v as an int8.
__device__ __forceinline__ uint2 unpack_nibbles(uint32_t w) {
    const uint32_t lo = w & 0x0f0f0f0fu, hi = (w >> 4) & 0x0f0f0f0fu;
    uint2 r;
    r.x = ((lo ^ 0x88888888u) - 0x08080808u) ^ 0x80808080u;
    r.y = ((hi ^ 0x88888888u) - 0x08080808u) ^ 0x80808080u;
    return r;
}

// LDS byte offset of 16-byte chunk c (0..3) of 64-byte row r: activation stages and epilogue staging blocks.
__device__ __forceinline__ int swz_offset(int r, int c) { return r * kBK + ((c ^ ((r >> 2) & 3)) << 4); }

// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt[5:4] in bits 15:14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }


// vmcnt(x) for a wave-uniform x (binary search over the immediate forms; scalar branches only).
template <int L, int H>
__device__ __forceinline__ void wait_vmcnt_range(int x) {
    if constexpr (L == H) {
        wait_vmcnt<L>();
    } else {
        constexpr int Mid = (L + H) / 2;
        if (x <= Mid)
            wait_vmcnt_range<L, Mid>(x);
        else
            wait_vmcnt_range<Mid + 1, H>(x);
    }
}
__device__ __forceinline__ void wait_vmcnt_dyn(int x) {
    x = x < 0 ? 0 : (x > 63 ? 63 : x);  // a smaller count is a stricter wait
    wait_vmcnt_range<0, 63>(x);
}

template <int BM, int SB, int SA, Epi EPI, int WBITS, bool TILED>
struct GemmCfg {
    static constexpr int TM = BM / 64;                 // 32-row blocks per wavefront (BM/2 rows)
    static constexpr int NBT = (WBITS == 8) ? 16 : 8;  // 1 KiB weight tiles per stage
    static constexpr int NBW = NBT / 4;                // weight DMAs per loader wavefront per stage
    static constexpr int A_BYTES = BM * kBK;
    static constexpr int NAW = A_BYTES / 4096;         // activation DMAs per loader wavefront per stage
    static constexpr int B_BYTES = NBT * 1024;
    static constexpr int B_RING = SB * B_BYTES;
    static constexpr int A_RING = SA * A_BYTES;
    static constexpr int SMAX = SB > SA ? SB : SA;
    // A tile's scales are loaded with its first stage, up to SMAX stages before the tile starts, and read by
    // its epilogue: SMAX + 1 slots keep them until then for any K.
    static constexpr int NSC = SMAX + 1;
    static constexpr int CSC_OFF = B_RING + A_RING;           // NSC slots of 256 column scales
    static constexpr int SROW_OFF = CSC_OFF + NSC * kBN * 4;  // NSC slots of BM row scales
    static constexpr int ROWS_OFF = SROW_OFF + NSC * BM * 4;  // 2 slots of BM gathered row indices
    static constexpr int SILU_OFF = ROWS_OFF + 2 * BM * 4;   // SwiGLU: the gate activation window
    static constexpr int LDS = SILU_OFF + (EPI == Epi::kSwiGLU ? kSiluBytes : 0);
    static_assert(BM == 64 || BM == 128 || BM == 256, "tile rows");
    static_assert(NAW >= 1 && NAW * 4096 == A_BYTES, "activation stage / loader mismatch");
    static_assert(SB >= 3 && SA >= 3, "ring depth");
    static_assert(TILED || WBITS == 8, "4-bit weights are only stored tiled");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <int BM, int SB, int SA, Epi EPI, int WBITS, bool TILED>
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_kernel(const GemmProblem p, int tiles_m, int tiles_n) {
    using Cfg = GemmCfg<BM, SB, SA, EPI, WBITS, TILED>;
    constexpr int TM = Cfg::TM, NBW = Cfg::NBW, NAW = Cfg::NAW;
    constexpr int A_BYTES = Cfg::A_BYTES, B_BYTES = Cfg::B_BYTES;
    constexpr int HALF = BM / 2;
    constexpr bool kScales = EPI != Epi::kI32;

    extern __shared__ __attribute__((aligned(16))) int8_t smem[];
    int8_t* const b_ring = smem;
    int8_t* const a_ring = smem + Cfg::B_RING;
    float* const csc_lds = reinterpret_cast<float*>(smem + Cfg::CSC_OFF);
    float* const srow_lds = reinterpret_cast<float*>(smem + Cfg::SROW_OFF);
    int32_t* const rows_lds = reinterpret_cast<int32_t*>(smem + Cfg::ROWS_OFF);
    float* const silu_lds = reinterpret_cast<float*>(smem + Cfg::SILU_OFF);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: role branches stay scalar
    const int mh = wave >> 2;  // M-half computed by this wavefront
    const int nq = wave & 3;   // weight-block pair computed by this wavefront; DMA share of the weight loaders
    const bool b_loader = wave < 4;
    const int aw = wave - 4;   // activation loader index (0..3)
    const int M = p.M, N = p.N, K = p.K;
    const int I = N >> 1;
    const int nk = (K + kBK - 1) / kBK;
    const int NBk = (N + 31) >> 5;  // row blocks per expert
    // Gathered row indices reach the activation loaders through LDS when the index DMA of tile i+1, issued
    // with the first stage of tile i, is published by the time tile i+1's loads are issued (nk >= SA).
    const bool rows_via_lds = p.a_rows != nullptr && nk >= SA;

    // ---- this workgroup's tiles: XCD x owns the contiguous range [xs, xs + xn); its workgroups interleave ----
    const int total = p.E * tiles_m * tiles_n;
    const int G = (int)gridDim.x;
    const int xcd = (int)blockIdx.x % 8, local = (int)blockIdx.x / 8;
    const int nwg_x = (G - xcd + 7) / 8;
    const int base = total / 8, extra = total % 8;
    const int xs = xcd * base + (xcd < extra ? xcd : extra);
    const int xn = base + (xcd < extra ? 1 : 0);
    const int my_tiles = local < xn ? (xn - local + nwg_x - 1) / nwg_x : 0;
    if (my_tiles == 0) return;  // workgroup-uniform
    const int total_stages = my_tiles * nk;
    // M-blocks fastest, then N-tiles, then experts
    auto decode = [&](int i, int& e, int& nt, int& mt) {
        const int t = xs + local + i * nwg_x;
        mt = t % tiles_m;
        nt = (t / tiles_m) % tiles_n;
        e = t / (tiles_m * tiles_n);
    };
    // weight row block held by stage block j (0..7) of N-tile nt; SwiGLU: blocks 0..3 are the gate blocks of
    // the tile's 4 output column blocks, blocks 4..7 their up blocks
    auto wblk = [&](int j, int nt) -> int {
        if constexpr (EPI == Epi::kSwiGLU) {
            const int jb = nt * 4 + (j & 3);
            return j < 4 ? jb : (I >> 5) + jb;
        } else {
            return nt * 8 + j;
        }
    };
    const int my_blk0 = (EPI == Epi::kSwiGLU) ? nq : 2 * nq;
    const int my_blk1 = (EPI == Epi::kSwiGLU) ? nq + 4 : 2 * nq + 1;
    auto slot_index = [&](int e, int mt, int r) -> int64_t {
        int m = mt * BM + r;
        m = m < M ? m : M - 1;
        return (int64_t)e * M + m;
    };
    auto clamp_row = [&](int64_t arow) -> int64_t {
        return arow < 0 ? 0 : (arow < p.a_nrows ? arow : p.a_nrows - 1);
    };

    // ---- count of vector memory operations this wavefront issued, and the count after each pending stage ----
    int ops = 0;
    int hist[Cfg::SMAX];
    const int S = b_loader ? SB : SA;  // this wavefront's ring depth

    // ---- loader state for the tile whose stages are being issued ----
    // weight loaders: DMA j covers stage tile t = nq * NBW + j: (block, slice) = (t / 2, t % 2) for int8,
    // block t for int4 (both slices in one tile)
    // activation loaders: DMA j fills LDS chunk slot s = (4 j + aw) * 64 + lane
    constexpr int NLMAX = NBW > NAW ? NBW : NAW;
    const int8_t* src[NLMAX];
    int src_off[NLMAX];
    int ld_tile = -1;
    auto set_loader_tile = [&](int i) {
        int e, nt, mt;
        decode(i, e, nt, mt);
        if (b_loader) {
#pragma unroll
            for (int j = 0; j < NLMAX; ++j) {
                src[j] = p.A;
                src_off[j] = 0;
                if (j >= NBW) continue;
                const int t = nq * NBW + j;
                const int blk = (WBITS == 8) ? t / 2 : t;
                int nb = wblk(blk, nt);
                nb = nb < NBk ? nb : NBk - 1;  // out-of-range blocks compute unused columns
                if constexpr (TILED) {
                    const int64_t expert_bytes = (int64_t)NBk * 32 * K * WBITS / 8;
                    src[j] = static_cast<const int8_t*>(p.B) + e * expert_bytes + (int64_t)nb * 32 * K * WBITS / 8 +
                             lane * 16 + ((WBITS == 8) ? (t & 1) * 1024 : 0);
                } else {
                    int n = nb * 32 + (lane & 31);
                    n = n < N ? n : N - 1;
                    src[j] = static_cast<const int8_t*>(p.B) + ((int64_t)e * N + n) * K + (lane >> 5) * 16;
                    src_off[j] = (t & 1) * 32;  // slice
                }
            }
            if constexpr (kScales) {
                // column scales of the tile; lane l of weight loader w fetches column (2w + l / 32) * 32 + l % 32
                const int j = 2 * nq + (lane >> 5);
                int n = wblk(j, nt) * 32 + (lane & 31);
                n = n < N ? n : N - 1;
                __builtin_amdgcn_global_load_lds(static_cast<const void*>(p.b_scale + (int64_t)e * N + n),
                                                 (lds_void*)(csc_lds + (i % Cfg::NSC) * kBN + nq * 64), 4, 0, 0);
                ++ops;
            }
        } else {
            const int32_t* rows_cur = rows_lds + (i & 1) * BM;
            auto arow_of = [&](int r) -> int64_t {
                if (p.a_rows == nullptr) return slot_index(e, mt, r);
                if (rows_via_lds && i > 0) return clamp_row(rows_cur[r]);
                return clamp_row(p.a_rows[slot_index(e, mt, r)]);  // first tile, or K too short to prefetch
            };
#pragma unroll
            for (int j = 0; j < NLMAX; ++j) {
                src[j] = p.A;
                src_off[j] = 0;
                if (j >= NAW) continue;
                const int slot = (4 * j + aw) * 64 + lane;
                const int r = slot >> 2;                    // tile row
                const int c = (slot & 3) ^ ((r >> 2) & 3);  // logical 16-byte chunk held by that slot
                src[j] = p.A + arow_of(r) * K;
                src_off[j] = c * 16;
            }
            if (aw * 64 < BM) {
                const int r = aw * 64 + lane;
                if constexpr (kScales) {
                    __builtin_amdgcn_global_load_lds(static_cast<const void*>(p.a_scale + arow_of(r)),
                                                     (lds_void*)(srow_lds + (i % Cfg::NSC) * BM + aw * 64), 4, 0, 0);
                    ++ops;
                }
                if (rows_via_lds && i + 1 < my_tiles) {
                    // raw row indices of the next tile (clamped where they are read)
                    int e1, nt1, mt1;
                    decode(i + 1, e1, nt1, mt1);
                    __builtin_amdgcn_global_load_lds(static_cast<const void*>(p.a_rows + slot_index(e1, mt1, r)),
                                                     (lds_void*)(rows_lds + ((i + 1) & 1) * BM + aw * 64), 4, 0, 0);
                    ++ops;
                }
            }
        }
        ld_tile = i;
    };

    // Loads of stage (tile i, K-step kt) into ring slot `slot` of this wavefront's role.
    auto issue = [&](int i, int kt, int slot) {
        if (i != ld_tile) set_loader_tile(i);
        if (b_loader) {
            int8_t* st = b_ring + slot * B_BYTES;
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
                const int t = nq * NBW + j;
                if constexpr (TILED) {
                    const int64_t off = (WBITS == 8) ? (int64_t)(2 * kt) * 1024 : (int64_t)kt * 1024;
                    __builtin_amdgcn_global_load_lds(static_cast<const void*>(src[j] + off), (lds_void*)(st + t * 1024),
                                                     16, 0, kNonTemporal);
                    ++ops;
                } else {
                    // row-major weights (plain GEMM) go through registers, zero past K; not counted: the
                    // ds_write is waited for (lgkmcnt) before the barrier that publishes the stage
                    const int k = kt * kBK + src_off[j] + (lane >> 5) * 16;
                    const v4i v = (k + 16 <= K) ? *reinterpret_cast<const v4i*>(src[j] + kt * kBK + src_off[j])
                                                : v4i{0, 0, 0, 0};
                    *reinterpret_cast<v4i*>(st + t * 1024 + lane * 16) = v;
                }
            }
        } else {
            int8_t* st = a_ring + slot * A_BYTES;
#pragma unroll
            for (int j = 0; j < NAW; ++j) {
                int k = kt * kBK + src_off[j];
                k = k <= K - 16 ? k : K - 16;  // past K the weights are zero, any in-bounds bytes do
                __builtin_amdgcn_global_load_lds(static_cast<const void*>(src[j] + k),
                                                 (lds_void*)(st + (4 * j + aw) * 1024), 16, 0, 0);
                ++ops;
            }
        }
    };

    v16i acc[TM][2];
    auto clear_acc = [&]() {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][q][r] = 0;
    };

    // Fragments of one 32-deep slice s of the stage in ring slots (as, bs): this wavefront's two weight blocks
    // and its TM activation row blocks.
    auto read_slice = [&](int as, int bs, int s, v4i (&bf)[2], v4i (&af)[TM]) {
        const int8_t* As = a_ring + as * A_BYTES;
        const int8_t* Bs = b_ring + bs * B_BYTES + lane * 16;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int blk = q ? my_blk1 : my_blk0;
            if constexpr (WBITS == 8) {
                bf[q] = *reinterpret_cast<const v4i*>(Bs + (2 * blk + s) * 1024);
            } else {
                const uint2 w = *reinterpret_cast<const uint2*>(Bs + blk * 1024 + 8 * s);
                const uint2 u0 = unpack_nibbles(w.x), u1 = unpack_nibbles(w.y);
                bf[q] = v4i{(int)u0.x, (int)u0.y, (int)u1.x, (int)u1.y};
            }
        }
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
            af[tm] = *reinterpret_cast<const v4i*>(As + swz_offset(mh * HALF + tm * 32 + (lane & 31), 2 * s + (lane >> 5)));
    };
    auto mfma_slice = [&](const v4i (&bf)[2], const v4i (&af)[TM]) {
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
            for (int q = 0; q < 2; ++q)
                acc[tm][q] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[q], af[tm], acc[tm][q], 0, 0, 0);
    };
    // Scheduling of a half step: the 2 * TM MFMAs of one slice alternate with the 2 + TM fragment reads of the
    // next slice, so the matrix pipe is fed while the LDS delivers.
    auto interleave = [&]() {
        constexpr int kMfma = 2 * TM, kReads = 2 + TM, kPairs = kMfma < kReads ? kMfma : kReads;
#pragma unroll
        for (int k = 0; k < kPairs; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        }
        if constexpr (kMfma > kPairs) __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kPairs, 0);
        if constexpr (kReads > kPairs) __builtin_amdgcn_sched_group_barrier(0x100, kReads - kPairs, 0);
    };

    // Epilogue of tile i.  The weights are the MFMA's first operand, so lane l holds activation row l % 32 of
    // each 32 x 32 block and, in register 4 j + i, weight row (output column) 8 j + 4 (l / 32) + i: each lane
    // owns runs of 4 consecutive output columns, and the gate and up values of one output sit in the same lane.
    auto epilogue = [&](int i) {
        int e, nt, mt;
        decode(i, e, nt, mt);
        const int h = lane >> 5;
        if constexpr (EPI == Epi::kI32) {
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) {
                const int m = mt * BM + mh * HALF + tm * 32 + (lane & 31);
                if (m >= M) continue;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int n = wblk(q ? my_blk1 : my_blk0, nt) * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                        if (n < N) static_cast<int32_t*>(p.out)[((int64_t)e * M + m) * N + n] = acc[tm][q][r];
                    }
                }
            }
        } else {
            const float* srow = srow_lds + (i % Cfg::NSC) * BM + mh * HALF;
            const float* csc = csc_lds + (i % Cfg::NSC) * kBN;
            const int ldo = (EPI == Epi::kSwiGLU) ? I : N;  // output row length (elements)
            const int rows_valid = (M - mt * BM) < BM ? (M - mt * BM) : BM;
            const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
                static_cast<uint16_t*>(p.out) + ((int64_t)e * M + mt * BM) * ldo, 0, rows_valid * ldo * 2, kBufferFlags);
            // column scales (and bias) of weight block q of this wavefront, per run j: 4 consecutive columns
            auto load_cs = [&](int q, float (&c)[16]) {
                const int blk = q ? my_blk1 : my_blk0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const v4i c4 = *reinterpret_cast<const v4i*>(csc + blk * 32 + 8 * j + 4 * h);
#pragma unroll
                    for (int x = 0; x < 4; ++x) c[4 * j + x] = __int_as_float(c4[x]);
                }
            };
            auto load_bias = [&](int q, float (&b)[16]) {
                const int blk = q ? my_blk1 : my_blk0;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    int n = wblk(blk, nt) * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                    n = n < N ? n : N - 1;
                    b[r] = bf16_to_float(p.bias[n]);
                }
            };
            // One 32 x 32 output block: v[j][x] is this lane's row row0 + l % 32, column colb + 8 j + 4 (l / 32) + x.
            // Packed to bf16, one swap between the lane halves per pair of runs gives lane l < 32 8-column chunk
            // j0 of row l and lane l + 32 chunk j1 of the same row (A: chunks 0, 1; B: chunks 2, 3).  One swap
            // between 16-lane rows then regroups A and B into X (rows 0-15) and Y (rows 16-31), where the four
            // lanes l % 16 + {0, 16, 32, 48} hold chunks {0, 2, 1, 3} of row l % 16: each 16-byte store writes
            // 64 contiguous bytes of 16 rows, half the write requests of 32-byte pieces.  Rows that are not
            // 8-aligned fall back to element stores.  Every store is issued; out-of-range ones are dropped by
            // the buffer range.
            const bool vec = (ldo & 7) == 0;
            // pk[j][k]: columns 8 j + 4 (l / 32) + 2 k and + 1, packed to bf16
            auto store_block = [&](int row0, int colb, const uint32_t (&pk)[4][2]) {
                if (vec) {
                    const auto a0 = __builtin_amdgcn_permlane32_swap(pk[0][0], pk[1][0], false, false);
                    const auto a1 = __builtin_amdgcn_permlane32_swap(pk[0][1], pk[1][1], false, false);
                    const auto b0 = __builtin_amdgcn_permlane32_swap(pk[2][0], pk[3][0], false, false);
                    const auto b1 = __builtin_amdgcn_permlane32_swap(pk[2][1], pk[3][1], false, false);
                    const uint32_t A[4] = {a0[0], a1[0], a0[1], a1[1]};
                    const uint32_t B[4] = {b0[0], b1[0], b0[1], b1[1]};
                    uint32_t X[4], Y[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const auto u = __builtin_amdgcn_permlane16_swap(A[k], B[k], false, false);
                        X[k] = u[0];
                        Y[k] = u[1];
                    }
                    const int col = colb + 8 * (((lane >> 4) & 1) * 2 + ((lane >> 5) & 1));  // chunk {0, 2, 1, 3}
                    const int r = row0 + (lane & 15);
                    const int offx = col < ldo ? (r * ldo + col) * 2 : kOobOffset;
                    const int offy = col < ldo ? ((r + 16) * ldo + col) * 2 : kOobOffset;
                    __builtin_amdgcn_raw_buffer_store_b128(v4i{(int)X[0], (int)X[1], (int)X[2], (int)X[3]}, orsrc, offx,
                                                           0, 0);
                    __builtin_amdgcn_raw_buffer_store_b128(v4i{(int)Y[0], (int)Y[1], (int)Y[2], (int)Y[3]}, orsrc, offy,
                                                           0, 0);
                    ops += 2;
                } else {
                    const int r = row0 + (lane & 31);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int col = colb + 8 * j + 4 * h;
#pragma unroll
                        for (int x = 0; x < 4; ++x) {
                            const int off = col + x < ldo ? (r * ldo + col + x) * 2 : kOobOffset;
                            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(pk[j][x >> 1] >> (16 * (x & 1))), orsrc, off,
                                                                  0, 0);
                        }
                    }
                    ops += 16;
                }
            };
            if constexpr (EPI == Epi::kBf16) {
                // weight block outer, so only one block's scales and bias are live
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int colb = wblk(q ? my_blk1 : my_blk0, nt) * 32;
                    auto rows_out = [&](auto with_bias, const float (&bias)[16]) {
#pragma unroll
                        for (int tm = 0; tm < TM; ++tm) {
                            const float sx = srow[tm * 32 + (lane & 31)];
                            // the block's column scales, read again for each row block: fewer live registers
                            float cs[16];
                            load_cs(q, cs);
                            uint32_t pk[4][2];
#pragma unroll
                            for (int j = 0; j < 4; ++j)
#pragma unroll
                                for (int k = 0; k < 2; ++k) {
                                    float t[2];
#pragma unroll
                                    for (int y = 0; y < 2; ++y) {
                                        const int r = 4 * j + 2 * k + y;
                                        t[y] = (float)acc[tm][q][r];
                                        t[y] = t[y] * sx;
                                        t[y] = t[y] * cs[r];
                                        if constexpr (decltype(with_bias)::value) t[y] = t[y] + bias[r];
                                    }
                                    pk[j][k] = pack_bf16x2(t[0], t[1]);
                                }
                            store_block(mh * HALF + tm * 32, colb, pk);
                        }
                    };
                    if (p.bias) {  // uniform: one copy of the loop per case
                        float bias[16];
                        load_bias(q, bias);
                        rows_out(std::true_type{}, bias);
                    } else {
                        float unused[16];
                        rows_out(std::false_type{}, unused);
                    }
                }
            } else {
                float cg[16], cu[16];
                load_cs(0, cg);
                load_cs(1, cu);
                const int colb = wblk(my_blk0, nt) * 32;  // gate block index = output column block
#pragma unroll
                for (int tm = 0; tm < TM; ++tm) {
                    const float sx = srow[tm * 32 + (lane & 31)];
                    // gate and up rounded to bf16 in one conversion; the gate's bits index the activation table
                    uint32_t gu[16];
                    float sg[16];
                    bool out_of_window = false;
                    // window entry 2 (m - kSiluLo) + sign holds the gate with magnitude pattern m
                    const float* const silu_win = silu_lds - 2 * kSiluLo;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float gt = (float)acc[tm][0][r];
                        gt = gt * sx;
                        gt = gt * cg[r];
                        float up = (float)acc[tm][1][r];
                        up = up * sx;
                        up = up * cu[r];
                        gu[r] = pack_bf16x2(gt, up);
                        // magnitude pattern clamped into the window (one med3); a clamped value is out of it
                        const uint32_t mag = gu[r] & 0x7fffu;
                        const uint32_t mc = min(max(mag, kSiluLo), kSiluLo + kSiluSpan - 1u);
                        out_of_window |= mag != mc;
                        const uint32_t sgn = __builtin_amdgcn_ubfe(gu[r], 15, 1);
                        sg[r] = silu_win[(mc << 1) + sgn];
                    }
                    if (__builtin_expect(__ballot(out_of_window) != 0, 0)) {  // wave-uniform
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            if ((gu[r] & 0x7fffu) - kSiluLo >= kSiluSpan) sg[r] = silu_fixed(__uint_as_float(gu[r] << 16));
                    }
                    uint32_t pk[4][2];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int k = 0; k < 2; ++k) {
                            const int r = 4 * j + 2 * k;
                            pk[j][k] = pack_bf16x2(sg[r] * __uint_as_float(gu[r] & 0xffff0000u),
                                                   sg[r + 1] * __uint_as_float(gu[r + 1] & 0xffff0000u));
                        }
                    store_block(mh * HALF + tm * 32, colb, pk);
                }
            }
        }
    };

    // ---- the pipeline ----
    // Stage g is consumed in two half steps.  Half step A: MFMAs of slice 0 while slice 1 is read from LDS.
    // Then the wavefront waits for its own loads of stage g+1 and for its LDS reads, and the workgroup barrier
    // publishes stage g+1 and frees the slots of stage g, which take the loads of stage g+S.  Half step B:
    // MFMAs of slice 1 while slice 0 of stage g+1 is read.  Every ring keeps S stages in flight.
    int ld_i = 0, ld_kt = 0, ld_slot = 0, ld_left = total_stages;  // next stage to issue
    auto issue_next = [&]() {
        if (ld_left <= 0) return;
        issue(ld_i, ld_kt, ld_slot);
        --ld_left;
        if (++ld_kt == nk) {
            ld_kt = 0;
            ++ld_i;
        }
        ld_slot = (ld_slot + 1 == S) ? 0 : ld_slot + 1;
    };
    // vmcnt that proves this wavefront's loads of a stage landed: x operations were issued after them.  In the
    // steady state x is the loads of S - 2 stages; otherwise the exact count goes through the general form.
    constexpr int kSteadyB = (SB - 2) * NBW;
    constexpr int kSteadyA = (SA - 2) * NAW;
    auto wait_landed = [&](int x) {
        if (b_loader && TILED && x == kSteadyB)
            wait_vmcnt<kSteadyB>();
        else if (!b_loader && x == kSteadyA)
            wait_vmcnt<kSteadyA>();
        else
            wait_vmcnt_dyn(x);
    };

    if constexpr (EPI == Epi::kSwiGLU) {
        // the activation window, published by the prologue's barrier
        for (int k = tid; k < (int)(2 * kSiluSpan); k += kThreads) {
            const uint32_t pat = (k & 1 ? 0x8000u : 0u) + kSiluLo + (uint32_t)(k >> 1);
            silu_lds[k] = __uint_as_float(kSiluTable[pat]);
        }
    }

    // prologue: every ring slot takes a stage; hist[t] = operations issued up to the end of stage t
#pragma unroll
    for (int t = 0; t < Cfg::SMAX; ++t) {
        if (t < S) issue_next();
        hist[t] = ops;
    }
    clear_acc();
    wait_landed(ops - hist[0]);
    if constexpr (!TILED) {
        if (b_loader) wait_lgkmcnt0();  // row-major weights reach the ring through ds_write
    }
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
    for (int t = 0; t + 1 < Cfg::SMAX; ++t) hist[t] = hist[t + 1];  // hist[j]: end of stage g + 1 + j

    v4i bf0[2], af0[TM], bf1[2], af1[TM];
    int a_slot = 0, b_slot = 0, ci = 0, ckt = 0;
    read_slice(0, 0, 0, bf0, af0);
    for (int g = 0; g + 1 < total_stages; ++g) {
        // half step A: slice 0 of stage g with the reads of slice 1
        read_slice(a_slot, b_slot, 1, bf1, af1);
        mfma_slice(bf0, af0);
        interleave();
        wait_landed(ops - hist[0]);  // this wavefront's part of stage g + 1
        wait_lgkmcnt0();             // its reads of stage g (and any row-major ds_write)
        __builtin_amdgcn_s_barrier();
        // keeps the LDS reads of stage g + 1 below the barrier (costs an lgkmcnt wait, not a vmcnt one)
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        a_slot = (a_slot + 1 == SA) ? 0 : a_slot + 1;
        b_slot = (b_slot + 1 == SB) ? 0 : b_slot + 1;
        // half step B: slice 1 of stage g with the reads of slice 0 of stage g + 1
        read_slice(a_slot, b_slot, 0, bf0, af0);
        mfma_slice(bf1, af1);
        interleave();
#pragma unroll
        for (int t = 0; t + 1 < Cfg::SMAX; ++t) hist[t] = hist[t + 1];
        issue_next();  // stage g + S into the slots of stage g
        if (b_loader)
            hist[SB - 2] = ops;
        else
            hist[SA - 2] = ops;
        if (++ckt == nk) {
            epilogue(ci);
            clear_acc();
            ckt = 0;
            ++ci;
        }
    }
    // last stage (always the last K-step of the last tile)
    read_slice(a_slot, b_slot, 1, bf1, af1);
    mfma_slice(bf0, af0);
    mfma_slice(bf1, af1);
    epilogue(ci);
}

template <int BM, int SB, int SA, Epi EPI, int WBITS, bool TILED>
hipError_t launch_cfg(const GemmProblem& p, hipStream_t st) {
    using Cfg = GemmCfg<BM, SB, SA, EPI, WBITS, TILED>;
    const int tiles_m = (p.M + BM - 1) / BM;
    const int tiles_n = (EPI == Epi::kSwiGLU) ? (p.N / 2 + kBN / 2 - 1) / (kBN / 2) : (p.N + kBN - 1) / kBN;
    auto kern = grouped_gemm_kernel<BM, SB, SA, EPI, WBITS, TILED>;
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::LDS);
    if (attr != hipSuccess) return attr;
    const int64_t total = (int64_t)p.E * tiles_m * tiles_n;
    if (total <= 0) return hipSuccess;
    if (total > 0x7fffffff) return hipErrorInvalidValue;
    const int64_t ldo = (EPI == Epi::kSwiGLU) ? p.N / 2 : p.N;
    if ((int64_t)BM * ldo * 2 >= kOobOffset) return hipErrorInvalidValue;  // an output tile must fit one range
    // compute units per device, looked up once (calls from several threads may race to store the same value)
    static std::atomic<int> ncu_cache[64];
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    int ncu = (dev >= 0 && dev < 64) ? ncu_cache[dev].load(std::memory_order_relaxed) : 0;
    if (ncu <= 0) {
        err = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
        if (err != hipSuccess) return err;
        if (ncu <= 0) return hipErrorInvalidValue;
        if (dev >= 0 && dev < 64) ncu_cache[dev].store(ncu, std::memory_order_relaxed);
    }
    const int grid = (int)(total < ncu ? total : ncu);  // one persistent workgroup per CU
    kern<<<dim3((unsigned)grid), dim3(kThreads), Cfg::LDS, st>>>(p, tiles_m, tiles_n);
    return hipGetLastError();
}

template <Epi EPI, int WBITS, bool TILED>
hipError_t launch_epi(const GemmProblem& p, hipStream_t st) {
    // Weight ring depth: what the LDS leaves after the 3-stage activation ring; 4-bit weight stages are half
    // the size, so about twice as many.
    // SwiGLU gives 18 KiB of LDS to the activation window, so its weight rings are shorter.
    constexpr bool kSw = EPI == Epi::kSwiGLU;
    if constexpr (WBITS == 8) {
        if (p.M <= 64) return launch_cfg<64, kSw ? 7 : 8, 3, EPI, WBITS, TILED>(p, st);
        if (p.M <= 128) return launch_cfg<128, kSw ? 6 : 7, 3, EPI, WBITS, TILED>(p, st);
        return launch_cfg<256, kSw ? 5 : 6, 3, EPI, WBITS, TILED>(p, st);
    } else {
        if (p.M <= 64) return launch_cfg<64, kSw ? 12 : 14, 3, EPI, WBITS, TILED>(p, st);
        if (p.M <= 128) return launch_cfg<128, kSw ? 11 : 13, 3, EPI, WBITS, TILED>(p, st);
        return launch_cfg<256, kSw ? 8 : 10, 3, EPI, WBITS, TILED>(p, st);
    }
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
