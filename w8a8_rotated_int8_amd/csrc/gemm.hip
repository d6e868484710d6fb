// Grouped INT8 x INT8 -> INT32 GEMM on gfx950 MFMA (v_mfma_i32_16x16x64_i8) with fused epilogues:
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
// Main loop: K-steps of 64 bytes (one MFMA deep), one pipeline running across all tiles of the workgroup, so
// the loads of the next tile's first stages overlap the current tile's last steps and its epilogue.
//   * Every operand moves global -> LDS with gfx950's global_load_lds (no register staging): the weights, the
//     gathered activation rows, the per-tile row indices, row scales and column scales.
//   * Weights are stored MFMA-tiled: each (32-row block, K-block) tile is 1 KiB in lane order, so a DMA is one
//     coalesced 16-byte load per lane (non-temporal: each byte is used once) and a fragment read is one
//     ds_read_b128 (ds_read_b64 and an unpack for 4-bit weights).  Activation rows are 64 bytes per stage, placed
//     within each 16-row block and chunk-swizzled so that the fragment reads are free of bank conflicts (the
//     layout is described at a_pos_of_row).
//   * Load roles: wavefronts 0-3 issue the weight DMAs into an SB-deep ring, wavefronts 4-7 the activation
//     DMAs into an SA-deep ring.  A wavefront's vector memory operations complete in issue order, so waiting
//     for vmcnt <= X, where X counts operations it issued after a stage, proves that the stage has landed.
//     Every wavefront counts the operations it issues (DMAs, and the epilogue's buffer stores, which are
//     always issued and drop out-of-range lanes in hardware) and waits with that exact X, so each ring keeps
//     its full depth in flight through tile boundaries and epilogues.  Operations left out of the count can
//     only make a wait stricter.
//   * Half steps: v_mfma_i32_16x16x64_i8 multiplies a 16-row weight fragment by a 16-token block over a whole
//     64-deep stage.  The MFMAs of the first half of a wavefront's token blocks run while the second half's
//     fragments are read from LDS; then one workgroup barrier publishes the next stage (and frees the slots of
//     this one for the loads S stages ahead), and the MFMAs of the second half run while the next stage's first
//     token half and all its weight fragments are read into a second set of registers.  The matrix pipe never
//     waits for a whole stage of fragment reads, and no weight fragment (nor its 4-bit unpacking) is read just
//     before its first use.
// INT32 accumulation is exact, so the result does not depend on the k order inside the MFMA.  4-bit weights
// are sign-extended to int8 in registers right before the MFMA.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "rotq_fast.h"

namespace crk {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
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

// Activation stage layout: each 16-row block is 1 KiB of 16 positions of 64 bytes.  Row r of the block sits at
// position a_pos_of_row(r), its 16-byte chunk c at slot c ^ ((r >> 1) & 3) of the position.  A fragment read
// (lane l: row l % 16, chunk l / 16) is served 16 lanes per LDS cycle, as two groups of 8 lanes that must each
// fall in one 128-byte half of a 256-byte bank line, on distinct 16-byte slots, and the two groups in opposite
// halves: rows 0-7 land on positions with (p & 2) == 0, rows 8-15 on (p & 2) == 2, and the four rows of a
// group that share a half and a slot column get four different chunk slots.  The DMA side keeps four
// consecutive lanes on one 64-byte row piece, so each row of a stage is still one coalesced request.
__device__ __forceinline__ int a_pos_of_row(int r) { return 4 * ((r >> 1) & 3) + 2 * (r >> 3) + (r & 1); }
__device__ __forceinline__ int a_row_of_pos(int q) { return 8 * ((q >> 1) & 1) + 2 * (q >> 2) + (q & 1); }

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

// Scheduling of NM MFMAs with NR LDS fragment reads spread evenly among them (group K of NR).
template <int NM, int NR, int K>
__device__ __forceinline__ void spread_reads() {
    constexpr int cnt = (K + 1) * NM / NR - K * NM / NR;
    if constexpr (cnt > 0) __builtin_amdgcn_sched_group_barrier(0x008, cnt, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                             // DS read
    if constexpr (K + 1 < NR) spread_reads<NM, NR, K + 1>();
}

template <int BM, int SB, int SA, Epi EPI, int WBITS, bool TILED>
struct GemmCfg {
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

// Split of `total` work items over G workgroups: XCD x (the workgroups with wg % 8 == x) owns the contiguous range
// [xs, xs + xn) of the items, and its workgroups take the items of that range round robin.  Below 8 workgroups
// each one is its own group, so that every item still has an owner.
struct XcdSplit {
    int xs, local, nwg_x, count;
    __device__ __forceinline__ XcdSplit(int total, int G, int wg) {
        const int nx = G < 8 ? G : 8;
        const int xcd = wg % nx;
        local = wg / nx;
        nwg_x = (G - xcd + nx - 1) / nx;
        const int base = total / nx, extra = total % nx;
        xs = xcd * base + (xcd < extra ? xcd : extra);
        const int xn = base + (xcd < extra ? 1 : 0);
        count = local < xn ? (xn - local + nwg_x - 1) / nwg_x : 0;
    }
    __device__ __forceinline__ int item(int i) const { return xs + local + i * nwg_x; }  // i-th item here
};

// The tiles of one grouped GEMM that the split gives this workgroup (all 8 wavefronts call it).
template <int BM, int SB, int SA, Epi EPI, int WBITS, bool TILED>
__device__ __forceinline__ void gemm_tiles(const GemmProblem& p, int tiles_m, int tiles_n, const XcdSplit split) {
    using Cfg = GemmCfg<BM, SB, SA, EPI, WBITS, TILED>;
    constexpr int NBW = Cfg::NBW, NAW = Cfg::NAW;
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

    // The thread index passes through an empty asm statement, so that where two of these bodies run in one
    // kernel nothing derived from it is computed once and kept live across both.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
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

    // ---- this workgroup's tiles ----
    const int my_tiles = split.count;
    if (my_tiles == 0) return;  // workgroup-uniform
    const int total_stages = my_tiles * nk;
    // M-blocks fastest, then N-tiles, then experts
    auto decode = [&](int i, int& e, int& nt, int& mt) {
        const int t = split.item(i);
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
                // 16-byte slot `lane` of the 1 KiB block 4 j + aw (16 tile rows): position lane / 4 holds row
                // a_row_of_pos(lane / 4) of the block, its chunk (lane & 3) ^ ((lane >> 4) & 3)
                const int r = (4 * j + aw) * 16 + a_row_of_pos(lane >> 2);  // tile row
                const int c = (lane & 3) ^ ((lane >> 4) & 3);               // logical 16-byte chunk
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

    // ---- fragments and accumulators ----
    // The wavefront's BM/2 token rows are MS blocks of 16, taken in two halves of MH blocks by the half steps.
    // Weight fragment (q, s) is rows 16 s .. 16 s + 15 of weight block q (my_blk0 / my_blk1).
    // v_mfma_i32_16x16x64_i8 takes the weights as its first operand and a 16-token block as its second; for
    // both, lane l holds row l % 16 and the 16 consecutive k of chunk l / 16 of the 64-deep step (the int32 sum
    // is exact, so only the pairing of the two operands' bytes matters), and register i of the result is the
    // product of weight row 4 (l / 16) + i with token l % 16.
    constexpr int MS = BM / 32;
    constexpr int MH = MS / 2;
    static_assert(MH >= 1, "half steps need two token blocks per wavefront");
    const int g4 = lane >> 4;  // the lane's k chunk; in the result, its 4-column group of each 16-column block
    // per-lane byte offsets inside a stage: weight fragment (q, s) of block blk is at b_lane + (2 blk) KiB +
    // 256 s (int8: two 1 KiB tiles per 64 k, the chunk's tile g4 / 2) or b_lane + blk KiB + 512 s (int4: one
    // tile, the fragment's 64 lanes on 512 contiguous bytes); token block m at a_lane + (m * 16 + the half's
    // first row) * 64 (placed and swizzled rows)
    const int b_lane = (WBITS == 8) ? ((lane & 15) + 32 * (g4 & 1)) * 16 + 1024 * (g4 >> 1) : lane * 8;
    const int a_lane = a_pos_of_row(lane & 15) * kBK + ((g4 ^ ((lane >> 1) & 3)) << 4);

    v4i acc[MS][2][2];
    auto clear_acc = [&]() {
#pragma unroll
        for (int m = 0; m < MS; ++m)
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int s = 0; s < 2; ++s) acc[m][q][s] = v4i{0, 0, 0, 0};
    };
    auto read_b = [&](int bs, int q, int s) -> v4i {
        const int blk = q ? my_blk1 : my_blk0;
        const int8_t* p = b_ring + bs * B_BYTES + b_lane + (WBITS == 8 ? 256 : 512) * s;
        if constexpr (WBITS == 8) {
            return *reinterpret_cast<const v4i*>(p + 2048 * blk);
        } else {
            const uint2 w = *reinterpret_cast<const uint2*>(p + 1024 * blk);
            const uint2 u0 = unpack_nibbles(w.x), u1 = unpack_nibbles(w.y);
            return v4i{(int)u0.x, (int)u0.y, (int)u1.x, (int)u1.y};
        }
    };
    auto read_a = [&](int as, int m) -> v4i {
        return *reinterpret_cast<const v4i*>(a_ring + as * A_BYTES + a_lane + (mh * HALF + 16 * m) * kBK);
    };
    // MFMAs of weight fragments bq[0..1] (block q) against the MH token blocks af, accumulating into blocks m0..
    auto mfma_q = [&](int m0, int q, const v4i (&bq)[2], const v4i (&af)[MH]) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int m = 0; m < MH; ++m)
                acc[m0 + m][q][s] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bq[s], af[m], acc[m0 + m][q][s], 0, 0, 0);
    };
    // nm MFMAs and nr fragment reads, the reads spread evenly among the MFMAs
    auto interleave = [&](auto nm_c, auto nr_c) {
        constexpr int nm = decltype(nm_c)::value, nr = decltype(nr_c)::value;
        if constexpr (nr == 0) {
            __builtin_amdgcn_sched_group_barrier(0x008, nm, 0);
        } else {
            spread_reads<nm, nr, 0>();
        }
    };

    // Epilogue of tile i.  Lane l holds, for token l % 16 of each 16-token block and each 16-column sub-block s
    // of its weight blocks, the 4 consecutive output columns 16 s + 4 g4 .. + 3; the gate and up values of one
    // output sit in the same lane and register.
    auto epilogue = [&](int i) {
        int e, nt, mt;
        decode(i, e, nt, mt);
        if constexpr (EPI == Epi::kI32) {
#pragma unroll
            for (int m = 0; m < MS; ++m) {
                const int row = mt * BM + mh * HALF + 16 * m + (lane & 15);
                if (row >= M) continue;
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int s = 0; s < 2; ++s)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int n = wblk(q ? my_blk1 : my_blk0, nt) * 32 + 16 * s + 4 * g4 + r;
                            if (n < N) static_cast<int32_t*>(p.out)[((int64_t)e * M + row) * N + n] = acc[m][q][s][r];
                        }
            }
        } else {
            const float* srow = srow_lds + (i % Cfg::NSC) * BM + mh * HALF;
            const float* csc = csc_lds + (i % Cfg::NSC) * kBN;
            const int ldo = (EPI == Epi::kSwiGLU) ? I : N;  // output row length (elements)
            const int rows_valid = (M - mt * BM) < BM ? (M - mt * BM) : BM;
            const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
                static_cast<uint16_t*>(p.out) + ((int64_t)e * M + mt * BM) * ldo, 0, rows_valid * ldo * 2, kBufferFlags);
            // column scales of weight block q for this lane: [s][r] = column 16 s + 4 g4 + r
            auto load_cs = [&](int q, float (&c)[2][4]) {
                const int blk = q ? my_blk1 : my_blk0;
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const v4i c4 = *reinterpret_cast<const v4i*>(csc + blk * 32 + 16 * s + 4 * g4);
#pragma unroll
                    for (int r = 0; r < 4; ++r) c[s][r] = __int_as_float(c4[r]);
                }
            };
            // One 16-token x 32-column output block: X (sub-block 0) and Y (sub-block 1) hold this lane's 4
            // columns packed to bf16 (2 words each).  A swap between the lane halves gives lane groups 0-3 the
            // values of groups (0, 1 | of X), (0, 1 | of Y) and (2, 3 | of X), (2, 3 | of Y); a swap between
            // 16-lane rows then leaves group c with columns 8 c .. 8 c + 7, so each 16-byte buffer store writes
            // 64 contiguous bytes of 16 rows.  Rows that are not 8-aligned fall back to element stores.  Every
            // store is issued; out-of-range ones are dropped by the buffer range.
            const bool vec = (ldo & 7) == 0;
            auto store_block = [&](int row0, int colb, const uint32_t (&X)[2], const uint32_t (&Y)[2]) {
                const int r = row0 + (lane & 15);
                if (vec) {
                    uint32_t R[2], S[2];
#pragma unroll
                    for (int d = 0; d < 2; ++d) {
                        const auto u = __builtin_amdgcn_permlane32_swap(X[d], Y[d], false, false);
                        const auto v = __builtin_amdgcn_permlane16_swap(u[0], u[1], false, false);
                        R[d] = v[0];
                        S[d] = v[1];
                    }
                    const int col = colb + 8 * g4;
                    const int off = col < ldo ? (r * ldo + col) * 2 : kOobOffset;
                    __builtin_amdgcn_raw_buffer_store_b128(v4i{(int)R[0], (int)R[1], (int)S[0], (int)S[1]}, orsrc, off,
                                                           0, 0);
                    ops += 1;
                } else {
#pragma unroll
                    for (int s = 0; s < 2; ++s)
#pragma unroll
                        for (int x = 0; x < 4; ++x) {
                            const int col = colb + 16 * s + 4 * g4 + x;
                            const uint32_t w = s ? Y[x >> 1] : X[x >> 1];
                            const int off = col < ldo ? (r * ldo + col) * 2 : kOobOffset;
                            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(w >> (16 * (x & 1))), orsrc, off, 0, 0);
                        }
                    ops += 8;
                }
            };
            if constexpr (EPI == Epi::kBf16) {
                // weight block outer, so only one block's scales and bias are live
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int colb = wblk(q ? my_blk1 : my_blk0, nt) * 32;
                    auto rows_out = [&](auto with_bias, const float (&bias)[2][4]) {
#pragma unroll
                        for (int m = 0; m < MS; ++m) {
                            const float sx = srow[16 * m + (lane & 15)];
                            // the block's column scales, read again for each token block: fewer live registers
                            float cs[2][4];
                            load_cs(q, cs);
                            uint32_t XY[2][2];
#pragma unroll
                            for (int s = 0; s < 2; ++s)
#pragma unroll
                                for (int k = 0; k < 2; ++k) {
                                    float t[2];
#pragma unroll
                                    for (int y = 0; y < 2; ++y) {
                                        const int r = 2 * k + y;
                                        t[y] = (float)acc[m][q][s][r];
                                        t[y] = t[y] * sx;
                                        t[y] = t[y] * cs[s][r];
                                        if constexpr (decltype(with_bias)::value) t[y] = t[y] + bias[s][r];
                                    }
                                    XY[s][k] = pack_bf16x2(t[0], t[1]);
                                }
                            store_block(mh * HALF + 16 * m, colb, XY[0], XY[1]);
                        }
                    };
                    if (p.bias) {  // uniform: one copy of the loop per case
                        float bias[2][4];
                        const int blk = q ? my_blk1 : my_blk0;
#pragma unroll
                        for (int s = 0; s < 2; ++s)
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                int n = wblk(blk, nt) * 32 + 16 * s + 4 * g4 + r;
                                n = n < N ? n : N - 1;
                                bias[s][r] = bf16_to_float(p.bias[n]);
                            }
                        rows_out(std::true_type{}, bias);
                    } else {
                        float unused[2][4];
                        rows_out(std::false_type{}, unused);
                    }
                }
            } else {
                float cg[2][4], cu[2][4];
                load_cs(0, cg);
                load_cs(1, cu);
                const int colb = wblk(my_blk0, nt) * 32;  // gate block index = output column block
                // window entry 2 (m - kSiluLo) + sign holds the gate with magnitude pattern m
                const float* const silu_win = silu_lds - 2 * kSiluLo;
#pragma unroll
                for (int m = 0; m < MS; ++m) {
                    const float sx = srow[16 * m + (lane & 15)];
                    // gate and up rounded to bf16 in one conversion; the gate's bits index the activation table
                    uint32_t gu[2][4];
                    float sg[2][4];
                    bool out_of_window = false;
#pragma unroll
                    for (int s = 0; s < 2; ++s)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            float gt = (float)acc[m][0][s][r];
                            gt = gt * sx;
                            gt = gt * cg[s][r];
                            float up = (float)acc[m][1][s][r];
                            up = up * sx;
                            up = up * cu[s][r];
                            gu[s][r] = pack_bf16x2(gt, up);
                            // magnitude pattern clamped into the window (one med3); a clamped value is out of it
                            const uint32_t mag = gu[s][r] & 0x7fffu;
                            const uint32_t mc = min(max(mag, kSiluLo), kSiluLo + kSiluSpan - 1u);
                            out_of_window |= mag != mc;
                            const uint32_t sgn = __builtin_amdgcn_ubfe(gu[s][r], 15, 1);
                            sg[s][r] = silu_win[(mc << 1) + sgn];
                        }
                    if (__builtin_expect(__ballot(out_of_window) != 0, 0)) {  // wave-uniform
#pragma unroll
                        for (int s = 0; s < 2; ++s)
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if ((gu[s][r] & 0x7fffu) - kSiluLo >= kSiluSpan)
                                    sg[s][r] = silu_fixed(__uint_as_float(gu[s][r] << 16));
                    }
                    uint32_t XY[2][2];
#pragma unroll
                    for (int s = 0; s < 2; ++s)
#pragma unroll
                        for (int k = 0; k < 2; ++k) {
                            const int r = 2 * k;
                            XY[s][k] = pack_bf16x2(sg[s][r] * __uint_as_float(gu[s][r] & 0xffff0000u),
                                                   sg[s][r + 1] * __uint_as_float(gu[s][r + 1] & 0xffff0000u));
                        }
                    store_block(mh * HALF + 16 * m, colb, XY[0], XY[1]);
                }
            }
        }
    };

    // ---- the pipeline ----
    // Stage g is consumed in two half steps over the two halves of the wavefront's token blocks.  Half step A:
    // the MFMAs of the first half while the second half's token fragments are read from LDS.  Then the
    // wavefront waits for its own loads of stage g+1 and for its LDS reads, and the workgroup barrier publishes
    // stage g+1 and frees the slots of stage g, which take the loads of stage g+S.  Half step B: the MFMAs of
    // the second half while stage g+1's first-half token fragments and all its weight fragments are read.
    // Every ring keeps S stages in flight.
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

    // weight fragments of the current stage (bc) and of the next (bn), read during half step B
    v4i bc0[2], bc1[2], bn0[2], bn1[2], alo[MH], ahi[MH];
    int a_slot = 0, b_slot = 0, ci = 0, ckt = 0;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        bc0[s] = read_b(0, 0, s);
        bc1[s] = read_b(0, 1, s);
    }
#pragma unroll
    for (int m = 0; m < MH; ++m) alo[m] = read_a(0, m);
    for (int g = 0; g + 1 < total_stages; ++g) {
        // half step A: first token half of stage g, with the reads of its second token half
#pragma unroll
        for (int m = 0; m < MH; ++m) ahi[m] = read_a(a_slot, MH + m);
        mfma_q(0, 0, bc0, alo);
        mfma_q(0, 1, bc1, alo);
        interleave(std::integral_constant<int, 4 * MH>{}, std::integral_constant<int, MH>{});
        wait_landed(ops - hist[0]);  // this wavefront's part of stage g + 1
        wait_lgkmcnt0();             // its reads of stage g (and any row-major ds_write)
        __builtin_amdgcn_s_barrier();
        // keeps the LDS reads of stage g + 1 below the barrier (costs an lgkmcnt wait, not a vmcnt one)
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        a_slot = (a_slot + 1 == SA) ? 0 : a_slot + 1;
        b_slot = (b_slot + 1 == SB) ? 0 : b_slot + 1;
        // half step B: second token half of stage g, with the reads of stage g + 1's first token half and weights
#pragma unroll
        for (int m = 0; m < MH; ++m) alo[m] = read_a(a_slot, m);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            bn0[s] = read_b(b_slot, 0, s);
            bn1[s] = read_b(b_slot, 1, s);
        }
        mfma_q(MH, 0, bc0, ahi);
        mfma_q(MH, 1, bc1, ahi);
        interleave(std::integral_constant<int, 4 * MH>{}, std::integral_constant<int, MH + 4>{});
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            bc0[s] = bn0[s];
            bc1[s] = bn1[s];
        }
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
#pragma unroll
    for (int m = 0; m < MH; ++m) ahi[m] = read_a(a_slot, MH + m);
    mfma_q(0, 0, bc0, alo);
    mfma_q(0, 1, bc1, alo);
    mfma_q(MH, 0, bc0, ahi);
    mfma_q(MH, 1, bc1, ahi);
    epilogue(ci);
}

template <int BM, int SB, int SA, Epi EPI, int WBITS, bool TILED>
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_kernel(const GemmProblem p, int tiles_m, int tiles_n) {
    gemm_tiles<BM, SB, SA, EPI, WBITS, TILED>(p, tiles_m, tiles_n,
                                              XcdSplit(p.E * tiles_m * tiles_n, (int)gridDim.x, (int)blockIdx.x));
}

// Compute units of the current device, looked up once per device (calls from several threads may race to store
// the same value).
hipError_t device_cus(int* ncu) {
    static std::atomic<int> ncu_cache[64];
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    int n = (dev >= 0 && dev < 64) ? ncu_cache[dev].load(std::memory_order_relaxed) : 0;
    if (n <= 0) {
        err = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (err != hipSuccess) return err;
        if (n <= 0) return hipErrorInvalidValue;
        if (dev >= 0 && dev < 64) ncu_cache[dev].store(n, std::memory_order_relaxed);
    }
    *ncu = n;
    return hipSuccess;
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
    int ncu = 0;
    const hipError_t err = device_cus(&ncu);
    if (err != hipSuccess) return err;
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

// ---- the expert part of the MoE layer in one persistent launch -----------------------------------------
// Three phases over the same workgroups, each split by XcdSplit, so that one expert's gate/up tiles, hidden rows
// and down tiles fall on the same XCD (and its L2) when the experts divide evenly over the XCDs:
//   1. the gate/up tiles with the SwiGLU epilogue, writing a;
//   2. rotate + quantise of a's rows in items of 8 rows, one row per wavefront; an item first waits until
//      every gate/up tile of its expert is published;
//   3. the down tiles with the bf16 epilogue; they first wait until every item of their experts is published.
// A workgroup publishes its tiles (or items) once it has finished all of them: every wavefront waits for its
// own stores, the workgroup barrier, then one thread's agent-scope release fence and one atomic add per tile
// or item on its expert's counter.  A wait is one thread polling the counter with relaxed agent-scope loads,
// an agent-scope acquire fence, and the workgroup barrier.  Phase 1 waits for nothing and the grid holds at
// most one workgroup per CU, all resident together, so every wait ends.  A poll still stops after kSpinLimit
// rounds (about a second): that could only leave wrong results, never a launch that does not finish.
constexpr int kSpinLimit = 1 << 20;

__device__ __forceinline__ void wait_count(uint32_t* c, uint32_t target) {
    for (int it = 0; it < kSpinLimit; ++it) {
        if (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) break;
        __builtin_amdgcn_s_sleep(40);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// All threads: publish the tiles or items of this workgroup, item i of the split counting once on counter
// 2 (item / per_expert) + slot.
__device__ __forceinline__ void publish(uint32_t* esync, int slot, const XcdSplit split, int per_expert) {
    wait_vmcnt<0>();
    __syncthreads();
    if (threadIdx.x == 0 && split.count > 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        for (int i = 0; i < split.count; ++i)
            __hip_atomic_fetch_add(esync + (2 * (split.item(i) / per_expert) + slot) * kEsyncStride, 1u,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

struct FusedExperts {
    GemmProblem gu, dn;
    const uint16_t* a;  // gu.out
    int8_t* qa;         // dn.A
    float* sa;          // dn.a_scale
    int group;          // rotation group of a's rows
    uint32_t* esync;    // counters (kEsyncStride apart): gate/up tiles of expert e at 2 e, its items at 2 e + 1
};

constexpr int kRowsInFlight = 8;

// This wavefront's rows of the workgroup's rotate + quantise items (row 8 (item % nrb) + wave of expert
// item / nrb), kRowsInFlight at a time: all their loads first, then each row's transform and stores.
template <int G, int R>
__device__ __forceinline__ void hidden_rows(const FusedExperts& f, const XcdSplit s2, int nrb, int wave) {
    const int C = f.gu.M, I = f.gu.N >> 1;
    for (int i0 = 0; i0 < s2.count; i0 += kRowsInFlight) {
        RotqRaw<G, R> raw[kRowsInFlight];
        int64_t row[kRowsInFlight];
        bool ok[kRowsInFlight];
#pragma unroll
        for (int b = 0; b < kRowsInFlight; ++b) {
            const int i = i0 + b;
            const int j = i < s2.count ? s2.item(i) : 0, e = j / nrb, r = (j - e * nrb) * 8 + wave;
            ok[b] = i < s2.count && r < C;  // wavefront-uniform
            row[b] = (int64_t)e * C + r;
            rotq_fast_load<G, R>(f.a, row[b], ok[b], I, 0, raw[b]);
        }
#pragma unroll
        for (int b = 0; b < kRowsInFlight; ++b)
            if (ok[b]) rotq_fast_finish<G, R, 1>(raw[b], row[b], true, I, 0, f.qa, f.sa, nullptr);
    }
}

template <int BM, int SBG, int SBD, int WBITS>
__global__ __launch_bounds__(kThreads, 2) void moe_experts_kernel(const FusedExperts f, int tiles_n_gu, int tiles_n_dn) {
    const int G = (int)gridDim.x, wg = (int)blockIdx.x;
    const int E = f.gu.E, C = f.gu.M, I = f.gu.N >> 1;
    const int tiles_m = (C + BM - 1) / BM;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);

    // phase 1: gate/up
    const int gu_per_e = tiles_m * tiles_n_gu;
    const XcdSplit s1(E * gu_per_e, G, wg);
    gemm_tiles<BM, SBG, 3, Epi::kSwiGLU, WBITS, true>(f.gu, tiles_m, tiles_n_gu, s1);
    publish(f.esync, 0, s1, gu_per_e);

    // phase 2: rotate + quantise of the hidden rows, after every gate/up tile of the experts of this workgroup's
    // items; wavefront w takes row 8 (item % nrb) + w of each item, with the loads of up to kRowsInFlight rows
    // issued before any of them is transformed (with only 8 wavefronts per CU, each would otherwise wait a
    // full memory latency per row)
    const int nrb = (C + 7) / 8;
    const XcdSplit s2(E * nrb, G, wg);
    if (threadIdx.x == 0) {
        int last = -1;
        for (int i = 0; i < s2.count; ++i) {
            const int e = s2.item(i) / nrb;  // non-decreasing in i
            if (e != last) wait_count(f.esync + (2 * e) * kEsyncStride, (uint32_t)gu_per_e);
            last = e;
        }
    }
    __syncthreads();
    const int R = I / (8 * f.group);
    if (f.group == 256)
        hidden_rows<256, 1>(f, s2, nrb, wave);
    else if (R == 1)
        hidden_rows<64, 1>(f, s2, nrb, wave);
    else if (R == 2)
        hidden_rows<64, 2>(f, s2, nrb, wave);
    else if (R == 3)
        hidden_rows<64, 3>(f, s2, nrb, wave);
    else
        hidden_rows<64, 4>(f, s2, nrb, wave);
    publish(f.esync, 1, s2, nrb);

    // phase 3: down
    const int dn_per_e = tiles_m * tiles_n_dn;
    const XcdSplit s3(E * dn_per_e, G, wg);
    if (threadIdx.x == 0) {
        int last = -1;
        for (int i = 0; i < s3.count; ++i) {
            const int e = s3.item(i) / dn_per_e;  // non-decreasing in i
            if (e != last) wait_count(f.esync + (2 * e + 1) * kEsyncStride, (uint32_t)nrb);
            last = e;
        }
    }
    __syncthreads();
    gemm_tiles<BM, SBD, 3, Epi::kBf16, WBITS, true>(f.dn, tiles_m, tiles_n_dn, s3);
}

template <int BM, int SBG, int SBD, int WBITS>
hipError_t launch_fused_cfg(const FusedExperts& f, hipStream_t st) {
    using CG = GemmCfg<BM, SBG, 3, Epi::kSwiGLU, WBITS, true>;
    using CD = GemmCfg<BM, SBD, 3, Epi::kBf16, WBITS, true>;
    constexpr int LDS = CG::LDS > CD::LDS ? CG::LDS : CD::LDS;
    auto kern = moe_experts_kernel<BM, SBG, SBD, WBITS>;
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (attr != hipSuccess) return attr;
    const int tiles_m = (f.gu.M + BM - 1) / BM;
    const int tiles_n_gu = (f.gu.N / 2 + kBN / 2 - 1) / (kBN / 2);
    const int tiles_n_dn = (f.dn.N + kBN - 1) / kBN;
    const int64_t work = (int64_t)f.gu.E * std::max<int64_t>(std::max(tiles_m * tiles_n_gu, tiles_m * tiles_n_dn),
                                                              (f.gu.M + 7) / 8);
    if (work <= 0) return hipSuccess;
    if (work > 0x7fffffff) return hipErrorInvalidValue;
    int ncu = 0;
    const hipError_t err = device_cus(&ncu);
    if (err != hipSuccess) return err;
    // no more workgroups than CUs, and each fits a CU on its own: all are resident together on an idle device
    const int grid = (int)(work < ncu ? work : ncu);
    kern<<<dim3((unsigned)grid), dim3(kThreads), LDS, st>>>(f, tiles_n_gu, tiles_n_dn);
    return hipGetLastError();
}

template <int WBITS>
hipError_t launch_fused_bits(const FusedExperts& f, hipStream_t st) {
    // the ring depths of launch_epi for the two epilogues
    if constexpr (WBITS == 8) {
        if (f.gu.M <= 64) return launch_fused_cfg<64, 7, 8, 8>(f, st);
        if (f.gu.M <= 128) return launch_fused_cfg<128, 6, 7, 8>(f, st);
        return launch_fused_cfg<256, 5, 6, 8>(f, st);
    } else {
        if (f.gu.M <= 64) return launch_fused_cfg<64, 12, 14, 4>(f, st);
        if (f.gu.M <= 128) return launch_fused_cfg<128, 11, 13, 4>(f, st);
        return launch_fused_cfg<256, 8, 10, 4>(f, st);
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

bool moe_experts_supported(const GemmProblem& gu, const GemmProblem& dn, int group) {
    const int I = gu.N / 2;
    const bool rows_ok = (group == 256 && I == 8 * 256) ||
                         (group == 64 && I % (8 * 64) == 0 && I / (8 * 64) >= 1 && I / (8 * 64) <= 4);
    const bool shapes_ok = gu.b_tiled && dn.b_tiled && gu.wbits == dn.wbits && (gu.wbits == 8 || gu.wbits == 4) &&
                           gu.epi == Epi::kSwiGLU && dn.epi == Epi::kBf16 && dn.E == gu.E && dn.M == gu.M &&
                           dn.K == I && gu.N % 2 == 0 && dn.a_rows == nullptr && gu.E >= 1 && gu.M >= 1;
    // an output tile must fit one buffer range (as in launch_cfg)
    return rows_ok && shapes_ok && (int64_t)256 * I * 2 < kOobOffset && (int64_t)256 * dn.N * 2 < kOobOffset;
}

hipError_t launch_moe_experts(const GemmProblem& gu, const GemmProblem& dn, const uint16_t* a, int8_t* qa, float* sa,
                              int group, uint32_t* esync, hipStream_t st) {
    if (!moe_experts_supported(gu, dn, group) || esync == nullptr) return hipErrorNotSupported;
    FusedExperts f{gu, dn, a, qa, sa, group, esync};
    return gu.wbits == 4 ? launch_fused_bits<4>(f, st) : launch_fused_bits<8>(f, st);
}

}  // namespace crk
