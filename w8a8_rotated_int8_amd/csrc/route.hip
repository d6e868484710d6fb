// Expert-choice routing ("MLX Nucleus-Image": each of the 64 routed experts picks its top-C tokens).
//
//  softmax_t     p[t, :] = softmax over experts in fp32 (max-subtracted, the fixed exponential, sum in
//                ascending expert order, one IEEE division per entry), written transposed as probs_t[e, t]
//                so that each expert's column is contiguous.  E <= 64: a workgroup takes a 32-token x E tile
//                of logits through LDS (coalesced 16-byte loads); eight lanes per token share the max, the
//                exponentials and the divisions, one lane keeps the sequential sum, and the probabilities
//                leave through a transposed LDS tile as 16-byte row stores.
//  select_topc   one workgroup per expert: radix select (passes of up to 11 bits, most significant first,
//                after the bits every key shares) of the C-th largest key over keys held in registers; once
//                at most 64 keys share the decided bits, one wavefront ranks those keys instead of further
//                passes.  Then one ordered compaction keeps every token above the threshold and the
//                lowest-index tokens equal to it.  The list comes out in ascending token order without a sort;
//                ties go to the lower token index by construction.
//  Slot table: slots[t, e] = position of token t in expert e's list, or -1, token-major so that one
//                coalesced load gives a token's entries for 64 experts.  The softmax launch, which runs before
//                the selection, fills the rows of its tokens with -1; the selections then write the entries of
//                the tokens they take.  build_slots does both for a given list (the stand-alone combine).
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "rotq_fast.h"

namespace crk {
namespace {

// Order-preserving map of an fp32 value to uint32 (-0 and +0 map to the same key, as they compare equal).
__device__ __forceinline__ uint32_t orderable(float f) {
    uint32_t b = __float_as_uint(f);
    if (b == 0x80000000u) b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// ---- softmax, E <= 64 ----------------------------------------------------------------------------------
// 32 tokens per 256-thread workgroup; thread (token tok = tid / 8, expert group eg = tid % 8) owns experts
// 8 eg .. 8 eg + 7 of its token, so a token's eight threads are neighbouring lanes of one wavefront.
constexpr int kSmTok = 32;
constexpr int kSmStride = 65;           // LDS row stride of the [token][expert] tile (floats)
constexpr int kSmTrStride = kSmTok + 1;  // LDS row stride of the [expert][token] tile

// LDS of one softmax tile, declared once per kernel (both instantiations below share it).
struct SoftmaxLds {
    float tile[kSmTok * kSmStride];  // logits, then exponentials
    float tr[64 * kSmTrStride];      // probabilities, transposed
    float zrow[kSmTok];
};

// Tokens [32 b, 32 b + 32) (one 256-thread workgroup).  EF > 0 fixes E = EF at compile time (the router's
// 64 experts), which removes every per-expert bound check.
template <int EF>
__device__ __forceinline__ void softmax_tile(const float* __restrict__ in, int is_probs, int T, int E_arg,
                                             float* __restrict__ probs_t, float* __restrict__ probs_out,
                                             int32_t* __restrict__ slots, int b, SoftmaxLds& lds) {
    const int E = EF > 0 ? EF : E_arg;
    float* const tile = lds.tile;
    float* const tr = lds.tr;
    float* const zrow = lds.zrow;
    const int t0 = b * kSmTok;
    const int ntok = (T - t0) < kSmTok ? (T - t0) : kSmTok;
    const int tid = threadIdx.x, tok = tid >> 3, eg = tid & 7;
    if (slots) {  // the tile's rows of the slot table (contiguous) to -1
        int32_t* const srow = slots + (int64_t)t0 * E;
        const int ns = ntok * E;
        if (EF == 64 && ntok == kSmTok && (reinterpret_cast<uintptr_t>(srow) & 15) == 0) {
#pragma unroll
            for (int k = 0; k < 2; ++k) reinterpret_cast<int4*>(srow)[tid + 256 * k] = make_int4(-1, -1, -1, -1);
        } else {
            for (int i = tid; i < ns; i += 256) srow[i] = -1;
        }
    }
    const float* src = in + (int64_t)t0 * E;
    const int n = ntok * E;  // the tile is contiguous in global memory
    if (E == 64 && ntok == kSmTok && (reinterpret_cast<uintptr_t>(src) & 15) == 0) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int f = tid + 256 * k;  // float4 index: row f / 16, columns 4 (f % 16) ..
            const float4 v = reinterpret_cast<const float4*>(src)[f];
            float* d = tile + (f >> 4) * kSmStride + 4 * (f & 15);
            d[0] = v.x;
            d[1] = v.y;
            d[2] = v.z;
            d[3] = v.w;
        }
    } else {
        for (int i = tid; i < n; i += 256) {
            const int r = i / E;
            tile[r * kSmStride + (i - r * E)] = src[i];
        }
    }
    __syncthreads();
    const bool tv = tok < ntok;
    float* row = tile + tok * kSmStride;
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = (tv && 8 * eg + k < E) ? row[8 * eg + k] : -__builtin_inff();
    if (!is_probs) {
        float m = v[0];
#pragma unroll
        for (int k = 1; k < 8; ++k) m = fmaxf(m, v[k]);
        m = fmaxf(m, __shfl_xor(m, 1));  // the token's eight lanes
        m = fmaxf(m, __shfl_xor(m, 2));
        m = fmaxf(m, __shfl_xor(m, 4));
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            v[k] = (8 * eg + k < E) ? exp_fixed(v[k] - m) : 0.0f;
            if (tv && 8 * eg + k < E) row[8 * eg + k] = v[k];
        }
        __syncthreads();
        if (eg == 0 && tv) {
            // the entries are read 16 at a time, one chunk ahead of the sum; an expert past E adds +0, which
            // leaves the sum of non-negative terms unchanged
            float ex[2][16];
#pragma unroll
            for (int i = 0; i < 16; ++i) ex[0][i] = row[i];
            float z = 0.0f;
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) {
                if (ch + 1 < 4) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) ex[(ch + 1) & 1][i] = row[16 * (ch + 1) + i];
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) z = z + (16 * ch + i < E ? ex[ch & 1][i] : 0.0f);  // ascending order
            }
            zrow[tok] = z;
        }
        __syncthreads();
        const float z = zrow[tok];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = v[k] / z;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
        if (tv && 8 * eg + k < E) tr[(8 * eg + k) * kSmTrStride + tok] = v[k];
    if (probs_out && tv) {
        float* o = probs_out + (int64_t)(t0 + tok) * E;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (8 * eg + k < E) o[8 * eg + k] = v[k];
    }
    __syncthreads();
    // probs_t rows: float4 f covers expert f / 8, tokens 4 (f % 8) .. + 3 of this tile
    if (ntok == kSmTok && (T & 3) == 0 && (reinterpret_cast<uintptr_t>(probs_t) & 15) == 0) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int f = tid + 256 * k, e = f >> 3, c = 4 * (f & 7);
            if (e < E) {
                const float* a = tr + e * kSmTrStride + c;
                *reinterpret_cast<float4*>(probs_t + (int64_t)e * T + t0 + c) = make_float4(a[0], a[1], a[2], a[3]);
            }
        }
    } else {
        for (int i = tid; i < E * kSmTok; i += 256) {
            const int e = i / kSmTok, c = i - e * kSmTok;
            if (c < ntok) probs_t[(int64_t)e * T + t0 + c] = tr[e * kSmTrStride + c];
        }
    }
}

__global__ __launch_bounds__(256) void softmax_t_small_kernel(const float* __restrict__ in, int is_probs, int T, int E,
                                                              float* __restrict__ probs_t, float* __restrict__ probs_out,
                                                              int32_t* __restrict__ slots) {
    __shared__ SoftmaxLds lds;
    if (E == 64)
        softmax_tile<64>(in, is_probs, T, E, probs_t, probs_out, slots, blockIdx.x, lds);
    else
        softmax_tile<0>(in, is_probs, T, E, probs_t, probs_out, slots, blockIdx.x, lds);
}

// The router softmax and token rotate+quantise in one launch: they do not depend on each other, so the first
// nsm workgroups take softmax tiles and the rest take four token rows each, rows [0, rows); the
// rotate+quantise workgroups fill the CUs the short softmax leaves idle, with no second stream to join.
template <int G, int R>
__global__ __launch_bounds__(256) void softmax_rotq_kernel(const float* __restrict__ logits, int T, int E,
                                                           float* __restrict__ probs_t, int32_t* __restrict__ slots,
                                                           int nsm, const uint16_t* __restrict__ x, int K,
                                                           int8_t* __restrict__ qx, float* __restrict__ sx,
                                                           int64_t rows) {
    __shared__ SoftmaxLds lds;
    if ((int)blockIdx.x < nsm) {  // workgroup-uniform
        if (E == 64)
            softmax_tile<64>(logits, 0, T, E, probs_t, nullptr, slots, blockIdx.x, lds);
        else
            softmax_tile<0>(logits, 0, T, E, probs_t, nullptr, slots, blockIdx.x, lds);
        return;
    }
    const int64_t row = (int64_t)(blockIdx.x - nsm) * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;  // wave-uniform
    rotq_fast_row<G, R>(x, row, K, qx, sx);
}

// ---- softmax, any E (one thread per token) ------------------------------------------------------------
__global__ __launch_bounds__(256) void softmax_t_kernel(const float* __restrict__ in, int is_probs, int T, int E,
                                                        float* __restrict__ probs_t, float* __restrict__ probs_out,
                                                        int32_t* __restrict__ slots) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= T) return;
    if (slots)
        for (int e = 0; e < E; ++e) slots[(int64_t)t * E + e] = -1;
    const float* l = in + (int64_t)t * E;
    if (is_probs) {
        for (int e = 0; e < E; ++e) {
            const float p = l[e];
            probs_t[(int64_t)e * T + t] = p;
            if (probs_out) probs_out[(int64_t)t * E + e] = p;
        }
        return;
    }
    float m = l[0];
    for (int e = 1; e < E; ++e) m = fmaxf(m, l[e]);
    float z = 0.0f;
    for (int e = 0; e < E; ++e) z = z + exp_fixed(l[e] - m);
    for (int e = 0; e < E; ++e) {
        const float p = exp_fixed(l[e] - m) / z;
        probs_t[(int64_t)e * T + t] = p;
        if (probs_out) probs_out[(int64_t)t * E + e] = p;
    }
}

// ---- top-C selection ----------------------------------------------------------------------------------
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

// Exclusive prefix sum of a per-thread count over the workgroup (thread order) and the workgroup total.
__device__ __forceinline__ int block_excl_sum(int v, int* scratch, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == 63) scratch[wave] = incl;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
        const int c = scratch[w];
        before += (w < wave) ? c : 0;
        total += c;
    }
    __syncthreads();
    return before + incl - v;
}

// Keys in registers, eight wavefronts per expert: wavefront w owns tokens [256 KR w, 256 KR (w + 1)), lane l
// the four tokens 256 j + 4 l .. + 3 of round j.  Radix passes of up to 11 bits (2048 LDS bins, one scan by
// wavefront 0); the compaction needs one exchange of per-wavefront counts: a selected token's slot is
// (# greater keys before it) + min(# equal keys before it, C - # greater keys overall), and both prefixes come
// from ballots within a round.
constexpr int kSelV = 8;  // wavefronts per workgroup
constexpr int kSelFew = 64;     // at most this many keys left in the threshold's bin: one wavefront ranks them
constexpr int kSelStageC = 960;  // C up to this: the selected tokens are staged in LDS (in the bins' space)
constexpr int kSelBins = 2048;  // radix bins of one pass (11 bits)
// the bins are cleared with one 16-byte chunk per thread of the workgroup
static_assert(kSelV * 64 * 4 == kSelBins, "selection workgroup size and bin count are tied");

// Wavefront-wide min / max / sum of a uint32 through DPP (quad permutations and row rotations reduce each
// 16-lane row) and four lane reads; the result is wave-uniform.
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op) {
    v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, false));  // row_ror:4
    v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false));  // row_ror:8
    const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
    const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
    return op(op(a, b), op(c, d));
}
__device__ __forceinline__ uint32_t umin2(uint32_t a, uint32_t b) { return a < b ? a : b; }
__device__ __forceinline__ uint32_t umax2(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t uadd2(uint32_t a, uint32_t b) { return a + b; }

// Inclusive prefix sum over the wavefront's lanes: row_shr 1, 2, 4, 8 within each 16-lane row, then the row
// totals carried by row_bcast:15 and row_bcast:31 (lanes without a source add 0).
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
    return v;
}

// Sum over the lanes below this one of a per-lane count in [0, 7], and the total over the wavefront.
__device__ __forceinline__ int lanes_below(int v, int& total) {
    const uint64_t b0 = __ballot(v & 1), b1 = __ballot(v & 2), b2 = __ballot(v & 4);
    total = __popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2);
    auto below = [](uint64_t b) {
        return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
    };
    return below(b0) + 2 * below(b1) + 4 * below(b2);
}

// Selection of expert e by one workgroup of kSelV wavefronts.
template <int KR>
__device__ __forceinline__ void select_topc_v_block(const float* __restrict__ probs_t, int T, int C,
                                                    int32_t* __restrict__ idx, float* __restrict__ wt,
                                                    int32_t* __restrict__ slots, int E, int e,
                                                    uint32_t* __restrict__ esync) {
    __shared__ __attribute__((aligned(16))) uint32_t hist[kSelBins];
    __shared__ uint32_t s_red[2 * kSelV];
    __shared__ uint32_t s_bcast[3];
    __shared__ int s_cnt[2 * kSelV];
    __shared__ uint32_t s_cand[kSelFew];
    __shared__ uint32_t s_ncand;  // zeroed by every pass's scan; the early finish only follows a pass
    // staged tokens at hist[slot], weights at hist[1024 + slot]; slots kSelStageC + lane take the writes of
    // lanes that select nothing
    static_assert(kSelStageC + 64 <= kSelBins / 2, "staged selection fits the bins");
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (esync && tid == 0) {  // this expert's counters of the fused expert launch that follows
        esync[(2 * e) * kEsyncStride] = 0u;
        esync[(2 * e + 1) * kEsyncStride] = 0u;
    }
    const float* p = probs_t + (int64_t)e * T;
    const int tb = w * 256 * KR + 4 * lane;  // token of (round j, c): tb + 256 j + c
    const bool vec = (T & 3) == 0 && (reinterpret_cast<uintptr_t>(p) & 15) == 0;
    // Up to 8 rounds the values stay in registers for the weights of the selected tokens; beyond that a
    // selected token's value comes back from its key, which is invertible apart from the sign of zero: one bit
    // per key records a negative zero (bit 4 j + c of word (4 j + c) / 32).
    constexpr bool kKeepVal = KR <= 8;
    uint32_t key[KR][4];
    float val[kKeepVal ? KR : 1][4];
    uint32_t negz[kKeepVal ? 1 : (4 * KR + 31) / 32] = {};
#pragma unroll
    for (int j = 0; j < KR; ++j) {
        const int t = tb + 256 * j;
        float f[4];
        if (vec && t < T) {
            const float4 q = *reinterpret_cast<const float4*>(p + t);
            f[0] = q.x;
            f[1] = q.y;
            f[2] = q.z;
            f[3] = q.w;
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) f[c] = (t + c < T) ? p[t + c] : 0.0f;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            key[j][c] = orderable(f[c]);
            if constexpr (kKeepVal)
                val[j][c] = f[c];
            else
                negz[(4 * j + c) >> 5] |= (__float_as_uint(f[c]) == 0x80000000u ? 1u : 0u) << ((4 * j + c) & 31);
        }
    }
    // Tokens past T hold key 0, the smallest key there is: they only add to the lowest bins, never exceed the
    // threshold, and as equal keys they come after every real token, so they change no decision (C <= T).

    // leading bits shared by every key (skipped by the passes)
    uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int j = 0; j < KR; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            kmin = key[j][c] < kmin ? key[j][c] : kmin;
            kmax = key[j][c] > kmax ? key[j][c] : kmax;
        }
    kmin = wave_reduce_u32(kmin, umin2);
    kmax = wave_reduce_u32(kmax, umax2);
    if (lane == 0) {
        s_red[2 * w] = kmin;
        s_red[2 * w + 1] = kmax;
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < kSelV; ++x) {
        kmin = s_red[2 * x] < kmin ? s_red[2 * x] : kmin;
        kmax = s_red[2 * x + 1] > kmax ? s_red[2 * x + 1] : kmax;
    }
    const uint32_t diff = kmin ^ kmax;
    const int common = diff ? __clz(diff) : 32;
    uint32_t mask = common ? (0xffffffffu << (32 - common)) : 0u;
    uint32_t prefix = kmin & mask, remaining = (uint32_t)C;
    uint32_t n_left = kSelV * 256 * KR;  // keys that share the decided bits (the padding past T included)
    for (int hi = 32 - common; hi > 0;) {  // bits [0, hi) still undecided
        if (n_left <= (uint32_t)kSelFew) {  // workgroup-uniform
            // Few keys left: gather them, and one wavefront finds the remaining-th largest among them by
            // counting, for each, the keys above and equal to it.  Every key is compared in full, so the
            // threshold and the number of equal keys to take are those the remaining passes would give.
#pragma unroll
            for (int j = 0; j < KR; ++j)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if ((key[j][c] & mask) == prefix) {
                        // n_left keys pass this test (the bin count the scan reported), so a slot past the
                        // array cannot occur; the bound keeps the LDS write local to s_cand regardless
                        const uint32_t at = atomicAdd(&s_ncand, 1u);
                        if (at < (uint32_t)kSelFew) s_cand[at] = key[j][c];
                    }
            __syncthreads();
            if (w == 0) {
                const int n = (int)n_left;
                const uint32_t ck = lane < n ? s_cand[lane] : 0u;
                uint32_t gt = 0u, eq = 0u;
                for (int j = 0; j < n; ++j) {
                    const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)ck, j);
                    gt += kj > ck ? 1u : 0u;
                    eq += kj == ck ? 1u : 0u;
                }
                // the candidates in descending order: the remaining-th one has fewer than `remaining` keys
                // above it and at least `remaining` at or above it (1 <= remaining <= n, so one lane does)
                const bool hit = lane < n && gt < remaining && remaining <= gt + eq;
                const int first = __ffsll((unsigned long long)__ballot(hit)) - 1;
                if (lane == first) {
                    s_bcast[0] = ck;
                    s_bcast[1] = remaining - gt;
                }
            }
            __syncthreads();
            prefix = s_bcast[0];
            remaining = s_bcast[1];
            break;
        }
        const int width = hi < 11 ? hi : 11;
        const int shift = hi - width;
        const uint32_t dmask = (1u << width) - 1u;
        hi = shift;
        __syncthreads();  // the previous scan is done with the bins
        reinterpret_cast<uint4*>(hist)[tid] = make_uint4(0u, 0u, 0u, 0u);  // one 16-byte chunk per thread
        __syncthreads();
#pragma unroll
        for (int j = 0; j < KR; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if ((key[j][c] & mask) == prefix) atomicAdd(&hist[(key[j][c] >> shift) & dmask], 1u);
        __syncthreads();
        if (w == 0) {
            // lane l covers bins 2047 - 32 l down to 2016 - 32 l
            uint32_t cnt[32], sum = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint4 q = reinterpret_cast<const uint4*>(hist)[(2016 - 32 * lane) / 4 + k];
                cnt[31 - 4 * k] = q.x;
                cnt[30 - 4 * k] = q.y;
                cnt[29 - 4 * k] = q.z;
                cnt[28 - 4 * k] = q.w;
            }
#pragma unroll
            for (int q = 0; q < 32; ++q) sum += cnt[q];
            const uint32_t incl = wave_incl_sum(sum);
            const uint64_t hit = __ballot(incl >= remaining);
            const int first = __ffsll((unsigned long long)hit) - 1;
            // in lane `first`: the bins (descending) whose running count stays below `remaining` come before
            // the digit's bin; the running count is monotone, so they are a prefix (no branches)
            uint32_t cum = incl - sum, above = cum;
            int nb = 0;
#pragma unroll
            for (int q = 0; q < 32; ++q) {
                cum += cnt[q];
                const bool below = cum < remaining;
                nb += below ? 1 : 0;
                above += below ? cnt[q] : 0u;
            }
            if (lane == first) {
                const int digit = 2047 - 32 * lane - nb;
                s_bcast[0] = prefix | ((uint32_t)digit << shift);
                s_bcast[1] = remaining - above;
                s_bcast[2] = hist[digit];  // keys that share the digit too
                s_ncand = 0u;
            }
        }
        __syncthreads();
        prefix = s_bcast[0];
        remaining = s_bcast[1];
        n_left = s_bcast[2];
        mask |= dmask << shift;
    }
    const uint32_t v = prefix;        // the C-th largest key
    const int need_eq = (int)remaining;  // equal keys to take, lowest token index first

    // per-wavefront counts of equal and greater keys, then this wavefront's bases
    int n_eq = 0, n_gt = 0;
#pragma unroll
    for (int j = 0; j < KR; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            n_eq += key[j][c] == v ? 1 : 0;
            n_gt += key[j][c] > v ? 1 : 0;
        }
    n_eq = (int)wave_reduce_u32((uint32_t)n_eq, uadd2);
    n_gt = (int)wave_reduce_u32((uint32_t)n_gt, uadd2);
    if (lane == 0) {
        s_cnt[w] = n_eq;
        s_cnt[kSelV + w] = n_gt;
    }
    __syncthreads();
    int eqb = 0, gtb = 0;
#pragma unroll
    for (int x = 0; x < kSelV; ++x) {
        eqb += x < w ? s_cnt[x] : 0;
        gtb += x < w ? s_cnt[kSelV + x] : 0;
    }
    // C <= kSelStageC: the selected tokens and weights go to LDS by slot (the bins are free: the last read of
    // them was before the last barrier), and leave in slot order once all are placed.  Up to 8 rounds the rounds
    // are compiled once per choice (workgroup-uniform), so neither path carries the other's branches; more
    // rounds keep one copy that decides per token (two copies of 16 rounds would spill).
    const bool stage = C <= kSelStageC;
    int32_t* const s_tok = reinterpret_cast<int32_t*>(hist);
    float* const s_w = reinterpret_cast<float*>(hist + kSelBins / 2);
    // mode 0: direct stores, 1: staged, 2: decided per token by `stage`
    auto rounds = [&](auto mode_c) {
        constexpr int kMode = decltype(mode_c)::value;
#pragma unroll
        for (int j = 0; j < KR; ++j) {
            const int t = tb + 256 * j;
            bool eq[4], gt[4];
            int ne = 0, ng = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                eq[c] = key[j][c] == v;
                gt[c] = key[j][c] > v;
                ne += eq[c] ? 1 : 0;
                ng += gt[c] ? 1 : 0;
            }
            int tot_eq, tot_gt;
            int eqr = eqb + lanes_below(ne, tot_eq);
            int gtr = gtb + lanes_below(ng, tot_gt);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bool sel = gt[c] || (eq[c] && eqr < need_eq);
                const int pos = gtr + (eqr < need_eq ? eqr : need_eq);
                if constexpr (kMode == 1) {
                    // branch-free: every lane writes, a lane that selects nothing into its own unused slot
                    const int dst = (sel && pos < C) ? pos : kSelStageC + lane;
                    float v_out;
                    if constexpr (kKeepVal) {
                        v_out = val[j][c];
                    } else {
                        const uint32_t k = key[j][c];
                        const uint32_t zbit = (negz[(4 * j + c) >> 5] >> ((4 * j + c) & 31)) & 1u;
                        v_out = __uint_as_float((k & 0x80000000u) ? ((k & 0x7fffffffu) | (zbit << 31)) : ~k);
                    }
                    s_tok[dst] = t + c;
                    s_w[dst] = v_out;
                } else if (sel && pos < C) {
                    float v_out;
                    if constexpr (kKeepVal) {
                        v_out = val[j][c];
                    } else {
                        const uint32_t k = key[j][c];
                        const uint32_t zbit = (negz[(4 * j + c) >> 5] >> ((4 * j + c) & 31)) & 1u;
                        v_out = __uint_as_float((k & 0x80000000u) ? ((k & 0x7fffffffu) | (zbit << 31)) : ~k);
                    }
                    if (kMode == 2 && stage) {
                        s_tok[pos] = t + c;
                        s_w[pos] = v_out;
                    } else {
                        idx[(int64_t)e * C + pos] = t + c;
                        if (slots) slots[(int64_t)(t + c) * E + e] = pos;
                        wt[(int64_t)e * C + pos] = v_out;
                    }
                }
                eqr += eq[c] ? 1 : 0;
                gtr += gt[c] ? 1 : 0;
            }
            eqb += tot_eq;
            gtb += tot_gt;
        }
    };
    if constexpr (KR <= 8) {
        if (stage)
            rounds(std::integral_constant<int, 1>{});
        else
            rounds(std::integral_constant<int, 0>{});
    } else {
        rounds(std::integral_constant<int, 2>{});
    }
    if (stage) {
        __syncthreads();
        for (int i = tid; i < C; i += kSelV * 64) {  // every slot below C holds one selected token (C <= T)
            const int tt = s_tok[i];
            idx[(int64_t)e * C + i] = tt;
            wt[(int64_t)e * C + i] = s_w[i];
            if (slots) slots[(int64_t)tt * E + e] = i;
        }
    }
}

template <int KR>
__global__ __launch_bounds__(kSelV * 64) void select_topc_v_kernel(const float* __restrict__ probs_t, int T, int C,
                                                                   int32_t* __restrict__ idx, float* __restrict__ wt,
                                                                   int32_t* __restrict__ slots, int E,
                                                                   uint32_t* __restrict__ esync) {
    select_topc_v_block<KR>(probs_t, T, C, idx, wt, slots, E, blockIdx.x, esync);
}

// The selection and the rest of the token rotate+quantise in one launch: the first E workgroups select (one
// expert each, a few CUs for a few microseconds), the others take kSelV token rows each from row0 on.
template <int KR, int G, int R>
__global__ __launch_bounds__(kSelV * 64) void select_rotq_kernel(const float* __restrict__ probs_t, int T, int C, int E,
                                                                 int32_t* __restrict__ idx, float* __restrict__ wt,
                                                                 int32_t* __restrict__ slots,
                                                                 const uint16_t* __restrict__ x, int K,
                                                                 int8_t* __restrict__ qx, float* __restrict__ sx,
                                                                 int64_t row0, uint32_t* __restrict__ esync) {
    if ((int)blockIdx.x < E) {  // workgroup-uniform
        select_topc_v_block<KR>(probs_t, T, C, idx, wt, slots, E, blockIdx.x, esync);
        return;
    }
    const int64_t row = row0 + (int64_t)(blockIdx.x - E) * kSelV + (threadIdx.x >> 6);
    if (row >= T) return;  // wave-uniform
    rotq_fast_row<G, R>(x, row, K, qx, sx);
}

// Any T: keys re-read from global memory in each pass.
__global__ __launch_bounds__(kSelThreads) void select_topc_kernel(const float* __restrict__ probs_t, int T, int C,
                                                                  int32_t* __restrict__ idx, float* __restrict__ wt,
                                                                  int32_t* __restrict__ slots, int E,
                                                                  uint32_t* __restrict__ esync) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t s_prefix, s_remaining;
    __shared__ int scratch[kSelWaves];

    const int e = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    if (esync && tid == 0) {  // this expert's counters of the fused expert launch that follows
        esync[(2 * e) * kEsyncStride] = 0u;
        esync[(2 * e + 1) * kEsyncStride] = 0u;
    }
    const float* p = probs_t + (int64_t)e * T;

    uint32_t prefix = 0, mask = 0, remaining = (uint32_t)C;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        for (int t = tid; t < T; t += kSelThreads) {
            const uint32_t k = orderable(p[t]);
            if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid < 64) {
            uint32_t c[4], sum = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                c[q] = hist[255 - 4 * lane - q];
                sum += c[q];
            }
            uint32_t incl = sum;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t o = __shfl_up(incl, off);
                if (lane >= off) incl += o;
            }
            const uint64_t hit = __ballot(incl >= remaining);
            const int first = __ffsll((unsigned long long)hit) - 1;
            if (lane == first) {
                uint32_t above = incl - sum;
                int digit = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (above + c[q] >= remaining) {
                        digit = 255 - 4 * lane - q;
                        break;
                    }
                    above += c[q];
                }
                s_prefix = prefix | ((uint32_t)digit << shift);
                s_remaining = remaining - above;
            }
        }
        __syncthreads();
        prefix = s_prefix;
        remaining = s_remaining;
        mask |= 255u << shift;
        __syncthreads();
    }
    const uint32_t v = prefix;
    const int need_eq = (int)remaining;

    int carry_eq = 0, carry_sel = 0;
    for (int base = 0; base < T; base += kSelThreads) {
        const int t = base + tid;
        const bool valid = t < T;
        const float pv = valid ? p[t] : 0.0f;
        const uint32_t k = orderable(pv);
        const bool is_eq = valid && k == v;
        const bool is_gt = valid && k > v;
        int tot_eq, tot_sel;
        const int eq_rank = carry_eq + block_excl_sum(is_eq ? 1 : 0, scratch, tot_eq);
        const bool sel = is_gt || (is_eq && eq_rank < need_eq);
        const int pos = carry_sel + block_excl_sum(sel ? 1 : 0, scratch, tot_sel);
        if (sel && pos < C) {
            idx[(int64_t)e * C + pos] = t;
            wt[(int64_t)e * C + pos] = pv;
            if (slots) slots[(int64_t)t * E + e] = pos;
        }
        carry_eq += tot_eq;
        carry_sel += tot_sel;
    }
}

// Entries of the given lists (idx [E, C]); tokens outside [0, T) are ignored.  The table is -1 beforehand.
__global__ __launch_bounds__(256) void build_slots_kernel(const int32_t* __restrict__ idx, int T, int E, int C,
                                                          int32_t* __restrict__ slots) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)E * C) return;
    const int e = (int)(i / C), c = (int)(i - (int64_t)e * C);
    const int t = idx[i];
    if (t >= 0 && t < T) slots[(int64_t)t * E + e] = c;
}

__global__ __launch_bounds__(256) void fill_minus_one_kernel(int32_t* __restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = -1;
}

}  // namespace

hipError_t launch_softmax_t(const float* in, int is_probs, int T, int E, float* probs_t, float* probs_out,
                            int32_t* slots, hipStream_t st) {
    if (E <= 64)
        softmax_t_small_kernel<<<dim3((T + kSmTok - 1) / kSmTok), dim3(256), 0, st>>>(in, is_probs, T, E, probs_t,
                                                                                      probs_out, slots);
    else
        softmax_t_kernel<<<dim3((T + 255) / 256), dim3(256), 0, st>>>(in, is_probs, T, E, probs_t, probs_out,
                                                                      slots);
    return hipGetLastError();
}

hipError_t launch_softmax_rotq(const float* logits, int T, int E, float* probs_t, int32_t* slots,
                               const uint16_t* x, int K, int group, int8_t* qx, float* sx, int64_t rows,
                               hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (E > 64 || K % (8 * group) != 0 || rows < 0 || rows > T) return hipErrorNotSupported;
    const int nsm = (T + kSmTok - 1) / kSmTok;
    const int64_t nrot = (rows + 3) / 4;
    const dim3 grid((unsigned)(nsm + nrot)), block(256);
    const int R = K / (8 * group);
#define CRK_SR(GG, RR)                                                                                  \
    if (group == GG && R == RR) {                                                                       \
        softmax_rotq_kernel<GG, RR><<<grid, block, 0, st>>>(logits, T, E, probs_t, slots, nsm, x, K, qx, sx,   \
                                                            rows);                                            \
        return hipGetLastError();                                                                       \
    }
    CRK_SR(256, 1)
    CRK_SR(256, 2)
    CRK_SR(256, 4)
    CRK_SR(64, 1)
    CRK_SR(64, 2)
    CRK_SR(64, 4)
#undef CRK_SR
    return hipErrorNotSupported;
}

hipError_t launch_select_topc(const float* probs_t, int T, int E, int C, int32_t* idx, float* wt,
                              int32_t* slots, uint32_t* esync, hipStream_t st) {
#define CRK_SEL(K)                                                                                              \
    if (T <= kSelV * 256 * K) {                                                                                 \
        select_topc_v_kernel<K><<<dim3(E), dim3(kSelV * 64), 0, st>>>(probs_t, T, C, idx, wt, slots, E, esync); \
        return hipGetLastError();                                                                               \
    }
    CRK_SEL(1)
    CRK_SEL(2)
    CRK_SEL(4)
    CRK_SEL(8)
    CRK_SEL(16)
#undef CRK_SEL
    select_topc_kernel<<<dim3(E), dim3(kSelThreads), 0, st>>>(probs_t, T, C, idx, wt, slots, E, esync);
    return hipGetLastError();
}

bool select_rotq_supported(int T, int E, int K, int group) {
    const int R = (group > 0 && K % (8 * group) == 0) ? K / (8 * group) : 0;
    return T >= 1 && T <= kSelV * 256 * 8 && E >= 1 && (group == 256 || group == 64) && (R == 1 || R == 2 || R == 4);
}

hipError_t launch_select_rotq(const float* probs_t, int T, int E, int C, int32_t* idx, float* wt, int32_t* slots,
                              const uint16_t* x, int K, int group, int8_t* qx, float* sx, int64_t row0,
                              uint32_t* esync, hipStream_t st) {
    if (!select_rotq_supported(T, E, K, group) || row0 < 0 || row0 > T) return hipErrorNotSupported;
    const int R = K / (8 * group);
    const int64_t nrot = (T - row0 + kSelV - 1) / kSelV;
    const dim3 grid((unsigned)(E + nrot)), block(kSelV * 64);
#define CRK_SR2(KK, GG, RR)                                                                                 \
    if (T <= kSelV * 256 * KK && group == GG && R == RR) {                                                  \
        select_rotq_kernel<KK, GG, RR><<<grid, block, 0, st>>>(probs_t, T, C, E, idx, wt, slots, x, K, qx, sx, \
                                                               row0, esync);                               \
        return hipGetLastError();                                                                           \
    }
#define CRK_SR2_G(KK) CRK_SR2(KK, 256, 1) CRK_SR2(KK, 256, 2) CRK_SR2(KK, 256, 4) CRK_SR2(KK, 64, 1) \
    CRK_SR2(KK, 64, 2) CRK_SR2(KK, 64, 4)
    CRK_SR2_G(1)
    CRK_SR2_G(2)
    CRK_SR2_G(4)
    CRK_SR2_G(8)
#undef CRK_SR2_G
#undef CRK_SR2
    return hipErrorNotSupported;
}

hipError_t launch_build_slots(const int32_t* idx, int T, int E, int C, int32_t* slots, hipStream_t st) {
    const int64_t n = (int64_t)T * E, m = (int64_t)E * C;
    fill_minus_one_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st>>>(slots, n);
    build_slots_kernel<<<dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st>>>(idx, T, E, C, slots);
    return hipGetLastError();
}

}  // namespace crk
