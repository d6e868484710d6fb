// Expert-choice routing ("MLX Nucleus-Image": each of the 64 routed experts picks its top-C tokens).
//
//  softmax_t     p[t, :] = softmax over experts in fp32 (max-subtracted, the fixed exponential, sum in
//                ascending expert order, one IEEE division per entry), written transposed as probs_t[e, t]
//                so that each expert's column is contiguous.  E <= 64: a workgroup stages a 64-token x E
//                tile of logits in LDS (coalesced loads), splits the exponentials and divisions over its
//                four wavefronts, and keeps the sequential sum in one lane per token.
//  select_topc   one workgroup per expert: radix select (four 8-bit passes, most significant first) of the
//                C-th largest key over keys held in registers, then one ordered compaction (a workgroup
//                scan of per-thread counts) that keeps every token above the threshold and the lowest-index
//                tokens equal to it.  The list comes out in ascending token order without a sort; ties go
//                to the lower token index by construction.
//  build_slotmap per expert: slotmap[e, t] = position of t in expert e's list, or -1.
#include "device_common.h"
#include "kernels.h"

namespace crk {
namespace {

// Order-preserving map of an fp32 value to uint32 (-0 and +0 map to the same key, as they compare equal).
__device__ __forceinline__ uint32_t orderable(float f) {
    uint32_t b = __float_as_uint(f);
    if (b == 0x80000000u) b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// ---- softmax, E <= 64 ----------------------------------------------------------------------------------
constexpr int kSmTok = 64;     // tokens per workgroup
constexpr int kSmStride = 65;  // LDS row stride (floats): lane t reads row t without bank conflicts

__global__ __launch_bounds__(256) void softmax_t_small_kernel(const float* __restrict__ in, int is_probs, int T, int E,
                                                              float* __restrict__ probs_t, float* __restrict__ probs_out) {
    __shared__ float tile[kSmTok * kSmStride];  // logits, then exponentials, then probabilities
    __shared__ float rowmax[4][kSmTok];
    __shared__ float rowsum[kSmTok];
    const int t0 = blockIdx.x * kSmTok;
    const int ntok = (T - t0) < kSmTok ? (T - t0) : kSmTok;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* src = in + (int64_t)t0 * E;
    for (int r = wave; r < ntok; r += 4)  // one coalesced row of E <= 64 floats per wavefront instruction
        if (lane < E) tile[r * kSmStride + lane] = src[(int64_t)r * E + lane];
    __syncthreads();
    // experts handled by this wavefront: e = wave, wave + 4, ...
    if (!is_probs) {
        if (lane < ntok) {
            const float* row = tile + lane * kSmStride;
            float m = -__builtin_inff();
            for (int e = wave; e < E; e += 4) m = fmaxf(m, row[e]);
            rowmax[wave][lane] = m;
        }
        __syncthreads();
        if (lane < ntok) {
            float* row = tile + lane * kSmStride;
            const float m = fmaxf(fmaxf(rowmax[0][lane], rowmax[1][lane]), fmaxf(rowmax[2][lane], rowmax[3][lane]));
            for (int e = wave; e < E; e += 4) row[e] = exp_fixed(row[e] - m);
        }
        __syncthreads();
        if (wave == 0 && lane < ntok) {
            const float* row = tile + lane * kSmStride;
            float z = 0.0f;
            for (int e = 0; e < E; ++e) z = z + row[e];  // ascending expert order
            rowsum[lane] = z;
        }
        __syncthreads();
        if (lane < ntok) {
            float* row = tile + lane * kSmStride;
            const float z = rowsum[lane];
            for (int e = wave; e < E; e += 4) row[e] = row[e] / z;
        }
        __syncthreads();
    }
    if (lane < ntok)
        for (int e = wave; e < E; e += 4) probs_t[(int64_t)e * T + t0 + lane] = tile[lane * kSmStride + e];
    if (probs_out)
        for (int r = wave; r < ntok; r += 4)
            if (lane < E) probs_out[(int64_t)(t0 + r) * E + lane] = tile[r * kSmStride + lane];
}

// ---- softmax, any E (one thread per token) ------------------------------------------------------------
__global__ __launch_bounds__(256) void softmax_t_kernel(const float* __restrict__ in, int is_probs, int T, int E,
                                                        float* __restrict__ probs_t, float* __restrict__ probs_out) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= T) return;
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

// Radix select: the key v with #(key > v) < C <= #(key >= v); returns v and sets need_eq = C - #(key > v).
// The leading bits all keys share (from the workgroup min and max) are skipped, so the passes work on bits
// that actually differ: softmax probabilities share their sign and high exponent bits, and a first pass
// over those would pile every key into one or two histogram bins.
template <int KPT>
__device__ uint32_t radix_select(const uint32_t (&key)[KPT], const bool (&valid)[KPT], int C, uint32_t* hist,
                                 uint32_t* s_prefix, uint32_t* s_remaining, uint32_t* s_minmax, int& need_eq) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int j = 0; j < KPT; ++j)
        if (valid[j]) {
            kmin = key[j] < kmin ? key[j] : kmin;
            kmax = key[j] > kmax ? key[j] : kmax;
        }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t a = __shfl_xor(kmin, off), b = __shfl_xor(kmax, off);
        kmin = a < kmin ? a : kmin;
        kmax = b > kmax ? b : kmax;
    }
    if (lane == 0) {
        s_minmax[2 * wave] = kmin;
        s_minmax[2 * wave + 1] = kmax;
    }
    __syncthreads();
    kmin = 0xffffffffu;
    kmax = 0u;
    for (int w = 0; w < kSelWaves; ++w) {
        kmin = s_minmax[2 * w] < kmin ? s_minmax[2 * w] : kmin;
        kmax = s_minmax[2 * w + 1] > kmax ? s_minmax[2 * w + 1] : kmax;
    }
    const uint32_t diff = kmin ^ kmax;
    const int common = diff ? __clz(diff) : 32;  // leading bits shared by every key
    uint32_t mask = common ? (0xffffffffu << (32 - common)) : 0u;
    uint32_t prefix = kmin & mask, remaining = (uint32_t)C;
    for (int hi = 32 - common; hi > 0;) {  // bits [0, hi) still undecided
        const int width = hi < 8 ? hi : 8;
        const int shift = hi - width;
        const uint32_t dmask = (1u << width) - 1u;
        hi = shift;
        __syncthreads();
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < KPT; ++j)
            if (valid[j] && (key[j] & mask) == prefix) atomicAdd(&hist[(key[j] >> shift) & dmask], 1u);
        __syncthreads();
        if (tid < 64) {
            // lane l covers bins 255-4l .. 252-4l (descending); find the bin where the count from the top
            // reaches `remaining`.
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
                *s_prefix = prefix | ((uint32_t)digit << shift);
                *s_remaining = remaining - above;
            }
        }
        __syncthreads();
        prefix = *s_prefix;
        remaining = *s_remaining;
        mask |= dmask << shift;
    }
    need_eq = (int)remaining;
    return prefix;
}

// Keys in registers: thread tid owns tokens tid*KPT .. tid*KPT + KPT - 1 (requires T <= 1024 * KPT).
template <int KPT>
__global__ __launch_bounds__(kSelThreads) void select_topc_reg_kernel(const float* __restrict__ probs_t, int T, int C,
                                                                      int32_t* __restrict__ idx, float* __restrict__ wt,
                                                                      int32_t* __restrict__ slotmap) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t s_prefix, s_remaining;
    __shared__ uint32_t s_minmax[2 * kSelWaves];
    __shared__ int scratch[kSelWaves];
    const int e = blockIdx.x;
    const int tid = threadIdx.x;
    const float* p = probs_t + (int64_t)e * T;
    const int tb = tid * KPT;
    float pv[KPT];
    uint32_t key[KPT];
    bool valid[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        valid[j] = tb + j < T;
        pv[j] = valid[j] ? p[tb + j] : 0.0f;
        key[j] = orderable(pv[j]);
    }
    int need_eq;
    const uint32_t v = radix_select<KPT>(key, valid, C, hist, &s_prefix, &s_remaining, s_minmax, need_eq);

    int n_eq = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) n_eq += (valid[j] && key[j] == v) ? 1 : 0;
    int tot;
    int eq_rank = block_excl_sum(n_eq, scratch, tot);
    bool sel[KPT];
    int n_sel = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const bool is_eq = valid[j] && key[j] == v;
        sel[j] = (valid[j] && key[j] > v) || (is_eq && eq_rank < need_eq);
        eq_rank += is_eq ? 1 : 0;
        n_sel += sel[j] ? 1 : 0;
    }
    int pos = block_excl_sum(n_sel, scratch, tot);
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        if (!valid[j]) continue;
        if (sel[j] && pos < C) {
            idx[(int64_t)e * C + pos] = tb + j;
            wt[(int64_t)e * C + pos] = pv[j];
        }
        if (slotmap) slotmap[(int64_t)e * T + tb + j] = sel[j] ? pos : -1;
        pos += sel[j] ? 1 : 0;
    }
}

// Any T: keys re-read from global memory in each pass.
__global__ __launch_bounds__(kSelThreads) void select_topc_kernel(const float* __restrict__ probs_t, int T, int C,
                                                                  int32_t* __restrict__ idx, float* __restrict__ wt,
                                                                  int32_t* __restrict__ slotmap) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t s_prefix, s_remaining;
    __shared__ int scratch[kSelWaves];

    const int e = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
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
        }
        if (valid && slotmap) slotmap[(int64_t)e * T + t] = sel ? pos : -1;
        carry_eq += tot_eq;
        carry_sel += tot_sel;
    }
}

__global__ __launch_bounds__(1024) void build_slotmap_kernel(const int32_t* __restrict__ idx, int T, int C,
                                                             int32_t* __restrict__ slotmap) {
    const int e = blockIdx.x;
    int32_t* row = slotmap + (int64_t)e * T;
    for (int t = threadIdx.x; t < T; t += 1024) row[t] = -1;
    __syncthreads();
    for (int c = threadIdx.x; c < C; c += 1024) {
        const int t = idx[(int64_t)e * C + c];
        if (t >= 0 && t < T) row[t] = c;  // entries outside [0, T) are ignored
    }
}

}  // namespace

hipError_t launch_softmax_t(const float* in, int is_probs, int T, int E, float* probs_t, float* probs_out,
                            hipStream_t st) {
    if (E <= 64)
        softmax_t_small_kernel<<<dim3((T + kSmTok - 1) / kSmTok), dim3(256), 0, st>>>(in, is_probs, T, E, probs_t,
                                                                                      probs_out);
    else
        softmax_t_kernel<<<dim3((T + 255) / 256), dim3(256), 0, st>>>(in, is_probs, T, E, probs_t, probs_out);
    return hipGetLastError();
}

hipError_t launch_select_topc(const float* probs_t, int T, int E, int C, int32_t* idx, float* wt,
                              int32_t* slotmap, hipStream_t st) {
    const dim3 grid(E), block(kSelThreads);
#define CRK_SEL(K)                                                                            \
    if (T <= kSelThreads * K) {                                                               \
        select_topc_reg_kernel<K><<<grid, block, 0, st>>>(probs_t, T, C, idx, wt, slotmap);   \
        return hipGetLastError();                                                             \
    }
    CRK_SEL(1)
    CRK_SEL(2)
    CRK_SEL(4)
    CRK_SEL(8)
    CRK_SEL(16)
#undef CRK_SEL
    select_topc_kernel<<<grid, block, 0, st>>>(probs_t, T, C, idx, wt, slotmap);
    return hipGetLastError();
}

hipError_t launch_build_slotmap(const int32_t* idx, int T, int E, int C, int32_t* slotmap, hipStream_t st) {
    build_slotmap_kernel<<<dim3(E), dim3(1024), 0, st>>>(idx, T, C, slotmap);
    return hipGetLastError();
}

}  // namespace crk
