// Expert-choice routing ("MLX Nucleus-Image": each of the 64 routed experts picks its top-C tokens).
//
//  softmax_t     one thread per token: p[t, :] = softmax over experts in fp32 (max-subtracted, the fixed
//                exponential, sum in ascending expert order, one IEEE division per entry), written
//                transposed as probs_t[e, t] so that each expert's column is contiguous.
//  select_topc   one workgroup per expert: radix select (four 8-bit passes, most significant first) of the
//                C-th largest key, then one ordered compaction pass that keeps every token above the
//                threshold and the lowest-index tokens equal to it.  The list comes out in ascending token
//                order without a sort; ties go to the lower token index by construction.
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

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

// Exclusive prefix count of a per-thread flag over the workgroup (thread order = token order) and the
// workgroup total.  `scratch` holds one count per wave.
__device__ __forceinline__ int block_excl_count(bool flag, int* scratch, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t mask = __ballot(flag);
    const int before_in_wave = __popcll(mask & ((1ull << lane) - 1ull));
    if (lane == 0) scratch[wave] = __popcll(mask);
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
    return before + before_in_wave;
}

__global__ __launch_bounds__(kSelThreads) void select_topc_kernel(const float* __restrict__ probs_t, int T, int C,
                                                                  int32_t* __restrict__ idx, float* __restrict__ wt,
                                                                  int32_t* __restrict__ slotmap) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t s_prefix, s_remaining;
    __shared__ int scan_scratch[kSelWaves];

    const int e = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    const float* p = probs_t + (int64_t)e * T;

    // ---- radix select: threshold key v such that #(key > v) < C <= #(key >= v) ----
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
    const int need_eq = (int)remaining;  // tokens equal to v to take, lowest indices first

    // ---- ordered compaction ----
    int carry_eq = 0, carry_sel = 0;
    for (int base = 0; base < T; base += kSelThreads) {
        const int t = base + tid;
        const bool valid = t < T;
        const float pv = valid ? p[t] : 0.0f;
        const uint32_t k = orderable(pv);
        const bool is_eq = valid && k == v;
        const bool is_gt = valid && k > v;
        int tot_eq, tot_sel;
        const int eq_rank = carry_eq + block_excl_count(is_eq, scan_scratch, tot_eq);
        const bool sel = is_gt || (is_eq && eq_rank < need_eq);
        const int pos = carry_sel + block_excl_count(sel, scan_scratch, tot_sel);
        if (sel && pos < C) {
            idx[(int64_t)e * C + pos] = t;
            wt[(int64_t)e * C + pos] = pv;
        }
        if (valid && slotmap) slotmap[(int64_t)e * T + t] = sel ? pos : -1;
        carry_eq += tot_eq;
        carry_sel += tot_sel;
    }
    (void)lane;
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
    softmax_t_kernel<<<dim3((T + 255) / 256), dim3(256), 0, st>>>(in, is_probs, T, E, probs_t, probs_out);
    return hipGetLastError();
}

hipError_t launch_select_topc(const float* probs_t, int T, int E, int C, int32_t* idx, float* wt,
                              int32_t* slotmap, hipStream_t st) {
    select_topc_kernel<<<dim3(E), dim3(kSelThreads), 0, st>>>(probs_t, T, C, idx, wt, slotmap);
    return hipGetLastError();
}

hipError_t launch_build_slotmap(const int32_t* idx, int T, int E, int C, int32_t* slotmap, hipStream_t st) {
    build_slotmap_kernel<<<dim3(E), dim3(1024), 0, st>>>(idx, T, C, slotmap);
    return hipGetLastError();
}

}  // namespace crk
