// Achievable-rate probes (measurement aids, not steps of the method): the int8 MFMA rate on changing register
// operands, and the HBM read rate through non-temporal LDS DMA.  One persistent workgroup of 8 wavefronts per
// compute unit; the caller times the launch.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/convrot_probes.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr size_t kMfmaSrcBytes = 256 * 1024;  // operand pool: 16384 16-byte lane operands
constexpr int kDmaDepth = 8;                   // 1 KiB DMAs in flight per wavefront
constexpr size_t kDmaChunk = (size_t)kWaves * 1024;
constexpr int kMaxIters = 1 << 20;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    // gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

__global__ __launch_bounds__(kThreads) void mfma_rate_kernel(const v4i* __restrict__ src, int iters,
                                                             int32_t* __restrict__ out) {
    constexpr int kVec = (int)(kMfmaSrcBytes / 16);
    const int lane = threadIdx.x & 63;
    const int w = blockIdx.x * kWaves + (threadIdx.x >> 6);
    v4i a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        a[j] = src[((w * 8 + j) * 64 + lane) % kVec];
        b[j] = src[((w * 8 + 4 + j) * 64 + lane) % kVec];
    }
    v4i acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = v4i{0, 0, 0, 0};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[(j + r) & 3], b[j & 3], acc[j], 0, 0, 0);
    }
    int x = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k) x ^= acc[j][k];
    out[(size_t)blockIdx.x * kThreads + threadIdx.x] = x;
}

__global__ __launch_bounds__(kThreads) void hbm_read_kernel(const int8_t* __restrict__ src, size_t per_wg,
                                                            int32_t* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) int8_t lds[kWaves * kDmaDepth * 1024];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const size_t per_wave = per_wg / kWaves;  // a multiple of 1 KiB
    const int8_t* base = src + blockIdx.x * per_wg + wave * per_wave + lane * 16;
    const size_t n = per_wave / 1024;
    for (size_t i = 0; i < n; ++i) {
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(base + i * 1024),
                                         (lds_void*)(lds + (wave * kDmaDepth + (int)(i % kDmaDepth)) * 1024), 16,
                                         0, 2 /* non-temporal */);
        wait_vmcnt<kDmaDepth - 1>();
    }
    wait_vmcnt<0>();
    __syncthreads();
    out[(size_t)blockIdx.x * kThreads + threadIdx.x] = lds[threadIdx.x * 16];
}

int compute_units() {
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return ncu > 0 ? ncu : 0;
}

}  // namespace

extern "C" {

size_t convrot_probe_out_words(void) { return (size_t)compute_units() * kThreads; }

convrot_status convrot_probe_mfma_i8(const int8_t* src, size_t src_bytes, int iters, int32_t* out,
                                     size_t out_words, double* ops, hipStream_t stream) {
    if (!src || !out || !ops) return CONVROT_ERR_NULL;
    const int ncu = compute_units();
    if (ncu == 0) return CONVROT_ERR_HIP;
    if (src_bytes < kMfmaSrcBytes || iters < 1 || iters > kMaxIters || out_words < (size_t)ncu * kThreads)
        return CONVROT_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(src) % 16) return CONVROT_ERR_ALIGN;
    mfma_rate_kernel<<<dim3((unsigned)ncu), dim3(kThreads), 0, stream>>>(reinterpret_cast<const v4i*>(src), iters,
                                                                          out);
    if (hipGetLastError() != hipSuccess) return CONVROT_ERR_HIP;
    *ops = (double)ncu * kWaves * iters * 32 * (2.0 * 16 * 16 * 64);
    return CONVROT_OK;
}

convrot_status convrot_probe_hbm_read(const int8_t* src, size_t src_bytes, int32_t* out, size_t out_words,
                                      double* bytes, hipStream_t stream) {
    if (!src || !out || !bytes) return CONVROT_ERR_NULL;
    const int ncu = compute_units();
    if (ncu == 0) return CONVROT_ERR_HIP;
    const size_t per_wg = src_bytes / (size_t)ncu / kDmaChunk * kDmaChunk;
    if (per_wg == 0 || out_words < (size_t)ncu * kThreads) return CONVROT_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(src) % 16) return CONVROT_ERR_ALIGN;
    hbm_read_kernel<<<dim3((unsigned)ncu), dim3(kThreads), 0, stream>>>(src, per_wg, out);
    if (hipGetLastError() != hipSuccess) return CONVROT_ERR_HIP;
    *bytes = (double)per_wg * ncu;
    return CONVROT_OK;
}

}  // extern "C"
