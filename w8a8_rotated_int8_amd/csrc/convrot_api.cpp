// C ABI of libconvrot_amd: host-side argument validation, workspace planning and launch sequencing.
// Every check runs before the first enqueue, so an invalid call touches no output.  The library allocates
// no device memory; the caller passes the workspace.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <vector>

#include "../../include/convrot.h"
#include "kernels.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int kRotqBesideSoftmaxPct = 25;  // share of the token rows rotated in the softmax launch
constexpr int kMaxRowLen = 8192;           // rotate/quantise keeps a row in registers of one wavefront
constexpr int64_t kMaxKInt32 = 131056;     // K * 128^2 < 2^31 for any int8 codes (-128 included), K % 16 == 0


size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool group_ok(int g) { return g == 64 || g == 256; }

convrot_status hip_status(hipError_t e) { return e == hipSuccess ? CONVROT_OK : CONVROT_ERR_HIP; }

// Carves consecutive 256-byte aligned buffers out of a workspace (or just measures when base == nullptr).
struct Carver {
    char* base;
    size_t used = 0;
    explicit Carver(void* b) : base(static_cast<char*>(b)) {}
    template <class T>
    T* take(size_t count) {
        T* p = base ? reinterpret_cast<T*>(base + used) : nullptr;
        used += round_up(count * sizeof(T));
        return p;
    }
};

struct MoeBuffers {
    float* probs_t;
    int32_t* slots;  // [T, E]: position of token t in expert e's list, or -1
    int8_t* qx;
    float* sx;
    int32_t* idx;
    float* wt;
    uint16_t* a;
    int8_t* qa;
    float* sa;
    uint16_t* z;
    uint32_t* esync;  // per-expert counters of the fused expert launch
};

size_t plan_moe(void* ws, int T, int C, const convrot_moe_weights& w, MoeBuffers* b) {
    Carver cv(ws);
    const size_t S = (size_t)w.E * (size_t)C;
    MoeBuffers m;
    m.probs_t = cv.take<float>((size_t)w.E * T);
    m.slots = cv.take<int32_t>((size_t)T * w.E);
    m.qx = cv.take<int8_t>((size_t)T * w.d);
    m.sx = cv.take<float>((size_t)T);
    m.idx = cv.take<int32_t>(S);
    m.wt = cv.take<float>(S);
    m.a = cv.take<uint16_t>(S * w.I);
    m.qa = cv.take<int8_t>(S * w.I);
    m.sa = cv.take<float>(S);
    m.z = cv.take<uint16_t>(S * w.d);
    m.esync = cv.take<uint32_t>((size_t)2 * w.E * crk::kEsyncStride);
    if (b) *b = m;
    return cv.used;
}

convrot_status check_weights(const convrot_moe_weights* w) {
    if (!w) return CONVROT_ERR_NULL;
    if (!w->q_gu || !w->s_gu || !w->q_dn || !w->s_dn) return CONVROT_ERR_NULL;
    if (w->E < 1 || w->d < 1 || w->I < 1) return CONVROT_ERR_SHAPE;
    if (w->d > kMaxRowLen || w->I > kMaxRowLen) return CONVROT_ERR_SHAPE;
    if (w->wbits != 8 && w->wbits != 4) return CONVROT_ERR_BITS;
    if (!group_ok(w->group_gu) || !group_ok(w->group_dn)) return CONVROT_ERR_GROUP;
    if (w->d % w->group_gu || w->I % w->group_dn) return CONVROT_ERR_GROUP;
    if (w->I % 64) return CONVROT_ERR_SHAPE;
    if (!aligned16(w->q_gu) || !aligned16(w->s_gu) || !aligned16(w->q_dn) || !aligned16(w->s_dn))
        return CONVROT_ERR_ALIGN;
    if ((int64_t)w->E * 2 * w->I > INT32_MAX || (int64_t)w->E * w->d > INT32_MAX) return CONVROT_ERR_SHAPE;
    return CONVROT_OK;
}

convrot_status check_tc(int T, int C, int E) {
    if (T < 1 || C < 1 || C > T || E < 1) return CONVROT_ERR_SHAPE;
    if ((int64_t)E * C > INT32_MAX || (int64_t)E * T > INT32_MAX) return CONVROT_ERR_SHAPE;
    return CONVROT_OK;
}

crk::GemmProblem gateup_problem(const int8_t* qx, const float* sx, int T, const int32_t* idx, int C,
                                const convrot_moe_weights& w, uint16_t* a) {
    crk::GemmProblem p{};
    p.A = qx;
    p.a_rows = idx;
    p.a_nrows = T;
    p.a_scale = sx;
    p.M = C;
    p.B = w.q_gu;
    p.b_tiled = true;
    p.b_scale = w.s_gu;
    p.wbits = w.wbits;
    p.N = 2 * w.I;
    p.K = w.d;
    p.E = w.E;
    p.bias = nullptr;
    p.out = a;
    p.epi = crk::Epi::kSwiGLU;
    return p;
}

crk::GemmProblem down_problem(const int8_t* qa, const float* sa, int C, const convrot_moe_weights& w,
                              uint16_t* z) {
    crk::GemmProblem p{};
    p.A = qa;
    p.a_rows = nullptr;
    p.a_nrows = (int64_t)w.E * C;
    p.a_scale = sa;
    p.M = C;
    p.B = w.q_dn;
    p.b_tiled = true;
    p.b_scale = w.s_dn;
    p.wbits = w.wbits;
    p.N = w.d;
    p.K = w.I;
    p.E = w.E;
    p.bias = nullptr;
    p.out = z;
    p.epi = crk::Epi::kBf16;
    return p;
}

#define CRK_TRY(expr)                                   \
    do {                                                \
        const hipError_t crk_e_ = (expr);               \
        if (crk_e_ != hipSuccess) return CONVROT_ERR_HIP; \
    } while (0)

convrot_status check_forward(const uint16_t* x, int T, const float* router_logits, int C,
                              const convrot_moe_weights* w, const uint16_t* out, const int32_t* idx_out,
                              const float* wt_out) {
    if (!x || !router_logits || !out) return CONVROT_ERR_NULL;
    convrot_status st = check_weights(w);
    if (st != CONVROT_OK) return st;
    st = check_tc(T, C, w->E);
    if (st != CONVROT_OK) return st;
    if (!aligned16(x) || !aligned16(router_logits) || !aligned16(out) || (idx_out && !aligned16(idx_out)) ||
        (wt_out && !aligned16(wt_out)))
        return CONVROT_ERR_ALIGN;
    return CONVROT_OK;
}

// The forward's launch sequence on a validated call; ws holds at least plan_moe(T, C, w) bytes.  Every
// workspace byte a launch reads was written by an earlier launch of the same call, so ws need not start
// cleared.
// fused: gate/up, rotate + quantise of the hidden rows and down as one persistent launch (the caller has checked
// that the shapes allow it); else three launches.
convrot_status enqueue_forward(const uint16_t* x, int T, const float* router_logits, int C,
                               const convrot_moe_weights& w, uint16_t* out, int32_t* idx_out, float* wt_out,
                               void* ws, bool fused, hipStream_t stream) {
    MoeBuffers b;
    plan_moe(ws, T, C, w, &b);
    int32_t* idx = idx_out ? idx_out : b.idx;
    float* wt = wt_out ? wt_out : b.wt;
    const int64_t S = (int64_t)w.E * C;

    // The token rotate+quantise does not depend on the routing.  Where the shapes allow, its rows are shared
    // between the softmax launch and the selection launch, both short and latency-bound, so both fill the chip.
    const int64_t t1 = (int64_t)T * kRotqBesideSoftmaxPct / 100;
    const bool split = w.E <= 64 && crk::select_rotq_supported(T, w.E, w.d, w.group_gu);
    if (split) {
        CRK_TRY(crk::launch_softmax_rotq(router_logits, T, w.E, b.probs_t, b.slots, x, w.d, w.group_gu, b.qx, b.sx,
                                         t1, stream));
        CRK_TRY(crk::launch_select_rotq(b.probs_t, T, w.E, C, idx, wt, b.slots, x, w.d, w.group_gu, b.qx,
                                        b.sx, t1, b.esync, stream));
    } else {
        CRK_TRY(crk::launch_softmax_t(router_logits, 0, T, w.E, b.probs_t, nullptr, b.slots, stream));
        CRK_TRY(crk::launch_rotq_act(x, T, w.d, w.group_gu, b.qx, b.sx, nullptr, stream));
        CRK_TRY(crk::launch_select_topc(b.probs_t, T, w.E, C, idx, wt, b.slots, b.esync, stream));
    }
    const crk::GemmProblem gu = gateup_problem(b.qx, b.sx, T, idx, C, w, b.a);
    const crk::GemmProblem dn = down_problem(b.qa, b.sa, C, w, b.z);
    if (fused) {
        CRK_TRY(crk::launch_moe_experts(gu, dn, b.a, b.qa, b.sa, w.group_dn, b.esync, stream));
    } else {
        CRK_TRY(crk::launch_grouped_gemm(gu, stream));
        CRK_TRY(crk::launch_rotq_act(b.a, S, w.I, w.group_dn, b.qa, b.sa, nullptr, stream));
        CRK_TRY(crk::launch_grouped_gemm(dn, stream));
    }
    CRK_TRY(crk::launch_combine(b.z, b.slots, wt, T, w.E, C, w.d, out, stream));
    return CONVROT_OK;
}

// Scratch of the allocation-free forward: one array per GPU, allocated with the code object when the library
// is loaded on that GPU and held until the process ends.  Its name is a host-side stand-in; host code uses
// only the device address that hipGetSymbolAddress returns for the current device, looked up once per device.
static __device__ __align__(256) __attribute__((used)) unsigned char scratch[CONVROT_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

hipError_t scratch_of_current_device(void** out) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!ptr) {
        // several threads may race here; each stores the same address
        err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (!ptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
    *out = ptr;
    return hipSuccess;
}

}  // namespace

extern "C" {

const char* convrot_status_str(convrot_status s) {
    switch (s) {
        case CONVROT_OK: return "CONVROT_OK";
        case CONVROT_ERR_NULL: return "CONVROT_ERR_NULL: required pointer is NULL";
        case CONVROT_ERR_SHAPE: return "CONVROT_ERR_SHAPE: size out of range or inconsistent";
        case CONVROT_ERR_GROUP: return "CONVROT_ERR_GROUP: rotation group must be 64 or 256 and divide the dimension";
        case CONVROT_ERR_BITS: return "CONVROT_ERR_BITS: weight bits must be 8 or 4";
        case CONVROT_ERR_ALIGN: return "CONVROT_ERR_ALIGN: pointer not 16-byte aligned";
        case CONVROT_ERR_WORKSPACE: return "CONVROT_ERR_WORKSPACE: workspace missing or too small";
        case CONVROT_ERR_NONFINITE: return "CONVROT_ERR_NONFINITE: non-finite weight";
        case CONVROT_ERR_HIP: return "CONVROT_ERR_HIP: HIP launch or runtime failure";
    }
    return "CONVROT_ERR_UNKNOWN";
}

size_t convrot_weight_bytes(int E, int N, int K, int bits, int layout) {
    if (E < 1 || N < 1 || K < 1 || (bits != 8 && bits != 4)) return 0;
    const size_t rows = layout == CONVROT_LAYOUT_MFMA ? (size_t)((N + 31) / 32) * 32 : (size_t)N;
    return (size_t)E * rows * (size_t)K * (size_t)bits / 8;
}

convrot_status convrot_quantize_weights(const uint16_t* w, int E, int N, int K, int group, int bits, int layout,
                                        void* q_out, float* scale_out, hipStream_t stream) {
    if (!w || !q_out || !scale_out) return CONVROT_ERR_NULL;
    if (bits != 8 && bits != 4) return CONVROT_ERR_BITS;
    if (layout != CONVROT_LAYOUT_ROWMAJOR && layout != CONVROT_LAYOUT_MFMA) return CONVROT_ERR_SHAPE;
    if (E < 1 || N < 1 || K < 1 || K > kMaxRowLen) return CONVROT_ERR_SHAPE;
    if ((int64_t)E * ((N + 31) / 32) * 32 > (int64_t)4 * INT32_MAX) return CONVROT_ERR_SHAPE;
    if (!group_ok(group) || K % group) return CONVROT_ERR_GROUP;
    if (!aligned16(w) || !aligned16(q_out) || !aligned16(scale_out)) return CONVROT_ERR_ALIGN;
    const int64_t rows = (int64_t)E * N;
    CRK_TRY(crk::launch_rotq_weights(w, E, N, K, group, bits, layout == CONVROT_LAYOUT_MFMA, q_out, scale_out,
                                     stream));
    // Rows holding NaN/Inf come back with a NaN scale; report them (the converter is offline, so it may wait).
    std::vector<float> s((size_t)rows);
    CRK_TRY(hipMemcpyAsync(s.data(), scale_out, sizeof(float) * (size_t)rows, hipMemcpyDeviceToHost, stream));
    CRK_TRY(hipStreamSynchronize(stream));
    for (float v : s)
        if (!std::isfinite(v)) return CONVROT_ERR_NONFINITE;
    return CONVROT_OK;
}

convrot_status convrot_requantize_lora(const int8_t* q_in, const float* s_in, int E, int N, int K, int group,
                                       const uint16_t* lora_b, const uint16_t* lora_a, int rank, float alpha,
                                       uint64_t seed, int rounding, int layout, int8_t* q_out, float* s_out,
                                       hipStream_t stream) {
    if (!q_in || !s_in || !q_out || !s_out) return CONVROT_ERR_NULL;
    if (rounding != CONVROT_ROUND_RANDOM && rounding != CONVROT_ROUND_NEAREST) return CONVROT_ERR_SHAPE;
    if (rank < 0 || rank > 4096) return CONVROT_ERR_SHAPE;
    if (rank > 0 && (!lora_b || !lora_a)) return CONVROT_ERR_NULL;
    if (layout != CONVROT_LAYOUT_ROWMAJOR && layout != CONVROT_LAYOUT_MFMA) return CONVROT_ERR_SHAPE;
    if (E < 1 || N < 1 || K < 1 || K > kMaxRowLen || !std::isfinite(alpha)) return CONVROT_ERR_SHAPE;
    if ((int64_t)E * ((N + 31) / 32) * 32 > (int64_t)4 * INT32_MAX) return CONVROT_ERR_SHAPE;
    if (!group_ok(group) || K % group) return CONVROT_ERR_GROUP;
    if (!aligned16(q_in) || !aligned16(q_out) || (rank > 0 && !aligned16(lora_a)) ||
        (reinterpret_cast<uintptr_t>(s_in) & 3) || (reinterpret_cast<uintptr_t>(s_out) & 3) ||
        (rank > 0 && (reinterpret_cast<uintptr_t>(lora_b) & 1)))
        return CONVROT_ERR_ALIGN;
    return hip_status(crk::launch_requantize_lora(q_in, s_in, E, N, K, group, lora_b, lora_a, rank, alpha, seed,
                                                  rounding == CONVROT_ROUND_NEAREST, layout == CONVROT_LAYOUT_MFMA,
                                                  q_out, s_out, stream));
}

size_t convrot_linear_workspace_bytes(int M, int K) {
    if (M < 1 || K < 1) return 0;
    Carver cv(nullptr);
    cv.take<int8_t>((size_t)M * K);
    cv.take<float>((size_t)M);
    return cv.used;
}

convrot_status convrot_linear_w8a8(const uint16_t* x, int M, int K, const int8_t* qw, const float* sw, int N,
                                   int group, const uint16_t* bias, uint16_t* y, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
    if (!x || !qw || !sw || !y) return CONVROT_ERR_NULL;
    if (M < 1 || N < 1 || K < 1 || K > kMaxRowLen) return CONVROT_ERR_SHAPE;
    if (!group_ok(group) || K % group) return CONVROT_ERR_GROUP;
    if (!aligned16(x) || !aligned16(qw) || !aligned16(sw) || !aligned16(y) || (bias && !aligned16(bias)))
        return CONVROT_ERR_ALIGN;
    if (!ws || ws_bytes < convrot_linear_workspace_bytes(M, K)) return CONVROT_ERR_WORKSPACE;
    if (!aligned16(ws)) return CONVROT_ERR_ALIGN;
    Carver cv(ws);
    int8_t* qx = cv.take<int8_t>((size_t)M * K);
    float* sx = cv.take<float>((size_t)M);
    CRK_TRY(crk::launch_rotq_act(x, M, K, group, qx, sx, nullptr, stream));
    return convrot_gemm_w8a8_bf16(qx, sx, M, K, qw, sw, N, bias, y, stream);
}

convrot_status convrot_gemm_w8a8_bf16(const int8_t* qx, const float* sx, int M, int K, const int8_t* qw,
                                      const float* sw, int N, const uint16_t* bias, uint16_t* y,
                                      hipStream_t stream) {
    if (!qx || !sx || !qw || !sw || !y) return CONVROT_ERR_NULL;
    if (M < 1 || N < 1 || K < 64 || K > kMaxRowLen || K % 64) return CONVROT_ERR_SHAPE;
    if (!aligned16(qx) || !aligned16(sx) || !aligned16(qw) || !aligned16(sw) || !aligned16(y) ||
        (bias && !aligned16(bias)))
        return CONVROT_ERR_ALIGN;
    crk::GemmProblem p{};
    p.A = qx;
    p.a_rows = nullptr;
    p.a_nrows = M;
    p.a_scale = sx;
    p.M = M;
    p.B = qw;
    p.b_tiled = true;
    p.b_scale = sw;
    p.wbits = 8;
    p.N = N;
    p.K = K;
    p.E = 1;
    p.bias = bias;
    p.out = y;
    p.epi = crk::Epi::kBf16;
    return hip_status(crk::launch_grouped_gemm(p, stream));
}

size_t convrot_weight_g16_bytes(int N, int K, int bits) {
    if (N < 1 || K < 1 || (bits != 4 && bits != 6)) return 0;
    return (size_t)N * (size_t)K * (size_t)bits / 8;
}

convrot_status convrot_quantize_weights_g16(const uint16_t* w, int N, int K, int group, int bits, uint8_t* q_out,
                                            uint8_t* f8_out, float* s_out, hipStream_t stream) {
    if (!w || !q_out || !f8_out || !s_out) return CONVROT_ERR_NULL;
    if (bits != 4 && bits != 6) return CONVROT_ERR_BITS;
    if (!group_ok(group) || K < group || K % group) return CONVROT_ERR_GROUP;
    if (N < 1 || K > kMaxRowLen) return CONVROT_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(q_out) || !aligned16(f8_out) || !aligned16(s_out)) return CONVROT_ERR_ALIGN;
    CRK_TRY(crk::launch_quantize_g16(w, N, K, group, bits, q_out, f8_out, s_out, stream));
    return CONVROT_OK;
}

convrot_status convrot_gemm_g16_bf16(const int8_t* qx, const float* sx, int M, int K, const uint8_t* qw,
                                     const uint8_t* f8, const float* s_row, int N, int bits, const uint16_t* bias,
                                     uint16_t* y, hipStream_t stream) {
    if (!qx || !sx || !qw || !f8 || !s_row || !y) return CONVROT_ERR_NULL;
    if (bits != 4 && bits != 6) return CONVROT_ERR_BITS;
    if (M < 1 || N < 1 || K < 64 || K > kMaxRowLen || K % 64 || (M + 255) / 256 > 65535) return CONVROT_ERR_SHAPE;
    if (!aligned16(qx) || !aligned16(sx) || !aligned16(qw) || !aligned16(f8) || !aligned16(s_row) ||
        !aligned16(y) || (bias && !aligned16(bias)))
        return CONVROT_ERR_ALIGN;
    CRK_TRY(crk::launch_gemm_g16(qx, sx, M, K, qw, f8, s_row, N, bits, bias, y, stream));
    return CONVROT_OK;
}

convrot_status convrot_linear_g16(const uint16_t* x, int M, int K, const uint8_t* qw, const uint8_t* f8,
                                  const float* s_row, int N, int group, int bits, const uint16_t* bias, uint16_t* y,
                                  void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!x || !qw || !f8 || !s_row || !y) return CONVROT_ERR_NULL;
    if (bits != 4 && bits != 6) return CONVROT_ERR_BITS;
    if (M < 1 || N < 1 || K < 1 || K > kMaxRowLen || (M + 255) / 256 > 65535) return CONVROT_ERR_SHAPE;
    if (!group_ok(group) || K % group) return CONVROT_ERR_GROUP;  // also makes K a multiple of 64
    if (!aligned16(x) || !aligned16(qw) || !aligned16(f8) || !aligned16(s_row) || !aligned16(y) ||
        (bias && !aligned16(bias)))
        return CONVROT_ERR_ALIGN;
    if (!ws || ws_bytes < convrot_linear_workspace_bytes(M, K)) return CONVROT_ERR_WORKSPACE;
    if (!aligned16(ws)) return CONVROT_ERR_ALIGN;
    Carver cv(ws);
    int8_t* qx = cv.take<int8_t>((size_t)M * K);
    float* sx = cv.take<float>((size_t)M);
    CRK_TRY(crk::launch_rotq_act(x, M, K, group, qx, sx, nullptr, stream));
    CRK_TRY(crk::launch_gemm_g16(qx, sx, M, K, qw, f8, s_row, N, bits, bias, y, stream));
    return CONVROT_OK;
}

int moe_expert_choice_fused(const convrot_moe_weights* w, int C) {
    if (!w || C < 1 || w->E < 1 || w->d < 1 || w->I < 1) return 0;
    if (w->wbits != 8 && w->wbits != 4) return 0;
    if ((int64_t)w->E * C > INT32_MAX || (int64_t)w->E * 2 * w->I > INT32_MAX) return 0;
    return crk::moe_experts_supported(gateup_problem(nullptr, nullptr, C, nullptr, C, *w, nullptr),
                                      down_problem(nullptr, nullptr, C, *w, nullptr), w->group_dn)
               ? 1
               : 0;
}

size_t moe_expert_choice_workspace_bytes(int T, int C, const convrot_moe_weights* w) {
    if (!w || T < 1 || C < 1 || w->E < 1 || w->d < 1 || w->I < 1) return 0;
    return plan_moe(nullptr, T, C, *w, nullptr);
}

convrot_status moe_expert_choice_forward(const uint16_t* x, int T, const float* router_logits, int C,
                                         const convrot_moe_weights* w, uint16_t* out, int32_t* idx_out,
                                         float* wt_out, void* ws, size_t ws_bytes, hipStream_t stream) {
    const convrot_status st = check_forward(x, T, router_logits, C, w, out, idx_out, wt_out);
    if (st != CONVROT_OK) return st;
    if (!ws || ws_bytes < plan_moe(nullptr, T, C, *w, nullptr)) return CONVROT_ERR_WORKSPACE;
    if (!aligned16(ws)) return CONVROT_ERR_ALIGN;
    return enqueue_forward(x, T, router_logits, C, *w, out, idx_out, wt_out, ws, false, stream);
}

convrot_status moe_expert_choice_forward_fused(const uint16_t* x, int T, const float* router_logits, int C,
                                               const convrot_moe_weights* w, uint16_t* out, int32_t* idx_out,
                                               float* wt_out, void* ws, size_t ws_bytes, hipStream_t stream) {
    const convrot_status st = check_forward(x, T, router_logits, C, w, out, idx_out, wt_out);
    if (st != CONVROT_OK) return st;
    if (!moe_expert_choice_fused(w, C)) return CONVROT_ERR_SHAPE;
    if (!ws || ws_bytes < plan_moe(nullptr, T, C, *w, nullptr)) return CONVROT_ERR_WORKSPACE;
    return enqueue_forward(x, T, router_logits, C, *w, out, idx_out, wt_out, ws, true, stream);
}

convrot_status moe_expert_choice_forward_noalloc(const uint16_t* x, int T, const float* router_logits, int C,
                                                 const convrot_moe_weights* w, uint16_t* out, int32_t* idx_out,
                                                 float* wt_out, hipStream_t stream) {
    const convrot_status st = check_forward(x, T, router_logits, C, w, out, idx_out, wt_out);
    if (st != CONVROT_OK) return st;
    if (plan_moe(nullptr, T, C, *w, nullptr) > CONVROT_NOALLOC_SCRATCH_BYTES) return CONVROT_ERR_WORKSPACE;
    void* ws = nullptr;
    if (scratch_of_current_device(&ws) != hipSuccess) return CONVROT_ERR_HIP;
    return enqueue_forward(x, T, router_logits, C, *w, out, idx_out, wt_out, ws, false, stream);
}

convrot_status convrot_rotq_rows(const uint16_t* x, int64_t rows, int K, int group, int8_t* q_out, float* s_out,
                                 float* rot_out, hipStream_t stream) {
    if (rows < 0 || K < 1 || K > kMaxRowLen) return CONVROT_ERR_SHAPE;
    if (rows > (int64_t)4 * INT32_MAX) return CONVROT_ERR_SHAPE;
    if (!group_ok(group) || K % group) return CONVROT_ERR_GROUP;
    if (rows == 0) return CONVROT_OK;  // nothing to do; empty buffers may be NULL
    if (!x || !q_out || !s_out) return CONVROT_ERR_NULL;
    if (!aligned16(x) || !aligned16(q_out) || !aligned16(s_out) || (rot_out && !aligned16(rot_out)))
        return CONVROT_ERR_ALIGN;
    return hip_status(crk::launch_rotq_act(x, rows, K, group, q_out, s_out, rot_out, stream));
}

convrot_status convrot_quantize_prerotated(const float* r, int64_t rows, int K, int bits, int8_t* q_out,
                                           float* s_out, hipStream_t stream) {
    if (bits != 8 && bits != 4) return CONVROT_ERR_BITS;
    if (rows < 0 || K < 8 || K > kMaxRowLen || K % 8) return CONVROT_ERR_SHAPE;
    if (rows > (int64_t)4 * INT32_MAX) return CONVROT_ERR_SHAPE;
    if (rows == 0) return CONVROT_OK;
    if (!r || !q_out || !s_out) return CONVROT_ERR_NULL;
    if (!aligned16(r) || !aligned16(q_out) || !aligned16(s_out)) return CONVROT_ERR_ALIGN;
    return hip_status(crk::launch_quantize_prerotated(r, rows, K, bits, q_out, s_out, stream));
}

convrot_status convrot_gemm_i8_i32(const int8_t* a, const int8_t* b, int M, int N, int K, int32_t* acc_out,
                                   hipStream_t stream) {
    if (!a || !b || !acc_out) return CONVROT_ERR_NULL;
    if (M < 1 || N < 1 || K < 16 || K % 16 || K > kMaxKInt32) return CONVROT_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(b) || !aligned16(acc_out)) return CONVROT_ERR_ALIGN;
    crk::GemmProblem p{};
    p.A = a;
    p.a_rows = nullptr;
    p.a_nrows = M;
    p.a_scale = nullptr;
    p.M = M;
    p.B = b;
    p.b_tiled = false;
    p.b_scale = nullptr;
    p.wbits = 8;
    p.N = N;
    p.K = K;
    p.E = 1;
    p.bias = nullptr;
    p.out = acc_out;
    p.epi = crk::Epi::kI32;
    return hip_status(crk::launch_grouped_gemm(p, stream));
}

size_t moe_route_workspace_bytes(int T, int E) {
    if (T < 1 || E < 1) return 0;
    Carver cv(nullptr);
    cv.take<float>((size_t)E * T);
    return cv.used;
}

convrot_status moe_route_expert_choice(const float* in, int is_probs, int T, int E, int C, int32_t* idx_out,
                                       float* wt_out, float* probs_out, void* ws, size_t ws_bytes,
                                       hipStream_t stream) {
    if (!in || !idx_out || !wt_out) return CONVROT_ERR_NULL;
    convrot_status st = check_tc(T, C, E);
    if (st != CONVROT_OK) return st;
    if (!aligned16(in) || !aligned16(idx_out) || !aligned16(wt_out) || (probs_out && !aligned16(probs_out)))
        return CONVROT_ERR_ALIGN;
    if (!ws || ws_bytes < moe_route_workspace_bytes(T, E)) return CONVROT_ERR_WORKSPACE;
    if (!aligned16(ws)) return CONVROT_ERR_ALIGN;
    float* probs_t = static_cast<float*>(ws);
    CRK_TRY(crk::launch_softmax_t(in, is_probs ? 1 : 0, T, E, probs_t, probs_out, nullptr, stream));
    CRK_TRY(crk::launch_select_topc(probs_t, T, E, C, idx_out, wt_out, nullptr, nullptr, stream));
    return CONVROT_OK;
}

convrot_status moe_gateup_swiglu(const int8_t* qx, const float* sx, int T, const int32_t* idx, int C,
                                 const convrot_moe_weights* w, uint16_t* a_out, hipStream_t stream) {
    if (!qx || !sx || !idx || !a_out) return CONVROT_ERR_NULL;
    convrot_status st = check_weights(w);
    if (st != CONVROT_OK) return st;
    st = check_tc(T, C, w->E);
    if (st != CONVROT_OK) return st;
    if (!aligned16(qx) || !aligned16(sx) || !aligned16(idx) || !aligned16(a_out)) return CONVROT_ERR_ALIGN;
    return hip_status(crk::launch_grouped_gemm(gateup_problem(qx, sx, T, idx, C, *w, a_out), stream));
}

convrot_status moe_down_proj(const int8_t* qa, const float* sa, int C, const convrot_moe_weights* w,
                             uint16_t* z_out, hipStream_t stream) {
    if (!qa || !sa || !z_out) return CONVROT_ERR_NULL;
    convrot_status st = check_weights(w);
    if (st != CONVROT_OK) return st;
    if (C < 1 || (int64_t)w->E * C > INT32_MAX) return CONVROT_ERR_SHAPE;
    if (!aligned16(qa) || !aligned16(sa) || !aligned16(z_out)) return CONVROT_ERR_ALIGN;
    return hip_status(crk::launch_grouped_gemm(down_problem(qa, sa, C, *w, z_out), stream));
}

size_t moe_combine_workspace_bytes(int T, int E) {
    if (T < 1 || E < 1) return 0;
    Carver cv(nullptr);
    cv.take<int32_t>((size_t)T * E);
    return cv.used;
}

convrot_status moe_combine(const uint16_t* z, const int32_t* idx, const float* wt, int T, int E, int C, int d,
                           uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!z || !idx || !wt || !out) return CONVROT_ERR_NULL;
    convrot_status st = check_tc(T, C, E);
    if (st != CONVROT_OK) return st;
    if (d < 8 || d % 8 || d > kMaxRowLen) return CONVROT_ERR_SHAPE;
    if (!aligned16(z) || !aligned16(idx) || !aligned16(wt) || !aligned16(out)) return CONVROT_ERR_ALIGN;
    if (!ws || ws_bytes < moe_combine_workspace_bytes(T, E)) return CONVROT_ERR_WORKSPACE;
    if (!aligned16(ws)) return CONVROT_ERR_ALIGN;
    Carver cv(ws);
    int32_t* slots = cv.take<int32_t>((size_t)T * E);
    CRK_TRY(crk::launch_build_slots(idx, T, E, C, slots, stream));
    CRK_TRY(crk::launch_combine(z, slots, wt, T, E, C, d, out, stream));
    return CONVROT_OK;
}

}  // extern "C"
