// Internal launchers of libconvrot_amd (host side).  Arguments are validated by the C-ABI layer before any
// of these is called; each launcher only enqueues on `st` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace crk {

// ---- rotate + quantise --------------------------------------------------------------------------------
hipError_t launch_rotq_act(const uint16_t* x, int64_t rows, int K, int group, int8_t* q, float* s, float* rot,
                           hipStream_t st);
// Weights [E, N, K]: row-major codes, or the MFMA-tiled layout when `tiled` (rows padded to blocks of 32).
// LoRA patch of row-major int8 weights [E, N, K], re-quantised with random or nearest rounding (int8,
// row-major or tiled)
hipError_t launch_requantize_lora(const int8_t* qin, const float* sin, int E, int N, int K, int group,
                                  const uint16_t* lb, const uint16_t* la, int rank, float alpha, uint64_t seed,
                                  bool nearest, bool tiled, int8_t* qout, float* sout, hipStream_t st);
// W6A8 / W4A8 with E4M3 group-16 scales: converter (row-major packing) and GEMM + dequant
hipError_t launch_quantize_g16(const uint16_t* w, int N, int K, int group, int bits, uint8_t* q, uint8_t* f8,
                               float* s_row, hipStream_t st);
hipError_t launch_gemm_g16(const int8_t* qx, const float* sx, int M, int K, const uint8_t* qw, const uint8_t* f8,
                           const float* s_row, int N, int bits, const uint16_t* bias, uint16_t* y, hipStream_t st);
hipError_t launch_rotq_weights(const uint16_t* w, int E, int N, int K, int group, int bits, bool tiled, void* q,
                               float* s, hipStream_t st);
hipError_t launch_quantize_prerotated(const float* r, int64_t rows, int K, int bits, int8_t* q, float* s,
                                      hipStream_t st);

// ---- routing ------------------------------------------------------------------------------------------
// probs^T [E, T] from logits [T, E] (or a transpose of given probabilities); optional probs [T, E] copy.
// slots [T, E] (or nullptr): the slot table (slots[t, e] = position of token t in expert e's list, or -1), its
// rows filled with -1 for the selection that follows.
hipError_t launch_softmax_t(const float* in, int is_probs, int T, int E, float* probs_t, float* probs_out,
                            int32_t* slots, hipStream_t st);
// Router softmax (E <= 64, logits) and token rotate+quantise (fast shapes) in one launch; returns
// hipErrorNotSupported, having launched nothing, for other shapes.
// softmax of all T tokens and rotate+quantise of token rows [0, rows) in one launch
hipError_t launch_softmax_rotq(const float* logits, int T, int E, float* probs_t, int32_t* slots,
                               const uint16_t* x, int K, int group, int8_t* qx, float* sx, int64_t rows,
                               hipStream_t st);
// Per expert: top-C selection on probs_t[e, :]; writes idx [E, C], wt [E, C] and, if slots != nullptr, the
// slot-table entries of the tokens it takes (the table must hold -1 elsewhere, as the softmax leaves it).
// selection of all E experts and rotate+quantise of token rows [row0, T) in one launch
bool select_rotq_supported(int T, int E, int K, int group);
hipError_t launch_select_rotq(const float* probs_t, int T, int E, int C, int32_t* idx, float* wt, int32_t* slots,
                              const uint16_t* x, int K, int group, int8_t* qx, float* sx, int64_t row0,
                              uint32_t* esync, hipStream_t st);
// esync (nullable): the 2E counters of launch_moe_experts, zeroed by the selection of each expert.
hipError_t launch_select_topc(const float* probs_t, int T, int E, int C, int32_t* idx, float* wt,
                              int32_t* slots, uint32_t* esync, hipStream_t st);
// The slot table [T, E] of the lists idx [E, C] (-1 where a token is in no list; entries outside [0, T)
// ignored).
hipError_t launch_build_slots(const int32_t* idx, int T, int E, int C, int32_t* slots, hipStream_t st);

// ---- grouped INT8 GEMM --------------------------------------------------------------------------------
enum class Epi : int { kI32 = 0, kBf16 = 1, kSwiGLU = 2 };

struct GemmProblem {
    const int8_t* A;        // activation codes, rows of K bytes
    const int32_t* a_rows;  // [E * M] row index into A per (expert, slot), or nullptr: row = e * M + m
    int64_t a_nrows;        // rows of A (gathered indices are clamped into [0, a_nrows))
    const float* a_scale;   // per A row (indexed like A), unused for kI32
    int M;                  // rows per expert (C for the MoE, M for a plain GEMM)
    const void* B;          // [E, N, K] codes: MFMA-tiled (b_tiled, int8 or int4) or row-major int8
    bool b_tiled;
    const float* b_scale;   // [E, N], unused for kI32
    int wbits;              // 8 or 4
    int N;                  // output columns of B (2I for gate/up)
    int K;
    int E;
    const uint16_t* bias;   // [N] bf16 or nullptr (kBf16 only)
    void* out;              // kI32: int32 [E*M, N]; kBf16: bf16 [E*M, N]; kSwiGLU: bf16 [E*M, N/2]
    Epi epi;
};
hipError_t launch_grouped_gemm(const GemmProblem& p, hipStream_t st);

// Counters of launch_moe_experts sit kEsyncStride words apart (one 256-byte line each): counter k (gate/up tiles
// of expert e at k = 2 e, rotate + quantise items at k = 2 e + 1) is esync[k * kEsyncStride].
constexpr int kEsyncStride = 64;

// The expert part of the MoE layer in one persistent launch: the gate/up GEMM gu (kSwiGLU, writing a), the
// rotate + quantise of a's rows (rotation group `group`, I = gu.N / 2 columns) into qa / sa, and the down GEMM
// dn (kBf16, reading qa / sa as its rows e * C + c), with per-expert dependencies through esync (2 gu.E
// counters kEsyncStride words apart, zero at the start).  hipErrorNotSupported: shape outside the fused kernels, use the three launches.
hipError_t launch_moe_experts(const GemmProblem& gu, const GemmProblem& dn, const uint16_t* a, int8_t* qa, float* sa,
                              int group, uint32_t* esync, hipStream_t st);
// Whether launch_moe_experts takes these problems (host logic only).
bool moe_experts_supported(const GemmProblem& gu, const GemmProblem& dn, int group);

// ---- combine ------------------------------------------------------------------------------------------
hipError_t launch_combine(const uint16_t* z, const int32_t* slots, const float* wt, int T, int E, int C, int d,
                          uint16_t* out, hipStream_t st);

}  // namespace crk
