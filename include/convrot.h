/*
 * convrot.h -- C ABI of the MI355X (gfx950) W8A8 ConvRot expert-choice MoE library (libconvrot_amd.so).
 *
 * What is computed (pages cited by title and section):
 *  - "Nucleus-Image INT8 Convrot Experts + FP8 Text Encoder" model card, "Quantization": each routed-expert
 *    matrix is rotated with ConvRot (a block Hadamard rotation along the input dimension; group 256 for the
 *    gate/up projection, 64 for the down projection), quantised to symmetric INT8 with nearest rounding and
 *    one FP32 scale per output row, and run through W8A8 ConvRot linears with BF16 outputs.
 *  - "NitroFusion2 for ComfyUI: int8, W6A8, W4A8", "How they were made": the int8 format is that block
 *    Hadamard rotation, one scale per row and 8-bit activations; rotation and rounding happen in fp32.
 *  - "MLX Nucleus-Image", overview and "Conversion notes": 64 routed experts with expert-choice routing (each
 *    expert picks its top-C tokens and the outputs are scattered back to the tokens); the expert SwiGLU is
 *    silu(gate) * up with the first half of the fused projection the gate.
 *  - "XB_UNetLoaderINTROCm", "The mechanism, briefly": multiply in INT8, dequantise on the fly.
 *
 * Numerics (identical on every entry point):
 *  - Rotation: per contiguous block of g values along K, v -> v . H_g / sqrt(g) with H_g the Sylvester
 *    Hadamard matrix in natural order, evaluated in fp32 as the fast transform with stages h = 1, 2, ..., g/2
 *    (pair (j, j+h) -> (a + b, a - b)) and then the exact power-of-two scale.  g is 64 or 256.
 *  - Quantiser, per row over all K: scale = max|r| / qmax (fp32 division), code = clamp(rint(r / scale),
 *    -qmax, qmax) (fp32 division, ties to even); scale 0 gives codes 0.  qmax = 127 (INT8) or 7 (INT4).
 *    Activations get one scale per token (row) computed from the call's own data.
 *  - Product: exact INT32 sum of INT8 x INT8 (|acc| <= K * 127^2, so K <= 133144).
 *  - Dequantisation: bf16_rne( ((float)acc * s_act) * s_w ) [+ (float)bias, added before the rounding].
 *  - SwiGLU: a = bf16_rne( silu(g) * u ), silu(g) = g / (1 + E(-g)) (g * E(g) for g < -64, where 1 + E(g)
 *    is exactly 1), g and u the bf16 gate/up outputs.
 *  - Router: p[t, :] = softmax over experts in fp32 (max-subtracted, E() of the differences, sum in ascending
 *    expert order, one division per entry).  Expert e takes the C tokens with the largest p[:, e], ties to the
 *    lower token index, listed in ascending token order; its gate weight is that p (not renormalised).
 *  - Combine: out[t, :] = bf16_rne( sum over experts e in ascending order that took t of w * (float)z ),
 *    fp32, starting from +0.0f; a token taken by no expert gets +0.
 *  - E(x) is a fixed fp32 exponential: x clamped to [-150, 100]; n = rint(x * log2e); r = fma(-n, ln2_lo,
 *    fma(-n, ln2_hi, x)) with ln2_hi = ln 2 rounded to 16 significant bits (Cody-Waite reduction); Taylor
 *    series of e^r through r^7 by Horner's rule in fused multiply-adds (coefficients 1/k! rounded to fp32);
 *    p * 2^n rounded once (exact when normal), so E underflows through the subnormals to 0 and overflows to
 *    +inf where the fp32 rounding of e^x does.  Every other fp32 step above is a separate IEEE operation (no contraction), so
 *    results are reproducible bit for bit.
 *
 * Conventions for every call:
 *  - Pointers marked (device) are device memory on the current HIP device; bf16 crosses the ABI as raw
 *    uint16_t bits.  The caller owns every buffer; the library allocates nothing and keeps no state between
 *    calls beyond what it sets up once (each GEMM kernel's LDS size attribute, and a per-device count of
 *    compute units held in an atomic), so calls are thread-safe.
 *    Calls only enqueue work on `stream` (0 = the null stream) and return.
 *  - Arguments are validated on the host before anything is enqueued; on an error nothing is written.
 *    CONVROT_ERR_HIP means a launch failed after validation; outputs are then unspecified.
 *  - Row strides equal the row length (dense row-major).  Every device pointer must be 16-byte aligned.
 *  - NaN or Inf in activations or logits are outside the contract (no per-call scan); the weight converter
 *    rejects non-finite weights with CONVROT_ERR_NONFINITE.
 */
#ifndef CONVROT_H
#define CONVROT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum convrot_status {
    CONVROT_OK = 0,
    CONVROT_ERR_NULL = 1,       /* a required pointer is NULL */
    CONVROT_ERR_SHAPE = 2,      /* a size is out of range or inconsistent */
    CONVROT_ERR_GROUP = 3,      /* rotation group not 64/256, or the dimension is not a multiple of it */
    CONVROT_ERR_BITS = 4,       /* weight bits not 8 or 4 */
    CONVROT_ERR_ALIGN = 5,      /* a pointer is not 16-byte aligned */
    CONVROT_ERR_WORKSPACE = 6,  /* workspace NULL or smaller than the matching *_workspace_bytes() */
    CONVROT_ERR_NONFINITE = 7,  /* the weight converter found NaN or Inf */
    CONVROT_ERR_HIP = 8         /* a HIP launch or runtime call failed */
} convrot_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* convrot_status_str(convrot_status s);

/* Layouts of quantised weight codes.
 *  CONVROT_LAYOUT_ROWMAJOR: codes of row n, column k at byte n*K + k (int8), or nibble k%2 of byte
 *    n*(K/2) + k/2 (int4; even k in bits 0-3).  Interchange / inspection format.
 *  CONVROT_LAYOUT_MFMA: the format the GEMMs stream.  Rows are grouped in blocks of 32 (NB = ceil(N/32)
 *    blocks, rows past N are zero); every (row block nb, K-block) is one contiguous 1 KiB tile, so that a
 *    wavefront fetches it with one coalesced 16-byte load per lane, laid out so that the gfx950 int8 MFMA
 *    operand fragments (16 rows by 16 consecutive k per lane) are read from LDS free of bank conflicts.
 *    With r = n % 32:
 *      int8 (K-blocks of 32):  byte ((nb*(K/32) + k/32)*1024 + (r + 32*((k%32)/16))*16 + k%16)
 *      int4 (K-blocks of 64):  byte ((nb*(K/64) + k/64)*1024 + (64*(r/16) + 16*((k%64)/16) + r%16)*8
 *                                    + 4*((k%16)/8) + k%4), low nibble if k%8 < 4, else high nibble (each
 *                                    4-byte word: k..k+3 in the low nibbles, k+4..k+7 in the high ones);
 *                                    requires K % 64 == 0.
 *    For [E, N, K] weights expert e starts at byte e * NB * K (int8) or e * NB * K / 2 (int4), i.e. the
 *    buffer holds E * NB * 32 * K (or half that) bytes. */
typedef enum convrot_layout { CONVROT_LAYOUT_ROWMAJOR = 0, CONVROT_LAYOUT_MFMA = 1 } convrot_layout;

/* Bytes of a quantised [E, N, K] weight tensor in the given layout and bit width. */
size_t convrot_weight_bytes(int E, int N, int K, int bits, int layout);

/* Quantised weights of one routed-expert MoE layer.  The struct itself lives in host memory.  Codes are in
 * CONVROT_LAYOUT_MFMA. */
typedef struct convrot_moe_weights {
    int E;             /* routed experts, >= 1 */
    int d;             /* model width (gate/up input, down output), multiple of group_gu */
    int I;             /* expert hidden width (down input), multiple of group_dn and of 64 */
    int group_gu;      /* rotation group of gate/up: 64 or 256 (the pages use 256) */
    int group_dn;      /* rotation group of down: 64 or 256 (the pages use 64) */
    int wbits;         /* 8: int8 codes; 4: nibble-packed int4 codes (even k in bits 0-3) */
    const void* q_gu;  /* (device) [E, 2I, d] codes, MFMA layout; rows 0..I-1 gate, I..2I-1 up */
    const float* s_gu; /* (device) [E, 2I] fp32 per-output-row scales */
    const void* q_dn;  /* (device) [E, d, I] codes, MFMA layout */
    const float* s_dn; /* (device) [E, d] fp32 */
} convrot_moe_weights;

/* ---------------------------------------------------------------------------------------------------- */
/* Offline weight converter  (model card "Quantization": rotate each expert matrix, quantise per row)     */
/* ---------------------------------------------------------------------------------------------------- */

/* w (device) [E, N, K] bf16 -> q_out (device, convrot_weight_bytes(E, N, K, bits, layout) bytes) codes in
 * `layout`, and scale_out (device) [E, N] fp32.  Each row is rotated along K in blocks of `group` and
 * quantised with its own scale (qmax 127 for bits = 8, 7 for bits = 4).  Requires E, N >= 1,
 * 1 <= K <= 8192, K % group == 0.  A non-finite weight makes the call return CONVROT_ERR_NONFINITE after
 * the stream work completes (this call synchronises `stream`); outputs are then unspecified. */
convrot_status convrot_quantize_weights(const uint16_t* w, int E, int N, int K, int group, int bits, int layout,
                                        void* q_out, float* scale_out, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------------- */
/* Single W8A8 ConvRot linear  (model card "Quantization": W8A8 ConvRot linear with BF16 outputs)          */
/* ---------------------------------------------------------------------------------------------------- */

/* Rounding of the LoRA re-quantisation ("XB_UNetLoaderINTROCm", "Inputs that matter": the loader's two LoRA
 * modes).  RANDOM: the stochastic mode, random-rounding the patched values.  NEAREST: the dynamic mode, which
 * re-quantises each patched layer: the weight quantiser's nearest rounding (ties to even). */
typedef enum convrot_rounding { CONVROT_ROUND_RANDOM = 0, CONVROT_ROUND_NEAREST = 1 } convrot_rounding;

/* LoRA patch of quantised weights, re-quantised with fresh scales ("NitroFusion2 for ComfyUI", "Why a
 * step-1 file": a LoRA on a quantised file is re-quantised with fresh scales and random rounding;
 * "XB_UNetLoaderINTROCm", "Inputs that matter": a stochastic LoRA mode bakes LoRAs in at load, a dynamic one
 * re-quantises per layer).
 * q_in (device) [E, N, K] int8 row-major codes and s_in (device) [E, N] scales of weights quantised with
 * `group` (convrot_quantize_weights, CONVROT_LAYOUT_ROWMAJOR, 8 bits); lora_b (device) [E, N, rank] and
 * lora_a (device) [E, rank, K] bf16, the LoRA factors in the original basis (both may be NULL when rank is 0);
 * alpha: the LoRA strength; seed: selects the random stream.  Writes q_out (device) in `layout` (int8;
 * convrot_weight_bytes(E, N, K, 8, layout) bytes) and s_out (device) [E, N].
 * Per row, in the rotated basis: V = (float)q * s + rotate(alpha * lora_b . lora_a) (delta summed over the
 * rank in ascending order in fp32, then rotated like the weights); scale = max|V| / 127; t = V / scale;
 * rounding CONVROT_ROUND_RANDOM: code = floor(t), plus 1 when u < t - floor(t), clamped to +-127, where u is
 * the top 24 bits (times 2^-24) of word k % 4 of Philox4x64-10 (Salmon et al., SC 2011) at counter
 * ((e N + n) K/4 + k/4, 0, 0, 0), key (seed, 0); deterministic for a given seed.  CONVROT_ROUND_NEAREST:
 * code = clamp(rint(t), -127, 127) (seed unused).  A zero row gets scale 0 and codes 0 in both.
 * Requires E, N >= 1, K <= 8192, K % group == 0, group 64 or 256, 0 <= rank <= 4096, alpha finite, rounding
 * one of the two modes (CONVROT_ERR_SHAPE otherwise), q_in, lora_a and q_out 16-byte aligned; errors write
 * nothing. */
convrot_status convrot_requantize_lora(const int8_t* q_in, const float* s_in, int E, int N, int K, int group,
                                       const uint16_t* lora_b, const uint16_t* lora_a, int rank, float alpha,
                                       uint64_t seed, int rounding, int layout, int8_t* q_out, float* s_out,
                                       hipStream_t stream);

/* Bytes of workspace convrot_linear_w8a8 needs for an [M, K] input. */
size_t convrot_linear_workspace_bytes(int M, int K);

/* y[M, N] = bf16( ((float)(rotq(x) . qw^T) * sx) * sw ) (+ bias).  x (device) [M, K] bf16; qw (device)
 * [N, K] int8 codes in CONVROT_LAYOUT_MFMA from convrot_quantize_weights with the same group; sw (device)
 * [N]; bias (device) [N] bf16
 * or NULL; y (device) [M, N] bf16; ws (device) at least convrot_linear_workspace_bytes(M, K).
 * Requires M, N >= 1, K <= 8192, K % group == 0, group 64 or 256. */
convrot_status convrot_linear_w8a8(const uint16_t* x, int M, int K, const int8_t* qw, const float* sw, int N,
                                   int group, const uint16_t* bias, uint16_t* y, void* ws, size_t ws_bytes,
                                   hipStream_t stream);

/* ---------------------------------------------------------------------------------------------------- */
/* Expert-choice MoE layer, routed experts  ("MLX Nucleus-Image": expert-choice, silu(gate) * up)          */
/* ---------------------------------------------------------------------------------------------------- */

/* Bytes of workspace moe_expert_choice_forward needs. */
size_t moe_expert_choice_workspace_bytes(int T, int C, const convrot_moe_weights* w);

/* x (device) [T, d] bf16; router_logits (device) [T, E] fp32; out (device) [T, d] bf16, overwritten;
 * idx_out (device) [E, C] int32 or NULL; wt_out (device) [E, C] fp32 or NULL (the routing decisions);
 * ws (device) at least moe_expert_choice_workspace_bytes(T, C, w).
 * Steps: softmax + top-C per expert; rotate+quantise x (group_gu); grouped INT8 gate/up GEMM over each
 * expert's C gathered tokens with fused dequant + SwiGLU; rotate+quantise the hidden rows (group_dn);
 * grouped INT8 down GEMM with dequant; probability-weighted combine into out.
 * Requires 1 <= C <= T, E >= 1, d % group_gu == 0, I % group_dn == 0, I % 64 == 0, d and I <= 8192. */
convrot_status moe_expert_choice_forward(const uint16_t* x, int T, const float* router_logits, int C,
                                         const convrot_moe_weights* w, uint16_t* out, int32_t* idx_out,
                                         float* wt_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_expert_choice_forward with the hidden rows' rotate+quantise fused with the two grouped GEMMs into one
 * persistent launch ("MLX Nucleus-Image", "Conversion notes": the expert FFN; "Nucleus-Image INT8 Convrot
 * Experts + FP8 Text Encoder", "Quantization": group 64 for the down projection's input).  Same arguments,
 * workspace and results, bit for bit.  The launch runs one workgroup per CU through three phases: the gate/up
 * tiles, then rotate+quantise of the hidden rows of every expert whose gate/up tiles are all done, then the
 * down tiles of every expert whose rows are all done, ordered through per-expert counters in the workspace
 * (a row's scale needs all of its I columns, which come from several CUs, so the quantisation cannot sit in
 * the gate/up epilogue itself).  It needs every one of its workgroups resident at once: a kernel of another
 * stream that holds CUs delays it, and one holding them for more than about a second per wait leaves wrong
 * results (the waits are bounded; the launch always finishes).  Two of these calls must not run concurrently
 * on one GPU (from two streams): each could hold CUs that the other's waiting workgroups need.  On MI355X it
 * is slower than the three launches of moe_expert_choice_forward, whose kernel boundaries cost next to
 * nothing.
 * CONVROT_ERR_SHAPE where moe_expert_choice_fused(w, C) is 0; other errors as moe_expert_choice_forward. */
convrot_status moe_expert_choice_forward_fused(const uint16_t* x, int T, const float* router_logits, int C,
                                               const convrot_moe_weights* w, uint16_t* out, int32_t* idx_out,
                                               float* wt_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* 1 if moe_expert_choice_forward_fused takes a layer with these weights and C, else 0 (also for invalid
 * arguments).  Shapes only; no GPU call: group_dn = 64 with I in {512, 1024, 1536, 2048}, or group_dn = 256
 * with I = 2048, for either weight width. */
int moe_expert_choice_fused(const convrot_moe_weights* w, int C);

/* Size of the static scratch the allocation-free forward uses: 192 MiB per GPU (the T = 8192, C = 256 layer
 * with E = 64, d = 2048, I = 1536 takes 163.8 MB of it). */
#define CONVROT_NOALLOC_SCRATCH_BYTES ((size_t)192 << 20)

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): moe_expert_choice_forward with the workspace taken from a static device array of
 * CONVROT_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on until the process ends.
 * Arguments, steps, results and errors are those of moe_expert_choice_forward; a call whose workspace
 * (moe_expert_choice_workspace_bytes) exceeds the scratch returns CONVROT_ERR_WORKSPACE and writes nothing.
 * The first call on a device looks up that device's scratch address once (a HIP runtime call, no
 * allocation); no call allocates or frees memory.  Every call on one GPU shares that GPU's scratch, which
 * keeps the last call's contents (nothing in it needs to start cleared): calls that overlap on one GPU, from
 * several streams or threads, race and give undefined results. */
convrot_status moe_expert_choice_forward_noalloc(const uint16_t* x, int T, const float* router_logits, int C,
                                                 const convrot_moe_weights* w, uint16_t* out, int32_t* idx_out,
                                                 float* wt_out, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------------- */
/* Stage entry points: each step of the forward on its own, so that every stage can be checked exactly     */
/* given identical inputs.  Same kernels as the forward.                                                   */
/* ---------------------------------------------------------------------------------------------------- */

/* Rotate + quantise rows (activations: qmax 127, one scale per row).  x (device) [rows, K] bf16 ->
 * q_out (device) [rows, K] int8, s_out (device) [rows] fp32, rot_out (device) [rows, K] fp32 rotated
 * values before quantisation, or NULL.  Requires rows >= 0, 1 <= K <= 8192, K % group == 0; rows == 0 is a
 * no-op (pointers may then be NULL). */
convrot_status convrot_rotq_rows(const uint16_t* x, int64_t rows, int K, int group, int8_t* q_out, float* s_out,
                                 float* rot_out, hipStream_t stream);

/* Quantise already-rotated fp32 rows: r (device) [rows, K] -> q_out (device) [rows, K] int8 codes (bits 8:
 * qmax 127; bits 4: qmax 7, unpacked) and s_out (device) [rows].  Requires K % 8 == 0, K <= 8192; rows == 0
 * is a no-op. */
convrot_status convrot_quantize_prerotated(const float* r, int64_t rows, int K, int bits, int8_t* q_out,
                                           float* s_out, hipStream_t stream);

/* acc_out[M, N] = a[M, K] . b[N, K]^T exactly in int32 (both row-major int8), with the same INT8 MFMA main
 * loop as the layer (B fetched row-major instead of tiled).  Requires M, N >= 1, 16 <= K <= 131056,
 * K % 16 == 0 (K * 128^2 < 2^31 for any int8 codes). */
convrot_status convrot_gemm_i8_i32(const int8_t* a, const int8_t* b, int M, int N, int K, int32_t* acc_out,
                                   hipStream_t stream);

/* The linear's GEMM stage on quantised tokens: y[M, N] = bf16( ((float)(qx . qw^T) * sx) * sw ) (+ bias),
 * the second half of convrot_linear_w8a8 ("Nucleus-Image INT8 Convrot Experts", "Quantization": W8A8
 * ConvRot linear with BF16 output; dequantisation as in that entry point).  qx (device) [M, K] int8 codes and
 * sx (device) [M] fp32 scales of the rotated rows (convrot_rotq_rows with the weights' group); qw (device)
 * [N, K] int8 codes in CONVROT_LAYOUT_MFMA; sw (device) [N]; bias (device) [N] bf16 or NULL; y (device)
 * [M, N] bf16.  Requires M, N >= 1, 64 <= K <= 8192, K % 64 == 0. */
convrot_status convrot_gemm_w8a8_bf16(const int8_t* qx, const float* sx, int M, int K, const int8_t* qw,
                                      const float* sw, int N, const uint16_t* bias, uint16_t* y,
                                      hipStream_t stream);

/* ---- W6A8 / W4A8 with an FP8 scale per group of 16 -----------------------------------------------------
 * "NitroFusion2 for ComfyUI: int8, W6A8, W4A8", "How they were made": 6- or 4-bit weights in the rotated
 * basis with an FP8 scale per group of 16, 8-bit activations.  The page fixes only the bit widths, the
 * group size and the scale type; the library reads it as follows.
 *  - Rotation: the block Hadamard above (group 64 or 256 along K), fp32, as for the int8 weights.
 *  - Codes: symmetric integers, qmax = 31 (bits = 6) or 7 (bits = 4), nearest rounding, ties to even.
 *  - Scales: FP8 E4M3 (sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, largest finite 448),
 *    one per 16 consecutive k, relative to one fp32 scale per row (E4M3 cannot hold the absolute group
 *    scales of typical weights):  s_row = amax / (qmax * 448);  f_j = E4M3((amax_j / amax) * 448), nearest
 *    E4M3 value with ties to the even mantissa;  code = clamp(rint(r / (s_row * f_j)), +-qmax), 0 where
 *    s_row * f_j = 0.  Each step is one IEEE fp32 operation in the order written.
 *  - Layouts, row-major: q [N, K/2] (4-bit: two's-complement nibbles, even k in bits 0-3) or [N, 3K/4]
 *    (6-bit: codes 4j..4j+3 of a row in bytes 3j..3j+2, code 4j+i in bits 6i..6i+5 of the little-endian
 *    24-bit word); f8 [N, K/16] E4M3 bytes; s_row [N] fp32.
 *  - Linear: tokens rotated and quantised to int8 per token as for W8A8; then
 *    y[m, n] = bf16( ((float)A[m, n] * sx[m]) * s_row[n] ) (+ bias[n] in fp32), A = sum_k qx[m, k] *
 *    (code[n, k] * f(n, k / 16)).  The kernel accumulates A in fp32 (every product exact), so y differs from
 *    the exactly summed A by the fp32 accumulation error only. */

/* Bytes of the packed codes of an [N, K] weight: N * K * bits / 8. */
size_t convrot_weight_g16_bytes(int N, int K, int bits);

/* Converter: w (device) [N, K] bf16 -> q_out (device, convrot_weight_g16_bytes bytes), f8_out (device)
 * [N, K/16] E4M3, s_out (device) [N] fp32.  Requires N >= 1, group in {64, 256}, K % group == 0,
 * K <= 8192, bits in {4, 6} (CONVROT_ERR_BITS otherwise).  Non-finite weights are outside the contract. */
convrot_status convrot_quantize_weights_g16(const uint16_t* w, int N, int K, int group, int bits, uint8_t* q_out,
                                            uint8_t* f8_out, float* s_out, hipStream_t stream);

/* GEMM stage on quantised tokens qx (device) [M, K] int8 and sx (device) [M] (convrot_rotq_rows with the
 * weights' group): y (device) [M, N] bf16 as above; bias (device) [N] bf16 or NULL.  Requires M, N >= 1,
 * 64 <= K <= 8192, K % 64 == 0, bits in {4, 6}. */
convrot_status convrot_gemm_g16_bf16(const int8_t* qx, const float* sx, int M, int K, const uint8_t* qw,
                                     const uint8_t* f8, const float* s_row, int N, int bits, const uint16_t* bias,
                                     uint16_t* y, hipStream_t stream);

/* The whole linear: x (device) [M, K] bf16; workspace as convrot_linear_workspace_bytes(M, K).  Requires
 * M, N >= 1, group in {64, 256}, K % group == 0, K <= 8192, bits in {4, 6}. */
convrot_status convrot_linear_g16(const uint16_t* x, int M, int K, const uint8_t* qw, const uint8_t* f8,
                                  const float* s_row, int N, int group, int bits, const uint16_t* bias, uint16_t* y,
                                  void* ws, size_t ws_bytes, hipStream_t stream);

/* Bytes of workspace moe_route_expert_choice needs. */
size_t moe_route_workspace_bytes(int T, int E);

/* Router alone.  in (device) [T, E]: logits (is_probs = 0) or probabilities (is_probs = 1, used as given);
 * idx_out (device) [E, C] int32; wt_out (device) [E, C] fp32; probs_out (device) [T, E] or NULL.
 * Requires 1 <= C <= T, E >= 1. */
convrot_status moe_route_expert_choice(const float* in, int is_probs, int T, int E, int C, int32_t* idx_out,
                                       float* wt_out, float* probs_out, void* ws, size_t ws_bytes,
                                       hipStream_t stream);

/* Gate/up stage: for every expert e and slot c, token t = idx[e, c]:
 * a_out[e*C + c, :] = SwiGLU of the dequantised gate/up product of qx[t] (device [T, d] int8, scale
 * sx[t], device [T] fp32) with expert e.  idx (device) [E, C] with entries in [0, T); a_out (device)
 * [E*C, I] bf16. */
convrot_status moe_gateup_swiglu(const int8_t* qx, const float* sx, int T, const int32_t* idx, int C,
                                 const convrot_moe_weights* w, uint16_t* a_out, hipStream_t stream);

/* Down stage: z_out[e*C + c, :] = bf16(dequant(qa[e*C + c] . q_dn[e]^T)).  qa (device) [E*C, I] int8,
 * sa (device) [E*C] fp32, z_out (device) [E*C, d] bf16. */
convrot_status moe_down_proj(const int8_t* qa, const float* sa, int C, const convrot_moe_weights* w,
                             uint16_t* z_out, hipStream_t stream);

/* Bytes of workspace moe_combine needs (the slot table [T, E] int32: each token's position in each list). */
size_t moe_combine_workspace_bytes(int T, int E);

/* Combine stage: out[T, d] from z (device) [E*C, d] bf16, idx (device) [E, C] (each row strictly
 * ascending, entries in [0, T)) and wt (device) [E, C]. */
convrot_status moe_combine(const uint16_t* z, const int32_t* idx, const float* wt, int T, int E, int C, int d,
                           uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CONVROT_H */
