/*
 * CPU oracle for the W8A8 ConvRot linear and the expert-choice MoE layer built on it.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this file's library.  The product path (the HIP library and its Python binding) never calls
 * it, shares no code, header, table or constant generator with it, and fails loudly when its own
 * extension is missing.
 *
 * Plain, slow, obviously-correct loops.  Every floating-point step that the method specifies is done in
 * IEEE fp32 with round-to-nearest-even, as separate operations (built with -ffp-contract=off, no fast
 * math), in the order written here.  Integer work is exact.
 *
 * Sources (pages, cited by title and section):
 *  [NUC]  "Nucleus-Image INT8 Convrot Experts + FP8 Text Encoder" model card, section "Quantization":
 *         routed experts are rotated with ConvRot, then quantised to symmetric INT8 with nearest
 *         rounding and one FP32 scale per output row; rotation groups are 256 for gate/up and 64 for
 *         down; inference runs W8A8 ConvRot linears that emit BF16.
 *  [NF2]  "NitroFusion2 for ComfyUI: int8, W6A8, W4A8", section "How they were made": int8 is a block
 *         Hadamard rotation (ConvRot), one scale per row, 8-bit activations; rotation and rounding are
 *         done in fp32.
 *  [MLX]  "MLX Nucleus-Image" (treadon/mlx-nucleus-image), overview and "Conversion notes" table:
 *         64 routed experts per MoE layer with expert-choice routing (each expert picks its top-C
 *         tokens, outputs are scattered back through one matmul); MoE expert SwiGLU is silu(gate)*up
 *         with the first half of the fused projection the gate and the second half the up projection.
 *  [XB]   "XB_UNetLoaderINTROCm" node page, "The mechanism, briefly": matmuls multiply in INT8 and
 *         dequantise back on the fly; "Inputs that matter": a stochastic LoRA mode bakes LoRAs into the
 *         quantised model with random-rounding deltas at load.
 *  [NF2s] The NitroFusion2 page, "Why a step-1 file": a LoRA patched onto a quantised file is
 *         re-quantised with fresh scales and random rounding.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - Hadamard: Sylvester construction, natural order, no random signs; block-diagonal with contiguous
 *    blocks of g along the input dimension; computed as the iterative fast transform with stages
 *    h = 1, 2, 4, ..., g/2 in that order, then scaled by 2^(-log2(g)/2), which is exact for g = 4^k.
 *  - The rotated fp32 values go straight into the quantiser (no bf16 rounding in between).
 *  - Quantiser: scale = amax / qmax (fp32 division), code = clamp(rint(r / scale), -qmax, qmax)
 *    (fp32 division, ties to even); an all-zero row has scale 0 and codes 0.  qmax = 127 for INT8,
 *    7 for INT4.  Activations use one scale per token over the whole rotated row.
 *  - Dequantisation: bf16( ((float)acc * s_act) * s_w ), optional bias added in fp32 before rounding.
 *  - silu(g) = g / (1 + E(-g)) (g * E(g) below g = -64, where 1 + E(g) is exactly 1), where E is the
 *    fixed fp32 exponential defined in oracle_exp below (Cody-Waite reduction, Taylor polynomial, fused
 *    multiply-adds as written, one rounding of p * 2^n, so it underflows and overflows as e^x does).
 *  - Router: softmax over the experts of each token in fp32 (max-subtracted, E() of the differences,
 *    sum in ascending expert order, one division).  Expert e takes the C tokens with the largest
 *    probability, ties to the lower token index; its list is written in ascending token order and its
 *    gate weight is that probability (not renormalised).
 *  - Combine: out[t] = bf16( sum over experts e ascending that took t of w * z ), accumulated in fp32
 *    starting from +0.0f with a separate multiply and add; tokens taken by no expert give +0.
 *  - INT4 packing: two's-complement nibbles, even k in bits 0-3, odd k in bits 4-7.
 *  - LoRA re-quantisation (oracle_requantize_lora): the patch is applied in the rotated basis to the
 *    dequantised weights, the delta alpha * B A rotated like the weights; fresh scale amax / 127; random
 *    rounding floor(t) + [u < t - floor(t)] with u uniform in [0, 1) from Philox4x64-10 (a counter-based
 *    generator, see oracle_philox4x64_10): counter ((e N + n) K/4 + k/4, 0, 0, 0), key (seed, 0), word
 *    k % 4, top 24 bits times 2^-24.  Delta sums in ascending rank index from +0.0f, separate multiply and
 *    add, then times alpha.  The pages fix none of these details (pinned by the oracle-pin tests).
 *    The loader's second mode, which re-quantises each patched layer ([XB] "Inputs that matter":
 *    Dynamic), takes the same patched values and fresh scale with nearest rounding instead,
 *    code = clamp(rint(V / scale), -127, 127): the weight quantiser applied to V.
 *  - W6A8 / W4A8 with an FP8 scale per group of 16 ([NF2] "How they were made"; oracle_quantize_g16,
 *    oracle_linear_g16): the same block rotation; symmetric integer codes, qmax = 31 (6 bits) or 7 (4 bits);
 *    FP8 = E4M3 (sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, largest finite 448),
 *    one per group of 16 consecutive k, relative to one fp32 scale per row: s_row = amax / (qmax * 448),
 *    f_j = E4M3((amax_j / amax) * 448) nearest-even, the group's scale S_j = s_row * f_j, and
 *    code = clamp(rint(r / S_j), +-qmax) (0 where S_j = 0).  The kernel decodes code * f_j (exact in fp16)
 *    and multiplies by the row scale after the sum.  Packing: 4-bit as INT4 above; 6-bit codes four to
 *    three bytes, code 4j+i in bits 6i..6i+5 of the little-endian 24-bit word j.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------------------- */
/* bf16 <-> fp32                                                                                       */
/* ------------------------------------------------------------------------------------------------- */

static float bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round an fp32 value to bf16, nearest, ties to even.  NaN stays a quiet NaN. */
static uint16_t f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

void oracle_bf16_round(const float* in, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16(in[i]);
}

/* ------------------------------------------------------------------------------------------------- */
/* E(x): the fixed fp32 exponential used by silu and softmax.                                          */
/*                                                                                                     */
/* Cody & Waite's additive range reduction ("Software Manual for the Elementary Functions", 1980):      */
/* n = rint(x * log2(e)), r = x - n*LN2_HI - n*LN2_LO, where LN2_HI is ln 2 rounded to 16 significant   */
/* bits (n*LN2_HI is exact for |n| < 256) and LN2_LO = ln 2 - LN2_HI rounded to fp32, each step one     */
/* fused multiply-add.  e^r comes from its Taylor series through r^7 (terms 1/k! rounded to fp32)       */
/* evaluated by Horner's rule with fused multiply-adds, and the result is p * 2^n rounded once to fp32  */
/* (ldexpf: exact for a normal result, one IEEE rounding for a subnormal one, +inf past the largest    */
/* finite value).  So E follows e^x into the subnormal range and reaches 0 below about -103.97 and     */
/* +inf above about 88.72, as the fp32 rounding of e^x does.  The argument is first clamped to          */
/* [-150, 100]: that keeps |n| < 256 (the reduction stays exact) and changes no result, since e^x       */
/* already rounds to 0 below -104 and to +inf above 89.                                                 */
/* ------------------------------------------------------------------------------------------------- */

float oracle_exp(float x) {
    const float log2e = 0x1.715476p+0f;       /* log2(e) rounded to fp32 */
    const float ln2_hi = 0x1.62e4p-1f;        /* 45426 / 65536 = 0.693145751953125 */
    const float ln2_lo = 0x1.7f7d1cp-20f;     /* ln 2 - ln2_hi, rounded to fp32 */
    if (x < -150.0f) x = -150.0f;
    if (x > 100.0f) x = 100.0f;
    float n = rintf(x * log2e);               /* -216 <= n <= 144 */
    float r = fmaf(-n, ln2_hi, x);
    r = fmaf(-n, ln2_lo, r);
    float p = 1.0f / 5040.0f;                 /* 1/7! */
    p = fmaf(p, r, 1.0f / 720.0f);
    p = fmaf(p, r, 1.0f / 120.0f);
    p = fmaf(p, r, 1.0f / 24.0f);
    p = fmaf(p, r, 1.0f / 6.0f);
    p = fmaf(p, r, 0.5f);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    return ldexpf(p, (int)n);                 /* p * 2^n, rounded once */
}

void oracle_exp_array(const float* x, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_exp(x[i]);
}

/* silu(g) = g * sigmoid(g) = g / (1 + e^-g)  [MLX: MoE experts use silu(gate) * up].
 * Below g = -64, e^-g would overflow fp32 from about -88.7 on while silu(g) is still a normal or
 * subnormal number; there 1 + e^g rounds to exactly 1 (e^g < 2^-92), so silu(g) = g * e^g, which is
 * the same function written without the overflow. */
float oracle_silu(float g) {
    if (g < -64.0f) return g * oracle_exp(g);
    float e = oracle_exp(-g);
    float den = 1.0f + e;
    return g / den;
}

void oracle_silu_array(const float* x, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_silu(x[i]);
}

/* ------------------------------------------------------------------------------------------------- */
/* Rotation: block-diagonal normalised Hadamard along the input dimension  [NUC], [NF2]               */
/* ------------------------------------------------------------------------------------------------- */

/* log4 of g if g is a power of four (1, 4, 16, 64, 256, 1024, ...), else -1.  g = 1 means no rotation. */
static int log4_of(int g) {
    int k = 0;
    if (g < 1) return -1;
    while (g > 1) {
        if (g % 4) return -1;
        g /= 4;
        ++k;
    }
    return k;
}

/* One block of g values, in place: Sylvester H_g applied by the fast transform (stages h = 1, 2, ...,
 * g/2; pair (j, j+h) with bit h of j clear becomes (a + b, a - b)), then scaled by 2^-(log2 g)/2. */
static void fwht_block(float* v, int g, float norm) {
    for (int h = 1; h < g; h *= 2)
        for (int i = 0; i < g; i += 2 * h)
            for (int j = i; j < i + h; ++j) {
                float a = v[j];
                float b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
    for (int j = 0; j < g; ++j) v[j] = v[j] * norm;
}

/* Rotate rows of fp32 values: rows x K, contiguous blocks of g along K.  Returns 0, or -1 on bad g/K. */
int oracle_rotate_rows_f32(const float* in, int64_t rows, int K, int g, float* out) {
    int k4 = log4_of(g);
    if (k4 < 0 || K % g) return -1;
    float norm = ldexpf(1.0f, -k4);
    for (int64_t r = 0; r < rows; ++r) {
        float* o = out + r * (int64_t)K;
        memcpy(o, in + r * (int64_t)K, sizeof(float) * (size_t)K);
        for (int b = 0; b < K; b += g) fwht_block(o + b, g, norm);
    }
    return 0;
}

/* Same, from bf16 input (widened to fp32 exactly). */
int oracle_rotate_rows_bf16(const uint16_t* in, int64_t rows, int K, int g, float* out) {
    int k4 = log4_of(g);
    if (k4 < 0 || K % g) return -1;
    float norm = ldexpf(1.0f, -k4);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float* o = out + r * (int64_t)K;
        for (int k = 0; k < K; ++k) o[k] = bf16_to_f32(in[r * (int64_t)K + k]);
        for (int b = 0; b < K; b += g) fwht_block(o + b, g, norm);
    }
    return 0;
}

/* ------------------------------------------------------------------------------------------------- */
/* Symmetric per-row quantiser  [NUC] (nearest rounding, one FP32 scale per row), [NF2] (fp32)          */
/* ------------------------------------------------------------------------------------------------- */

void oracle_quantize_rows(const float* r, int64_t rows, int K, int qmax, int8_t* q, float* s) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        const float* v = r + i * (int64_t)K;
        float amax = 0.0f;
        for (int k = 0; k < K; ++k) {
            float a = fabsf(v[k]);
            if (a > amax) amax = a;
        }
        float sc = amax / (float)qmax;
        s[i] = sc;
        for (int k = 0; k < K; ++k) {
            float c = 0.0f;
            if (sc != 0.0f) {
                c = rintf(v[k] / sc);
                if (c > (float)qmax) c = (float)qmax;
                if (c < -(float)qmax) c = -(float)qmax;
            }
            q[i * (int64_t)K + k] = (int8_t)c;
        }
    }
}

/* Rotate then quantise bf16 rows (activations: one scale per token over the whole row). */
int oracle_rotq_rows(const uint16_t* x, int64_t rows, int K, int g, int qmax, int8_t* q, float* s,
                     float* rot_out) {
    float* r = (float*)malloc(sizeof(float) * (size_t)rows * (size_t)K);
    if (!r) return -2;
    int st = oracle_rotate_rows_bf16(x, rows, K, g, r);
    if (st == 0) {
        oracle_quantize_rows(r, rows, K, qmax, q, s);
        if (rot_out) memcpy(rot_out, r, sizeof(float) * (size_t)rows * (size_t)K);
    }
    free(r);
    return st;
}

/* INT4 nibble packing: byte j of a row holds code 2j in bits 0-3 and code 2j+1 in bits 4-7. */
void oracle_pack_int4(const int8_t* q, int64_t rows, int K, uint8_t* out) {
    for (int64_t i = 0; i < rows; ++i)
        for (int j = 0; j < K / 2; ++j) {
            uint8_t lo = (uint8_t)q[i * (int64_t)K + 2 * j] & 0x0f;
            uint8_t hi = (uint8_t)q[i * (int64_t)K + 2 * j + 1] & 0x0f;
            out[i * (int64_t)(K / 2) + j] = (uint8_t)(lo | (hi << 4));
        }
}

void oracle_unpack_int4(const uint8_t* p, int64_t rows, int K, int8_t* q) {
    for (int64_t i = 0; i < rows; ++i)
        for (int j = 0; j < K / 2; ++j) {
            uint8_t b = p[i * (int64_t)(K / 2) + j];
            int lo = b & 0x0f, hi = b >> 4;
            q[i * (int64_t)K + 2 * j] = (int8_t)(lo >= 8 ? lo - 16 : lo);
            q[i * (int64_t)K + 2 * j + 1] = (int8_t)(hi >= 8 ? hi - 16 : hi);
        }
}

/* Offline weight converter: each row of each [N, K] expert matrix is rotated along K (group g) and
 * quantised with its own FP32 scale  [NUC].  bits = 8: q_out is int8 [E, N, K];  bits = 4: q_out is the
 * nibble-packed u8 [E, N, K/2] with qmax = 7. */
int oracle_quantize_weights(const uint16_t* w, int E, int N, int K, int g, int bits, void* q_out,
                            float* s_out) {
    if (bits != 8 && bits != 4) return -1;
    int64_t rows = (int64_t)E * N;
    int8_t* q = (int8_t*)malloc((size_t)rows * (size_t)K);
    if (!q) return -2;
    int st = oracle_rotq_rows(w, rows, K, g, bits == 8 ? 127 : 7, q, s_out, NULL);
    if (st == 0) {
        if (bits == 8)
            memcpy(q_out, q, (size_t)rows * (size_t)K);
        else
            oracle_pack_int4(q, rows, K, (uint8_t*)q_out);
    }
    free(q);
    return st;
}

/* ------------------------------------------------------------------------------------------------- */
/* Counter-based random numbers: Philox4x64 with 10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel    */
/* random numbers: as easy as 1, 2, 3", SC 2011).  Each round multiplies counter words 0 and 2 by the    */
/* two Philox constants (full 128-bit products), and the new counter is (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2),  */
/* hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the key is bumped by the two Weyl constants before every round but   */
/* the first.                                                                                          */
/* ------------------------------------------------------------------------------------------------- */

static void mulhilo64(uint64_t a, uint64_t b, uint64_t* hi, uint64_t* lo) {
    unsigned __int128 p = (unsigned __int128)a * (unsigned __int128)b;
    *hi = (uint64_t)(p >> 64);
    *lo = (uint64_t)p;
}

void oracle_philox4x64_10(const uint64_t* ctr, const uint64_t* key, uint64_t* out) {
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
    uint64_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3], k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        uint64_t hi0, lo0, hi1, lo1;
        mulhilo64(M0, c0, &hi0, &lo0);
        mulhilo64(M1, c2, &hi1, &lo1);
        uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

/* ------------------------------------------------------------------------------------------------- */
/* LoRA patch of quantised weights with re-quantisation  [NF2s], [XB]                                  */
/* ------------------------------------------------------------------------------------------------- */

/* q [E, N, K] int8 and s [E, N]: weights quantised in the rotated basis (group g).  lb [E, N, rank] and
 * la [E, rank, K] bf16: the LoRA factors (original basis), delta = alpha * lb . la.  Writes fresh codes
 * q_out [E, N, K] and scales s_out [E, N]:
 *   R = (float)q * s;  D[k] = alpha * sum_j lb[n, j] * la[j, k];  V = R + rotate_g(D);
 *   scale = amax|V| / 127;  t = V / scale (0 when scale is 0);
 *   code = clamp(floor(t) + (u < t - floor(t) ? 1 : 0), -127, 127): rounded up with probability t - floor(t)
 *   (the difference is exact in fp32), so integers stay put and the rounding is unbiased to 2^-24. 
 * Returns 0, or -1 on a bad group or K (K must be a multiple of g and of 4). */
int oracle_requantize_lora(const int8_t* q, const float* s, int E, int N, int K, int g, const uint16_t* lb,
                           const uint16_t* la, int rank, float alpha, uint64_t seed, int nearest, int8_t* q_out,
                           float* s_out) {
    int k4 = log4_of(g);
    if (k4 < 0 || K % g || K % 4 || rank < 0) return -1;
    float norm = ldexpf(1.0f, -k4);
    int64_t rows = (int64_t)E * N;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < rows; ++row) {
        int64_t e = row / N;
        float* d = (float*)malloc(sizeof(float) * (size_t)K);
        float* v = (float*)malloc(sizeof(float) * (size_t)K);
        for (int k = 0; k < K; ++k) {
            float acc = 0.0f;
            for (int j = 0; j < rank; ++j) {
                float p = bf16_to_f32(lb[row * rank + j]) * bf16_to_f32(la[(e * rank + j) * (int64_t)K + k]);
                acc = acc + p;
            }
            d[k] = alpha * acc;
        }
        for (int b = 0; b < K; b += g) fwht_block(d + b, g, norm);
        float amax = 0.0f;
        for (int k = 0; k < K; ++k) {
            float r = (float)q[row * (int64_t)K + k] * s[row];
            v[k] = r + d[k];
            float a = fabsf(v[k]);
            if (a > amax) amax = a;
        }
        float sc = amax / 127.0f;
        s_out[row] = sc;
        uint64_t key[2] = {seed, 0}, ctr[4] = {0, 0, 0, 0}, w[4];
        for (int k = 0; k < K; ++k) {
            if (k % 4 == 0) {
                ctr[0] = (uint64_t)row * (uint64_t)(K / 4) + (uint64_t)(k / 4);
                oracle_philox4x64_10(ctr, key, w);
            }
            float u = (float)(w[k % 4] >> 40) * 0x1p-24f;
            float c = 0.0f;
            if (sc != 0.0f) {
                float t = v[k] / sc;
                if (nearest) {
                    c = rintf(t);
                } else {
                    float fl = floorf(t);
                    c = fl + (u < t - fl ? 1.0f : 0.0f);
                }
                if (c > 127.0f) c = 127.0f;
                if (c < -127.0f) c = -127.0f;
            }
            q_out[row * (int64_t)K + k] = (int8_t)c;
        }
        free(d);
        free(v);
    }
    return 0;
}

/* ------------------------------------------------------------------------------------------------- */
/* INT8 x INT8 -> INT32 product and dequantisation  [NUC] (W8A8 linear, BF16 outputs), [XB]             */
/* ------------------------------------------------------------------------------------------------- */

/* acc[m, n] = sum_k a[m, k] * b[n, k]  (both row-major with K contiguous; exact in int32). */
void oracle_gemm_i8_i32(const int8_t* a, const int8_t* b, int M, int N, int K, int32_t* acc) {
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            const int8_t* ar = a + (int64_t)m * K;
            const int8_t* br = b + (int64_t)n * K;
            int32_t s = 0;
            for (int k = 0; k < K; ++k) s += (int32_t)ar[k] * (int32_t)br[k];
            acc[(int64_t)m * N + n] = s;
        }
}

static float dequant(int32_t acc, float sa, float sb) {
    float v = (float)acc;
    v = v * sa;
    v = v * sb;
    return v;
}

void oracle_dequant_bf16(const int32_t* acc, const float* sa, const float* sb, const uint16_t* bias, int M,
                         int N, uint16_t* y) {
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            float v = dequant(acc[(int64_t)m * N + n], sa[m], sb[n]);
            if (bias) v = v + bf16_to_f32(bias[n]);
            y[(int64_t)m * N + n] = f32_to_bf16(v);
        }
}

/* The single W8A8 ConvRot linear: y = bf16(dequant(rotq(x) . qw^T)) (+ bias). */
int oracle_linear_w8a8(const uint16_t* x, int M, int K, const int8_t* qw, const float* sw, int N, int g,
                       const uint16_t* bias, uint16_t* y, int8_t* qx_out, float* sx_out) {
    int8_t* qx = (int8_t*)malloc((size_t)M * (size_t)K);
    float* sx = (float*)malloc(sizeof(float) * (size_t)M);
    int32_t* acc = (int32_t*)malloc(sizeof(int32_t) * (size_t)M * (size_t)N);
    int st = -2;
    if (qx && sx && acc) {
        st = oracle_rotq_rows(x, M, K, g, 127, qx, sx, NULL);
        if (st == 0) {
            oracle_gemm_i8_i32(qx, qw, M, N, K, acc);
            oracle_dequant_bf16(acc, sx, sw, bias, M, N, y);
            if (qx_out) memcpy(qx_out, qx, (size_t)M * (size_t)K);
            if (sx_out) memcpy(sx_out, sx, sizeof(float) * (size_t)M);
        }
    }
    free(qx);
    free(sx);
    free(acc);
    return st;
}

/* ------------------------------------------------------------------------------------------------- */
/* W6A8 / W4A8: 6- or 4-bit codes with an FP8 (E4M3) scale per group of 16  [NF2]                        */
/* ------------------------------------------------------------------------------------------------- */

/* E4M3 byte -> value: sign bit 7, exponent bits 3-6 (bias 7), mantissa bits 0-2; exponent field 0 holds
 * the subnormals m * 2^-9; exponent 15 with mantissa 7 is NaN (no infinities). */
float oracle_e4m3_decode(uint8_t b) {
    int e = (b >> 3) & 15, m = b & 7;
    float v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexpf((float)m, -9);
    else
        v = ldexpf((float)(8 + m), e - 10);
    return (b & 0x80) ? -v : v;
}

/* Non-negative fp32 -> E4M3 byte: the nearest E4M3 value, ties to the even mantissa; 448 and above give
 * 448 (0x7e); zero and values below half the smallest subnormal give 0. */
uint8_t oracle_e4m3_encode(float x) {
    if (!(x > 0.0f)) return 0;
    if (x >= 448.0f) return 0x7e;
    int e2;
    frexpf(x, &e2); /* x in [2^(e2-1), 2^e2) */
    int E = e2 - 1;
    if (E < -6) E = -6; /* below 2^-6 the spacing stays 2^-9 (subnormals) */
    float steps = rintf(ldexpf(x, 3 - E)); /* x in units of the spacing 2^(E-3), exact before rounding */
    int n = (int)steps;
    if (E == -6 && n < 8) return (uint8_t)n; /* subnormal or zero */
    if (n == 16) {                           /* rounded up into the next binade */
        E += 1;
        n = 8;
    }
    return (uint8_t)(((E + 7) << 3) | (n - 8));
}

void oracle_e4m3_encode_array(const float* x, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(x[i]);
}

void oracle_e4m3_decode_array(const uint8_t* b, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_decode(b[i]);
}

/* 6-bit packing: codes 4j..4j+3 of a row in bytes 3j..3j+2, code 4j+i in bits 6i..6i+5 (two's complement)
 * of the little-endian 24-bit word. */
void oracle_pack_int6(const int8_t* q, int64_t rows, int K, uint8_t* out) {
    for (int64_t r = 0; r < rows; ++r)
        for (int j = 0; j < K / 4; ++j) {
            uint32_t w = 0;
            for (int i = 0; i < 4; ++i) w |= ((uint32_t)(uint8_t)q[r * (int64_t)K + 4 * j + i] & 63u) << (6 * i);
            uint8_t* o = out + r * (int64_t)(K / 4 * 3) + 3 * j;
            o[0] = (uint8_t)w;
            o[1] = (uint8_t)(w >> 8);
            o[2] = (uint8_t)(w >> 16);
        }
}

void oracle_unpack_int6(const uint8_t* p, int64_t rows, int K, int8_t* q) {
    for (int64_t r = 0; r < rows; ++r)
        for (int j = 0; j < K / 4; ++j) {
            const uint8_t* b = p + r * (int64_t)(K / 4 * 3) + 3 * j;
            uint32_t w = (uint32_t)b[0] | ((uint32_t)b[1] << 8) | ((uint32_t)b[2] << 16);
            for (int i = 0; i < 4; ++i) {
                int c = (int)((w >> (6 * i)) & 63u);
                q[r * (int64_t)K + 4 * j + i] = (int8_t)(c >= 32 ? c - 64 : c);
            }
        }
}

/* Group-16 quantiser of rotated rows r [rows, K] (K a multiple of 16): codes q (int8 holding the 6- or
 * 4-bit values), E4M3 group scales f8 [rows, K/16], row scales s_row [rows]. */
void oracle_quantize_g16_rows(const float* r, int64_t rows, int K, int qmax, int8_t* q, uint8_t* f8,
                              float* s_row) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        const float* v = r + i * (int64_t)K;
        float amax = 0.0f;
        for (int k = 0; k < K; ++k)
            if (fabsf(v[k]) > amax) amax = fabsf(v[k]);
        const float sr = amax / (float)(qmax * 448);
        s_row[i] = sr;
        for (int j = 0; j < K / 16; ++j) {
            float aj = 0.0f;
            for (int k = 16 * j; k < 16 * j + 16; ++k)
                if (fabsf(v[k]) > aj) aj = fabsf(v[k]);
            uint8_t f = 0;
            if (amax > 0.0f) {
                float ratio = aj / amax;
                f = oracle_e4m3_encode(ratio * 448.0f);
            }
            f8[i * (int64_t)(K / 16) + j] = f;
            const float S = sr * oracle_e4m3_decode(f);
            for (int k = 16 * j; k < 16 * j + 16; ++k) {
                float c = 0.0f;
                if (S != 0.0f) {
                    c = rintf(v[k] / S);
                    if (c > (float)qmax) c = (float)qmax;
                    if (c < -(float)qmax) c = -(float)qmax;
                }
                q[i * (int64_t)K + k] = (int8_t)c;
            }
        }
    }
}

/* Weight converter: rows of w [N, K] bf16 rotated along K (group g), then quantised per group of 16.
 * bits = 6: q_out [N, 3K/4] bytes; bits = 4: [N, K/2] nibble-packed.  codes_out (optional) [N, K] int8. */
int oracle_quantize_g16(const uint16_t* w, int N, int K, int g, int bits, uint8_t* q_out, uint8_t* f8_out,
                        float* s_out, int8_t* codes_out) {
    if ((bits != 6 && bits != 4) || K % 16) return -1;
    float* r = (float*)malloc(sizeof(float) * (size_t)N * (size_t)K);
    int8_t* q = (int8_t*)malloc((size_t)N * (size_t)K);
    int st = -2;
    if (r && q) {
        st = oracle_rotate_rows_bf16(w, N, K, g, r);
        if (st == 0) {
            oracle_quantize_g16_rows(r, N, K, bits == 6 ? 31 : 7, q, f8_out, s_out);
            if (bits == 6)
                oracle_pack_int6(q, N, K, q_out);
            else
                oracle_pack_int4(q, N, K, q_out);
            if (codes_out) memcpy(codes_out, q, (size_t)N * (size_t)K);
        }
    }
    free(r);
    free(q);
    return st;
}

/* The W6A8 / W4A8 linear on given token codes qx [M, K], sx [M] and weight codes q [N, K] (int8 holding the
 * 6- or 4-bit values), f8 [N, K/16], s_row [N]:
 *   A[m, n] = sum_k qx[m, k] * (q[n, k] * f(n, k/16)), exact (each term is an integer times a multiple of
 *   2^-9 below 2^21, so |A| < 2^34 in steps of 2^-9 fits the 53-bit fp64 significand), rounded once to fp32;
 *   y = bf16(((float)A * sx[m]) * s_row[n]) (+ bias[n] in fp32 before the rounding).
 * acc_out (optional) gets A in fp64 and abs_out (optional) the sum of |terms|, for error bounds. */
void oracle_gemm_g16(const int8_t* qx, const float* sx, int M, int K, const int8_t* q, const uint8_t* f8,
                     const float* s_row, int N, const uint16_t* bias, uint16_t* y, double* acc_out,
                     double* abs_out) {
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            double a = 0.0, aa = 0.0;
            for (int k = 0; k < K; ++k) {
                double wk = (double)q[(int64_t)n * K + k] * (double)oracle_e4m3_decode(f8[(int64_t)n * (K / 16) + k / 16]);
                double term = (double)qx[(int64_t)m * K + k] * wk;
                a += term;
                aa += fabs(term);
            }
            float v = (float)a;
            v = v * sx[m];
            v = v * s_row[n];
            if (bias) v = v + bf16_to_f32(bias[n]);
            y[(int64_t)m * N + n] = f32_to_bf16(v);
            if (acc_out) acc_out[(int64_t)m * N + n] = a;
            if (abs_out) abs_out[(int64_t)m * N + n] = aa;
        }
}

/* ------------------------------------------------------------------------------------------------- */
/* Expert-choice routing  [MLX]                                                                        */
/* ------------------------------------------------------------------------------------------------- */

/* p[t, e] = softmax over the E experts of token t. */
void oracle_softmax_experts(const float* logits, int T, int E, float* p) {
    for (int t = 0; t < T; ++t) {
        const float* l = logits + (int64_t)t * E;
        float m = l[0];
        for (int e = 1; e < E; ++e)
            if (l[e] > m) m = l[e];
        float z = 0.0f;
        for (int e = 0; e < E; ++e) z = z + oracle_exp(l[e] - m);
        for (int e = 0; e < E; ++e) p[(int64_t)t * E + e] = oracle_exp(l[e] - m) / z;
    }
}

typedef struct {
    float p;
    int t;
} scored_token;

/* Higher probability first; equal probability -> lower token index first. */
static int by_score_then_index(const void* x, const void* y) {
    const scored_token* a = (const scored_token*)x;
    const scored_token* b = (const scored_token*)y;
    if (a->p > b->p) return -1;
    if (a->p < b->p) return 1;
    return (a->t > b->t) - (a->t < b->t);
}

static int by_index(const void* x, const void* y) {
    int a = *(const int*)x, b = *(const int*)y;
    return (a > b) - (a < b);
}

/* Each expert e takes the C tokens ranked highest by p[:, e] (ties to the lower token index);
 * idx[e, :] lists them in ascending token order and wt[e, c] = p[idx[e, c], e]. */
int oracle_route_from_probs(const float* p, int T, int E, int C, int32_t* idx, float* wt) {
    if (C < 1 || C > T) return -1;
    scored_token* s = (scored_token*)malloc(sizeof(scored_token) * (size_t)T);
    int* pick = (int*)malloc(sizeof(int) * (size_t)C);
    if (!s || !pick) {
        free(s);
        free(pick);
        return -2;
    }
    for (int e = 0; e < E; ++e) {
        for (int t = 0; t < T; ++t) {
            s[t].p = p[(int64_t)t * E + e];
            s[t].t = t;
        }
        qsort(s, (size_t)T, sizeof *s, by_score_then_index);
        for (int c = 0; c < C; ++c) pick[c] = s[c].t;
        qsort(pick, (size_t)C, sizeof *pick, by_index);
        for (int c = 0; c < C; ++c) {
            idx[(int64_t)e * C + c] = pick[c];
            wt[(int64_t)e * C + c] = p[(int64_t)pick[c] * E + e];
        }
    }
    free(s);
    free(pick);
    return 0;
}

int oracle_route(const float* logits, int T, int E, int C, int32_t* idx, float* wt, float* p_out) {
    float* p = (float*)malloc(sizeof(float) * (size_t)T * (size_t)E);
    if (!p) return -2;
    oracle_softmax_experts(logits, T, E, p);
    int st = oracle_route_from_probs(p, T, E, C, idx, wt);
    if (p_out) memcpy(p_out, p, sizeof(float) * (size_t)T * (size_t)E);
    free(p);
    return st;
}

/* ------------------------------------------------------------------------------------------------- */
/* Expert FFN pieces                                                                                   */
/* ------------------------------------------------------------------------------------------------- */

/* a[r, j] = bf16( silu(gate) * up ) with gate = gu[r, j], up = gu[r, I + j] (both bf16)  [MLX] */
void oracle_swiglu(const uint16_t* gu, int64_t rows, int I, uint16_t* a) {
    for (int64_t r = 0; r < rows; ++r)
        for (int j = 0; j < I; ++j) {
            float g = bf16_to_f32(gu[r * 2 * I + j]);
            float u = bf16_to_f32(gu[r * 2 * I + I + j]);
            float v = oracle_silu(g) * u;
            a[r * I + j] = f32_to_bf16(v);
        }
}

/* out[t, :] = bf16( sum over e ascending, over c with idx[e, c] == t, of wt[e, c] * z[e*C + c, :] ) */
void oracle_combine(const uint16_t* z, const int32_t* idx, const float* wt, int T, int E, int C, int d,
                    uint16_t* out) {
    float* acc = (float*)malloc(sizeof(float) * (size_t)T * (size_t)d);
    for (int64_t i = 0; i < (int64_t)T * d; ++i) acc[i] = 0.0f;
    for (int e = 0; e < E; ++e)
        for (int c = 0; c < C; ++c) {
            int t = idx[(int64_t)e * C + c];
            float w = wt[(int64_t)e * C + c];
            const uint16_t* zr = z + ((int64_t)e * C + c) * d;
            for (int j = 0; j < d; ++j) {
                float prod = w * bf16_to_f32(zr[j]);
                acc[(int64_t)t * d + j] = acc[(int64_t)t * d + j] + prod;
            }
        }
    oracle_bf16_round(acc, (int64_t)T * d, out);
    free(acc);
}

/* Widen stored expert weights to int8 codes [rows, K] (unpacking nibbles for 4-bit weights). */
static int8_t* expert_codes(const void* q, int bits, int64_t rows, int K) {
    int8_t* c = (int8_t*)malloc((size_t)rows * (size_t)K);
    if (!c) return NULL;
    if (bits == 8)
        memcpy(c, q, (size_t)rows * (size_t)K);
    else
        oracle_unpack_int4((const uint8_t*)q, rows, K, c);
    return c;
}

/* Gate/up stage for every (expert, slot): a[e*C + c, :] from the quantised token row idx[e, c]. */
void oracle_moe_gateup(const int8_t* qx, const float* sx, int d, const int32_t* idx, int E, int C, int I,
                       const void* q_gu, const float* s_gu, int wbits, uint16_t* a) {
    int8_t* w = expert_codes(q_gu, wbits, (int64_t)E * 2 * I, d);
#pragma omp parallel for schedule(dynamic, 1)
    for (int ec = 0; ec < E * C; ++ec) {
        int e = ec / C;
        int t = idx[ec];
        const int8_t* xr = qx + (int64_t)t * d;
        uint16_t* gu = (uint16_t*)malloc(sizeof(uint16_t) * 2 * (size_t)I);
        for (int n = 0; n < 2 * I; ++n) {
            const int8_t* wr = w + ((int64_t)e * 2 * I + n) * d;
            int32_t acc = 0;
            for (int k = 0; k < d; ++k) acc += (int32_t)xr[k] * (int32_t)wr[k];
            gu[n] = f32_to_bf16(dequant(acc, sx[t], s_gu[(int64_t)e * 2 * I + n]));
        }
        oracle_swiglu(gu, 1, I, a + (int64_t)ec * I);
        free(gu);
    }
    free(w);
}

/* Down stage: z[e*C + c, :] = bf16(dequant(qa[e*C + c] . q_dn[e]^T)). */
void oracle_moe_down(const int8_t* qa, const float* sa, int E, int C, int I, int d, const void* q_dn,
                     const float* s_dn, int wbits, uint16_t* z) {
    int8_t* w = expert_codes(q_dn, wbits, (int64_t)E * d, I);
#pragma omp parallel for schedule(dynamic, 1)
    for (int ec = 0; ec < E * C; ++ec) {
        int e = ec / C;
        const int8_t* ar = qa + (int64_t)ec * I;
        for (int n = 0; n < d; ++n) {
            const int8_t* wr = w + ((int64_t)e * d + n) * I;
            int32_t acc = 0;
            for (int k = 0; k < I; ++k) acc += (int32_t)ar[k] * (int32_t)wr[k];
            z[(int64_t)ec * d + n] = f32_to_bf16(dequant(acc, sa[ec], s_dn[(int64_t)e * d + n]));
        }
    }
    free(w);
}

/* ------------------------------------------------------------------------------------------------- */
/* The whole expert-choice MoE layer (routed experts only)                                            */
/* ------------------------------------------------------------------------------------------------- */

/* x [T, d] bf16, logits [T, E] fp32; gate/up codes [E, 2I, d] (or packed [E, 2I, d/2]) with scales
 * [E, 2I]; down codes [E, d, I] (or [E, d, I/2]) with scales [E, d].  Writes out [T, d] bf16,
 * idx [E, C], wt [E, C].  Every *_out intermediate may be NULL:
 *   p_out [T, E], qx_out [T, d], sx_out [T], a_out [E*C, I] bf16, qa_out [E*C, I], sa_out [E*C],
 *   z_out [E*C, d] bf16.
 * Returns 0, -1 for invalid arguments, -2 if memory ran out. */
int oracle_moe_forward(const uint16_t* x, int T, int d, const float* logits, int E, int C, int I,
                       const void* q_gu, const float* s_gu, int g_gu, const void* q_dn, const float* s_dn,
                       int g_dn, int wbits, uint16_t* out, int32_t* idx, float* wt, float* p_out,
                       int8_t* qx_out, float* sx_out, uint16_t* a_out, int8_t* qa_out, float* sa_out,
                       uint16_t* z_out) {
    if (C < 1 || C > T || E < 1 || (wbits != 8 && wbits != 4)) return -1;
    if (log4_of(g_gu) < 0 || log4_of(g_dn) < 0 || d % g_gu || I % g_dn) return -1;
    int64_t S = (int64_t)E * C;
    int8_t* qx = (int8_t*)malloc((size_t)T * (size_t)d);
    float* sx = (float*)malloc(sizeof(float) * (size_t)T);
    uint16_t* a = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)S * (size_t)I);
    int8_t* qa = (int8_t*)malloc((size_t)S * (size_t)I);
    float* sa = (float*)malloc(sizeof(float) * (size_t)S);
    uint16_t* z = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)S * (size_t)d);
    int st = -2;
    if (qx && sx && a && qa && sa && z) {
        st = oracle_route(logits, T, E, C, idx, wt, p_out);
        if (st == 0) st = oracle_rotq_rows(x, T, d, g_gu, 127, qx, sx, NULL);
        if (st == 0) {
            oracle_moe_gateup(qx, sx, d, idx, E, C, I, q_gu, s_gu, wbits, a);
            st = oracle_rotq_rows(a, S, I, g_dn, 127, qa, sa, NULL);
        }
        if (st == 0) {
            oracle_moe_down(qa, sa, E, C, I, d, q_dn, s_dn, wbits, z);
            oracle_combine(z, idx, wt, T, E, C, d, out);
            if (qx_out) memcpy(qx_out, qx, (size_t)T * (size_t)d);
            if (sx_out) memcpy(sx_out, sx, sizeof(float) * (size_t)T);
            if (a_out) memcpy(a_out, a, sizeof(uint16_t) * (size_t)S * (size_t)I);
            if (qa_out) memcpy(qa_out, qa, (size_t)S * (size_t)I);
            if (sa_out) memcpy(sa_out, sa, sizeof(float) * (size_t)S);
            if (z_out) memcpy(z_out, z, sizeof(uint16_t) * (size_t)S * (size_t)d);
        }
    }
    free(qx);
    free(sx);
    free(a);
    free(qa);
    free(sa);
    free(z);
    return st;
}

/* Layer output rows for a list of tokens only, for checking large layers at sampled tokens.  Given the
 * routing (idx, wt) and the quantised tokens (qx, sx), out_rows[i, :] is the output of token tokens[i]:
 * the same per-(expert, slot) arithmetic as oracle_moe_forward (gate/up, SwiGLU, rotate + quantise with
 * group g_dn, down) and the same combine order (experts ascending). */
int oracle_moe_rows(const int8_t* qx, const float* sx, int d, const int32_t* idx, const float* wt, int E, int C,
                    int I, const void* q_gu, const float* s_gu, const void* q_dn, const float* s_dn, int g_dn,
                    int wbits, const int32_t* tokens, int ntok, uint16_t* out_rows) {
    if (log4_of(g_dn) < 0 || I % g_dn || (wbits != 8 && wbits != 4)) return -1;
    int8_t* wg = expert_codes(q_gu, wbits, (int64_t)E * 2 * I, d);
    int8_t* wd = expert_codes(q_dn, wbits, (int64_t)E * d, I);
    if (!wg || !wd) {
        free(wg);
        free(wd);
        return -2;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < ntok; ++i) {
        int t = tokens[i];
        float* acc = (float*)malloc(sizeof(float) * (size_t)d);
        uint16_t* gu = (uint16_t*)malloc(sizeof(uint16_t) * 2 * (size_t)I);
        uint16_t* a = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)I);
        int8_t* qa = (int8_t*)malloc((size_t)I);
        for (int j = 0; j < d; ++j) acc[j] = 0.0f;
        for (int e = 0; e < E; ++e) {
            int c = -1;
            for (int k = 0; k < C; ++k)
                if (idx[(int64_t)e * C + k] == t) c = k;
            if (c < 0) continue;
            const int8_t* xr = qx + (int64_t)t * d;
            for (int n = 0; n < 2 * I; ++n) {
                const int8_t* wr = wg + ((int64_t)e * 2 * I + n) * d;
                int32_t s = 0;
                for (int k = 0; k < d; ++k) s += (int32_t)xr[k] * (int32_t)wr[k];
                gu[n] = f32_to_bf16(dequant(s, sx[t], s_gu[(int64_t)e * 2 * I + n]));
            }
            oracle_swiglu(gu, 1, I, a);
            float sa;
            oracle_rotq_rows(a, 1, I, g_dn, 127, qa, &sa, NULL);
            float w = wt[(int64_t)e * C + c];
            for (int n = 0; n < d; ++n) {
                const int8_t* wr = wd + ((int64_t)e * d + n) * I;
                int32_t s = 0;
                for (int k = 0; k < I; ++k) s += (int32_t)qa[k] * (int32_t)wr[k];
                float z = bf16_to_f32(f32_to_bf16(dequant(s, sa, s_dn[(int64_t)e * d + n])));
                float prod = w * z;
                acc[n] = acc[n] + prod;
            }
        }
        oracle_bf16_round(acc, d, out_rows + (int64_t)i * d);
        free(acc);
        free(gu);
        free(a);
        free(qa);
    }
    free(wg);
    free(wd);
    return 0;
}
