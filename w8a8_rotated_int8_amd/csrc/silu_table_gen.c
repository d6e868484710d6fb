/* Writes the SwiGLU gate activation for every bf16 bit pattern g: silu(g) = g / (1 + E(-g)) in fp32 (g * E(g)
 * below g = -64, where 1 + E(g) is exactly 1), with E the library's fixed exponential (argument clamped to
 * [-150, 100]; Cody-Waite reduction x = n ln2 + r with ln2 split into a 16-significant-bit head and an fp32
 * tail; Taylor series through r^7 with coefficients 1/k! rounded to fp32, by Horner's rule in fused
 * multiply-adds; p * 2^n rounded once, so it underflows and overflows as e^x does).
 *
 * The gate value reaching the activation is always bf16 (the dequantised gate is rounded to bf16 first, as
 * in the Nucleus-Image MLX expert MLP), so the activation has exactly 65536 possible inputs and the GEMM
 * epilogue looks it up instead of evaluating it.  Built and run on the host at library build time; every
 * operation is a single IEEE fp32 operation (compile with -ffp-contract=off).
 *
 *   silu_table_gen inc  > silu_table.inc     initializer list of 65536 hex floats, index = bf16 bits
 *   silu_table_gen bin  > silu_table.bin     the same 65536 floats, little-endian binary
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float fixed_exp(float x) {
    const float log2e = 0x1.715476p+0f;
    const float ln2_hi = 0x1.62e4p-1f;
    const float ln2_lo = 0x1.7f7d1cp-20f;
    if (x < -150.0f) x = -150.0f;
    if (x > 100.0f) x = 100.0f;
    const float n = rintf(x * log2e);
    float r = fmaf(-n, ln2_hi, x);
    r = fmaf(-n, ln2_lo, r);
    float p = 1.0f / 5040.0f;
    p = fmaf(p, r, 1.0f / 720.0f);
    p = fmaf(p, r, 1.0f / 120.0f);
    p = fmaf(p, r, 1.0f / 24.0f);
    p = fmaf(p, r, 1.0f / 6.0f);
    p = fmaf(p, r, 0.5f);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    return ldexpf(p, (int)n); /* p * 2^n, rounded once (C99 ldexpf) */
}

static float silu_of_bits(uint32_t b16) {
    const uint32_t bits = b16 << 16;
    float g;
    memcpy(&g, &bits, 4);
    if (g < -64.0f) return g * fixed_exp(g);
    const float den = 1.0f + fixed_exp(-g);
    return g / den;
}

int main(int argc, char** argv) {
    const int bin = argc > 1 && strcmp(argv[1], "bin") == 0;
    for (uint32_t i = 0; i < 65536u; ++i) {
        const float v = silu_of_bits(i);
        if (bin) {
            fwrite(&v, 4, 1, stdout);
        } else {
            uint32_t u;
            memcpy(&u, &v, 4);
            printf("%s0x%08xu", (i % 8) ? ", " : (i ? ",\n" : ""), u);
        }
    }
    if (!bin) printf("\n");
    return 0;
}
