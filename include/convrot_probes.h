/* Achievable-rate probes of the chip the library runs on.
 *
 * These are measurement aids, not steps of the method: they let a kernel's time be read against what the
 * chip sustains as well as against its datasheet peaks.  Each launches one persistent workgroup of 512
 * threads per compute unit on the current HIP device and only enqueues work on `stream`; the caller times it
 * (HIP events) and divides the work reported in *ops / *bytes by the time.
 *
 * Errors: CONVROT_ERR_NULL for a NULL pointer, CONVROT_ERR_SHAPE for a buffer below its minimum or iters
 * outside [1, 1 << 20], CONVROT_ERR_ALIGN for a src not 16-byte aligned, CONVROT_ERR_HIP when a HIP call
 * fails.  Nothing is enqueued on an error.
 */
#ifndef CONVROT_PROBES_H
#define CONVROT_PROBES_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "convrot.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Words of `out` the probes write: 512 per compute unit of the current device (0 if it cannot be read). */
size_t convrot_probe_out_words(void);

/* int8 MFMA rate on changing operands.  Every wavefront loads 8 operand registers from src (device, at least
 * 256 KiB, read cyclically) and runs iters rounds of 32 v_mfma_i32_16x16x64_i8 (the grouped GEMMs'
 * instruction) over 8 independent accumulators, each MFMA taking a different operand pair from the one before (the MFMA's power, and with it
 * the clock the chip holds, depends on the bits it multiplies: random bytes give the rate a GEMM on random
 * data can reach).  out (device, convrot_probe_out_words() words) receives the accumulators' xor per thread.
 * *ops (host) = the int8 operations the launch performs (2 per multiply-add). */
convrot_status convrot_probe_mfma_i8(const int8_t* src, size_t src_bytes, int iters, int32_t* out,
                                     size_t out_words, double* ops, hipStream_t stream);

/* HBM read rate through non-temporal LDS DMA (the path the GEMM's weight stream takes).  Each workgroup
 * streams its own contiguous share of src (device, at least 8 KiB per compute unit; size it well above the
 * 256 MB memory-side cache) with 8 wavefronts keeping 8 KiB each in flight.  out as above.  *bytes (host) =
 * the bytes read (the whole 8 KiB-per-workgroup multiple of src_bytes that is streamed). */
convrot_status convrot_probe_hbm_read(const int8_t* src, size_t src_bytes, int32_t* out, size_t out_words,
                                      double* bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CONVROT_PROBES_H */
