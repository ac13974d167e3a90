/*
 * bsattn_probe.h — achievable-peak probes (measurement support), exported by their own
 * library libbsattn_probe.so, which the benchmark loads; libbsattn.so does not contain them.
 *
 * The roofline of the path compares each kernel with the vendor peaks of the chip (dense bf16
 * MFMA, HBM bandwidth). These probes measure what the chip sustains for the same resources
 * under load (clock throttling under sustained matrix work, memory-system efficiency), so
 * that a kernel can also be set against an achievable ceiling. They compute nothing of the
 * method. The caller times the launches (HIP events on `stream`) and owns every buffer.
 * Status codes as in bsattn.h (0 ok, 1 invalid argument, 4 HIP error); the text of the last
 * failure on the calling thread comes from bsattn_probe_last_error().
 */
#ifndef BSATTN_PROBE_H
#define BSATTN_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Text detail of the last failing probe call on this thread ("" if none). */
const char* bsattn_probe_last_error(void);

/* Sink size (floats) the probes write: one float per launched thread. */
size_t bsattn_probe_sink_floats(int groups);

/* Dense bf16 MFMA stream: `groups` work-groups of 4 waves, each wave issuing iters x 8
 * independent v_mfma_f32_32x32x16_bf16 (32x32x16 multiply-adds each, operands in registers).
 * *flops receives the multiply-add count x 2 of the launch. sink: device fp32, at least
 * bsattn_probe_sink_floats(groups) floats, 4-byte aligned. 1 <= groups <= 65535,
 * 1 <= iters <= 2^30; else BSATTN_E_INVALID. */
int bsattn_probe_mfma_bf16(int64_t iters, int groups, float* sink, double* flops, void* stream);

/* The same on the fp8 MFMA: iters x 8 independent v_mfma_scale_f32_32x32x64_f8f6f4 per wave
 * (e4m3 operands of unit scale, unit block scales; 32x32x64 multiply-adds each). */
int bsattn_probe_mfma_fp8(int64_t iters, int groups, float* sink, double* flops, void* stream);

/* HBM read stream: reads `bytes` (a multiple of 16, > 0) from src (device, 16-byte aligned)
 * once with 16-byte loads in `groups` work-groups of 256 threads; sink as above. */
int bsattn_probe_read(const void* src, size_t bytes, int groups, float* sink, void* stream);

/* HBM copy stream: copies `bytes` (a multiple of 16, > 0) from src to dst (device, 16-byte
 * aligned, not overlapping): `bytes` read + `bytes` written. */
int bsattn_probe_copy(const void* src, void* dst, size_t bytes, int groups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BSATTN_PROBE_H */
