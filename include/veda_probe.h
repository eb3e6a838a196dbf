/*
 * veda_probe.h -- measurement aids for benchmarking libveda on MI355X (gfx950).
 *
 * Not part of the method's interface (include/veda.h): these entry points live in a
 * separate library, libveda_probe.so, and exist so that a benchmark can report the
 * attention kernel's matrix-core use against the rate this device actually reaches as
 * well as against the specification.
 */
#ifndef VEDA_PROBE_H
#define VEDA_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * An MFMA-only loop: each of `workgroups` workgroups of 256 threads runs iters x 16
 * products of v_mfma_f32_32x32x16_bf16 per wave (32768 flops each), i.e.
 * 2,097,152 * iters * workgroups flops in total.  out: fp32 device buffer of
 * workgroups * 256 elements (receives checksums).  Asynchronous on `stream` (a
 * hipStream_t, NULL = default stream).  Returns 0, -1 for a null `out` or a
 * non-positive count, or -6 when the launch fails.
 */
int veda_probe_mfma_peak(float* out, int32_t iters, int32_t workgroups, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* VEDA_PROBE_H */
