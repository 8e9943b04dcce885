/*
 * qlora_nf4_profile.h - opt-in kernel timing for benchmarks.
 *
 * Instrumentation, not part of the computation.  A benchmark that wants the
 * duration of one kernel inside an entry point of qlora_nf4.h attaches a
 * pair of hipEvent_t (passed as void*) to a kernel id; from then on, every
 * launch of that kernel made BY THE CALLING THREAD is bracketed by
 * hipEventRecord(start) and hipEventRecord(stop) on the launch stream, until
 * the pair is replaced or detached (both NULL).  Events are created, read
 * and destroyed by the caller; the library only records them.  Attachments
 * are per thread and per kernel id; other threads are unaffected.
 *
 * Returns QLORA_OK, or QLORA_ERR_INVALID_ARG for an unknown kernel id or a
 * half-NULL pair.
 */
#ifndef QLORA_NF4_PROFILE_H
#define QLORA_NF4_PROFILE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QLORA_KERNEL_QUANTIZE = 0,   /* NF4 codes + block absmax (qlora_nf4_quantize)   */
  QLORA_KERNEL_DEQUANTIZE = 1, /* qlora_nf4_dequantize                            */
  QLORA_KERNEL_FWD_MAIN = 2,   /* weight product of qlora_linear_fwd: the fused dequant GEMM, or for M <= 16 the weight-streaming kernel */
  QLORA_KERNEL_BWD_DX = 3,     /* fused dequant GEMM for dX in qlora_linear_bwd   */
  QLORA_KERNEL_COUNT = 4
} qlora_kernel_id;

int qlora_profile_events(int32_t kernel_id, void* start_event, void* stop_event);

/*
 * qlora_probe_read - measurement probe, not part of the computation: reads
 * `bytes` bytes of the device buffer `src` once, with 16-byte loads, four in
 * flight per thread, consecutive lanes on consecutive pieces (at most 4096
 * workgroups of 512 threads, grid-stride), so that a benchmark can report
 * what this device streams next to the datasheet HBM figure.
 *
 *   src      device pointer, 16-byte aligned; not modified.
 *   bytes    a multiple of 16, >= 0 (0 enqueues nothing).
 *   out      device pointer to 4 writable bytes; written only to keep the
 *            loads alive (its contents afterwards are unspecified).
 *   stream   hipStream_t as void* (NULL: the default stream).
 * Returns QLORA_OK, QLORA_ERR_INVALID_ARG (misaligned src, bytes not a
 * multiple of 16, NULL pointers) before anything is enqueued, or
 * QLORA_ERR_HIP if the launch fails.
 */
int qlora_probe_read(const void* src, int64_t bytes, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_NF4_PROFILE_H */
