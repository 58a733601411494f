/*
 * pf_probe.h - measurement primitive of the benchmark, not part of the GEMM: the time
 * one kernel launch takes to stream a given number of bytes from HBM, the floor a
 * weight-streaming kernel (the GEMV) of the same bytes per launch is compared with.
 */
#ifndef PF_PROBE_H
#define PF_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes at `src` (device, 16-byte aligned, bytes a multiple of 16) once,
 * in 16-byte loads spread over every CU, and stores one 32-bit fold (xor) of them per
 * workgroup into sink[0 .. pf_probe_read_sink_words()) (device), so that no load can
 * be dropped. Enqueued on `stream`; allocates nothing. Returns 0, or 5 (shape), 1
 * (null), 6 (alignment) or 8 (launch refused) as the PF_E_* codes of pf_gemm.h. */
int pf_probe_read(const void *src, int64_t bytes, uint32_t *sink, void *stream);

/* Words pf_probe_read may write into sink. */
int64_t pf_probe_read_sink_words(void);

#ifdef __cplusplus
}
#endif

#endif /* PF_PROBE_H */
