/*
 * sa_measure.h -- measurement utility in the same library as sink_attn.h
 * (libsinkattn.so, gfx950).  It is not a step of the attention method: it
 * measures the device's practical streaming-read rate, the yardstick for the
 * HBM-bound kernels (the split-KV decode reads its K/V once, with the same loads).
 */
#ifndef SA_MEASURE_H
#define SA_MEASURE_H

#include <stdint.h>

#include "sink_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads bytes bytes of buf once, with 16-byte nontemporal loads spread over
 * num_blocks workgroups of 512 threads (4 loads in flight per thread), and
 * writes to out[b] the XOR of the 32-bit words that workgroup b read.  The XOR
 * of all num_blocks entries equals the XOR of every 32-bit word of the buffer,
 * so a pass can be checked against the host.
 *
 * buf        device pointer, 16-byte aligned (read only)
 * bytes      >= 0, a multiple of 16
 * num_blocks 1 .. 65535
 * out        device pointer to num_blocks uint32 (written)
 * The caller owns both buffers; the call is asynchronous on `stream`.
 * Errors: SA_EINVAL for null pointers, misalignment, bytes < 0 or not a
 * multiple of 16, num_blocks out of range; SA_ELAUNCH for launch failures.
 * bytes = 0 reads nothing (buf may then be null) and writes num_blocks zeros.
 */
sa_status_t sink_attn_read_probe(const void *buf, int64_t bytes, int32_t num_blocks,
                                 uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SA_MEASURE_H */
