/*
 * lbsa_probe.h - measurement helpers of liblbsa.so (not part of the attention method).
 *
 * attn_probe_stream_read: reads `bytes` bytes (a multiple of 16) of device memory at `buf` with
 * 16-byte loads spread over `blocks` workgroups of 256 threads and writes one XOR digest per
 * thread to `sink` (device uint32[blocks * 256]) so the loads cannot be elided.  It gives the
 * measured streaming-read ceiling of the device, the yardstick for the decode kernel's HBM
 * rate.  Returns LBSA_OK, LBSA_ERR_INVALID (null pointer, misaligned, bytes % 16 != 0,
 * blocks < 1) or LBSA_ERR_HIP.  Asynchronous on `stream`.
 */
#ifndef LBSA_PROBE_H
#define LBSA_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int attn_probe_stream_read(const void* buf, int64_t bytes, int32_t blocks, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LBSA_PROBE_H */
