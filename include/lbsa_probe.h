/*
 * lbsa_probe.h - measurement helpers of liblbsa.so (not part of the attention method).
 *
 * attn_probe_stream_read: reads `bytes` bytes (a multiple of 16) of device memory at `buf` with
 * 16-byte loads spread over `blocks` workgroups of 256 threads and writes one XOR digest per
 * thread to `sink` (device uint32[blocks * 256]) so the loads cannot be elided.  It gives the
 * measured streaming-read ceiling of the device, the yardstick for the decode kernel's HBM
 * rate.  Returns LBSA_OK, LBSA_ERR_INVALID (null pointer, misaligned, bytes % 16 != 0,
 * blocks < 1) or LBSA_ERR_HIP.  Asynchronous on `stream`.
 *
 * attn_probe_stream_read_rated: the same read with per-XCD shares.  Workgroup b runs on XCD b mod 8
 * (the dispatcher places workgroups round robin over the eight XCDs).  The buffer is cut into the
 * plain read's 8 KiB steps, dealt to the XCDs in repeating cycles in which XCD x owns q[x]
 * consecutive steps, q[x] = xcd_rates[x] scaled so the largest is 64 (host int32[8], each in
 * [0, LBSA_RATE_MAX], not all zero; a positive rate owns at least one step), and XCD x's waves take
 * its steps in turn: every XCD moves through the buffer with the others, at its own share.  With
 * rates in proportion to the XCDs' streaming rates every XCD finishes at once: the ceiling for a
 * kernel whose work is shared out by measured XCD rates.  blocks must be a positive multiple of 8;
 * sink as attn_probe_stream_read.  Returns LBSA_OK, LBSA_ERR_INVALID (as attn_probe_stream_read, or
 * bad rates, or blocks not a positive multiple of 8) or LBSA_ERR_HIP.
 *
 * attn_probe_mfma_rate: `blocks` workgroups of 256 threads (four waves) in which every wave runs
 * `iters` rounds of eight independent v_mfma_f32_16x16x32_bf16 products on register operands
 * (random finite bf16 values, no memory reads), then writes the sum of each thread's accumulators
 * (fp32 bits) to `sink` (device uint32[blocks * 256]).  One launch performs
 * blocks * 4 * iters * 8 * 16384 flops; divided by its duration, that is the bf16 matrix-core rate
 * the device sustains at the clock it holds under that load, the yardstick for the prefill
 * kernel's MFMA rate beside the 2.5 PFLOP/s dense figure.  Returns LBSA_OK, LBSA_ERR_INVALID (null or
 * misaligned sink, iters < 1, blocks < 1) or LBSA_ERR_HIP.  Asynchronous on `stream`.
 */
#ifndef LBSA_PROBE_H
#define LBSA_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int attn_probe_stream_read(const void* buf, int64_t bytes, int32_t blocks, uint32_t* sink, void* stream);
int attn_probe_stream_read_rated(const void* buf, int64_t bytes, int32_t blocks, const int32_t* xcd_rates,
                                 uint32_t* sink, void* stream);
int attn_probe_mfma_rate(int32_t iters, int32_t blocks, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LBSA_PROBE_H */
