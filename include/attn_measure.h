/*
 * Measurement aid beside the attention path (it computes nothing of the method): a plain
 * streaming read over a device buffer, every byte read once with the 16-byte
 * non-temporal loads the decode kernels use.  Its rate over the same bytes as a decode
 * step is the practical HBM read ceiling that the step's effective bandwidth is compared
 * against (the pages report decode speed as bytes moved per second on the stored rows,
 * pegainfer PR #1055, Description).
 *
 * Ownership and errors as for attn_decode.h: the caller owns both buffers, nothing is
 * allocated, the launch is asynchronous on `stream`, and every check runs before it.
 */
#ifndef ATTN_MEASURE_H
#define ATTN_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Workgroups of one attn_stream_read launch (a fixed grid: one round on the chip). */
#define ATTN_STREAM_READ_GROUPS 2048

/*
 * Read `bytes` bytes of `buf` (device, 16-byte aligned, bytes a multiple of 16).
 *   partial  device, uint32 [ATTN_STREAM_READ_GROUPS][4]: workgroup w writes the XOR of the
 *            16-byte words it read; the XOR of all entries is the XOR of every 16-byte word
 *            of buf (a check that every word was read).  Only these 32 KB are written.
 * Returns ATTN_E_INVALID_ARG on null pointers, misalignment or a byte count that is not a
 * multiple of 16, ATTN_E_LAUNCH if HIP refuses.  bytes == 0 writes zeros to partial.
 */
int attn_stream_read(const void* buf, size_t bytes, uint32_t* partial, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MEASURE_H */
