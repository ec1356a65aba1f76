/*
 * pa_measure.h -- a measurement aid of libpa_decode.so: the achievable HBM
 * read rate on this device, against which the paged kernels' KV-read rate is
 * judged beside the nominal peak.
 *
 * Decode attention reads every cached K / V element once per call, and
 * decoding is limited by memory bandwidth (page "PagedAttention by hand",
 * section "Why not set B = 1").  The reference for how fast this device can
 * read is therefore a plain streaming read of a buffer far larger than the
 * caches, made with the same 16-byte non-temporal loads as the paged kernels.
 */
#ifndef PA_MEASURE_H
#define PA_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#include "pa_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes of device memory at `buf` once (asynchronous on `stream`,
 * a hipStream_t; NULL = the default stream).
 *   buf    device pointer, 16-byte aligned, owned by the caller; only read.
 *   bytes  a multiple of 16 (0: no launch, PA_OK).
 *   sink   device pointer to 4 writable bytes owned by the caller; the kernel
 *          writes a fold of the data there only when that fold equals a fixed
 *          constant, so that the reads cannot be optimised away.  Its content
 *          afterwards carries no meaning.
 * Errors: PA_ERR_NULL (buf or sink NULL with bytes > 0), PA_ERR_SHAPE (bytes
 * not a multiple of 16 or buf misaligned), PA_ERR_HIP (launch failure, or a
 * buffer beyond 2^32 work-groups of 32 KiB).
 * Allocates nothing. */
pa_status pa_read_bytes(const void *buf, size_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_MEASURE_H */
