/* rssm_probes.h -- HBM probes of a separate measurement library,
 * librssm_probes.so: a streaming copy, a streaming read, and a chunked read
 * with a trickle of writes.  They measure the device's practical ceilings and
 * calibrate the memory counters against kernels of known traffic; they are
 * not part of the decode method and are not exported by libreplayssm.so.
 *
 * Every call is asynchronous on `stream` (a hipStream_t; NULL = the default
 * stream), allocates nothing and returns RSSM_OK, RSSM_EINVAL for a bad
 * argument (nothing launched) or RSSM_EHIP if the launch failed.  All
 * pointers are device pointers.
 */
#ifndef RSSM_PROBES_H
#define RSSM_PROBES_H

#include "replayssm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Copy `bytes` (a multiple of 16) from src to dst, both 16-byte aligned,
 * grid-stride with 16-byte non-temporal loads and stores. */
RSSM_API rssm_status rssm_probe_copy(void* dst, const void* src, size_t bytes, void* stream);

/* Read `bytes` (a multiple of 16) of src (16-byte aligned), grid-stride with
 * 16-byte non-temporal loads.  sink (device float[1]) is written only if the
 * xor of everything read equals one fixed NaN pattern: the test keeps the
 * loads from being dropped, and sink's content means nothing. */
RSSM_API rssm_status rssm_probe_read(const void* src, size_t bytes, float* sink, void* stream);

/* Chunked read with a trickle of writes, the traffic mix of a decode step:
 * workgroup i reads bytes [32768 i, 32768 (i+1)) of src with non-temporal
 * loads and then stores write_bytes (0..4096, a multiple of 16) with plain
 * stores at dst + write_bytes * i.  bytes: a positive multiple of 32768; dst
 * (device, 16-byte aligned) holds bytes / 32768 * write_bytes bytes and may be
 * NULL when write_bytes is 0; sink: device float[1], as for rssm_probe_read. */
RSSM_API rssm_status rssm_probe_read_chunked(const void* src, size_t bytes, void* dst, size_t write_bytes,
                                             float* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* RSSM_PROBES_H */
