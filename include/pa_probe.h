/*
 * pa_probe.h - read-bandwidth probes of libpagedkv (measurement helpers).
 *
 * Decode attention is bound by HBM reads ("How PagedAttention Powers vLLM's
 * KV Cache", section "Where it bites": gathering keys and values through a
 * block table is more work than striding one contiguous array while the
 * kernel is memory-bound).  These calls measure what the GPU delivers to a
 * read-only stream of the same shape, so a decode rate can be set beside a
 * measured ceiling as well as beside the datasheet peak.  They are not part
 * of the decode path.
 */
#ifndef PA_PROBE_H_
#define PA_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the sink buffer pa_probe_read needs for `workgroups`. */
size_t pa_probe_sink_bytes(int32_t workgroups);

/*
 * Read n_chunks chunks of chunk_bytes bytes each, chunk order[i] being the
 * bytes [order[i] * chunk_bytes, (order[i] + 1) * chunk_bytes) of buf, with
 * 16-byte non-temporal loads; workgroup w reads chunks i = w, w + workgroups,
 * and so on, each of its 256 threads keeping loads_in_flight (1, 2, 4 or 8)
 * loads outstanding.  The XOR of the bytes each thread read goes to sink.
 *   buf:   device buffer holding every chunk order names (caller-checked);
 *   order: int32 [n_chunks] device array of chunk indices (a permutation
 *          for a random gather, the identity for a contiguous stream);
 *   sink:  device buffer of pa_probe_sink_bytes(workgroups) bytes.
 * chunk_bytes must be a positive multiple of 16 (PA_EINVAL otherwise, and
 * for null pointers or non-positive counts).  Asynchronous on `stream`.
 */
pa_status pa_probe_read(const void* buf, const int32_t* order, int32_t n_chunks,
                        uint32_t chunk_bytes, int32_t workgroups, int32_t loads_in_flight,
                        void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H_ */
