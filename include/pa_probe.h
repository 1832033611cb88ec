/*
 * pa_probe.h -- measurement helper shipped beside libpa.so (libpa_probe.so).
 *
 * Not part of the paged-attention API: the benchmark uses it to measure the
 * HBM read bandwidth this GPU actually sustains, so kernel throughput can be
 * reported against both the published peak and an attainable one.
 */
#ifndef PA_PROBE_H_
#define PA_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Enqueue one streaming read of `bytes` bytes at device pointer `buf`
 * (16-byte aligned, bytes a multiple of 16) on `stream` (a hipStream_t,
 * NULL = default): `blocks` workgroups of 256 threads each read 16-byte
 * chunks grid-stride with non-temporal loads and fold them into a checksum
 * that is written to device word `sink` only if it equals one fixed value
 * (so the reads cannot be optimised away; the sink's content is meaningless).  Returns 0, or -1 for invalid
 * arguments, -6 if the launch fails.
 */
int pa_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t blocks,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H_ */
