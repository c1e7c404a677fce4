/*
 * hspec_probe.h -- measurement aid of libhspec.so (not part of the drafter
 * layer): the HBM read bandwidth this GPU actually sustains, against which the
 * in-place KV attention's bandwidth is reported next to the vendor peak.
 */
#ifndef HSPEC_PROBE_H
#define HSPEC_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Streaming read of `bytes` bytes at device pointer `buf` (16-byte aligned,
 * bytes a multiple of 16) with nontemporal 16-byte loads: 512 workgroups of
 * 256 threads, each reading its own contiguous slice with eight loads in
 * flight per thread -- the best of the shapes measured on MI355X for a 4 GiB
 * buffer (7.0-7.2 TB/s; a grid-strided read of the same buffer, 6.6-6.7
 * TB/s).  The data are XOR-folded and `sink`
 * (one device uint32) is written only if the fold hits a fixed value, so the
 * loads cannot be elided; the caller times the call.  Enqueues on `stream`
 * and returns HSPEC_OK (0), HSPEC_ERR_INVALID_ARG (-1) or HSPEC_ERR_HIP (-4).
 */
int hspec_probe_stream_read(void* stream, const void* buf, size_t bytes, uint32_t* sink);

#ifdef __cplusplus
}
#endif
#endif /* HSPEC_PROBE_H */
