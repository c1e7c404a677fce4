/*
 * hspec_probe.h -- measurement aids of libhspec.so (not part of the drafter
 * layer): the HBM read bandwidth this GPU actually sustains, against which the
 * in-place KV attention's bandwidth is reported next to the vendor peak; and
 * the LDS cost of one wave-wide access pattern, with which the attention
 * stage's LDS reads and writes are profiled one kind at a time.
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

/*
 * LDS access-pattern probe: `grid` workgroups of four waves, each with 16 KiB
 * of LDS, every wave repeating one access `iters` times (a multiple of 8, at
 * most 2^20) with lane l at byte offset offsets[l] of the workgroup's LDS.
 * kind 0: 16-byte read (ds_read_b128), 1: 16-byte write (ds_write_b128),
 * 2: 8-byte read (ds_read_b64).  `offsets` is a HOST array of 64 entries, each
 * aligned to the access size and inside the 16 KiB; the kernel touches no
 * global memory except `sink` (one device uint32), written only if the
 * folded data hit a fixed value.  Used under a counter profiler: per
 * dispatch, SQ_LDS_BANK_CONFLICT over SQ_INSTS_LDS is the conflict cost of
 * the pattern.  Enqueues on `stream`; returns HSPEC_OK (0),
 * HSPEC_ERR_INVALID_ARG (-1) or HSPEC_ERR_HIP (-4).
 */
int hspec_probe_lds_pattern(void* stream, int kind, const uint32_t* offsets, int iters, int grid,
                            uint32_t* sink);

#ifdef __cplusplus
}
#endif
#endif /* HSPEC_PROBE_H */
