/*
 * paged_kv_probe.h -- measurement utility, libpagedkv_probe.so (not part of the attention
 * path or of libpagedkv.so).
 *
 * pagedkv_read_probe -- read `bytes` (rounded down to a multiple of 16) of device memory at
 * `buf` (16-byte aligned) with a grid-stride kernel of `grid` workgroups of 256 threads, on
 * `stream`, asynchronously. `sink` (device, >= grid uint32 words) receives a word only in the
 * rare case that a block's XOR of its data equals a fixed sentinel; it exists so the loads
 * cannot be optimised away. Time the launch with events to obtain the achievable streaming-read
 * rate. Returns 0, 1 for a bad argument, or 5 if the launch failed.
 *
 * pagedkv_read_probe_nt -- the same read with the non-temporal (streaming) hint on every load,
 * the hint the attention kernels put on their V loads.
 *
 * pagedkv_read_probe_chunked_nt -- workgroup w reads the w-th of `grid` contiguous chunks,
 * four 16-byte loads in flight per thread, with the non-temporal hint. Of the simple read
 * patterns measured on MI355X this one got the most out of HBM (about 7.0 TB/s on 2 GB with
 * 1024 workgroups, against 6.3-6.5 for the grid-stride forms). Arguments and status as above.
 */
#ifndef PAGED_KV_PROBE_H
#define PAGED_KV_PROBE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

int pagedkv_read_probe(const void* buf, size_t bytes, uint32_t* sink, int32_t grid,
                       hipStream_t stream);
int pagedkv_read_probe_nt(const void* buf, size_t bytes, uint32_t* sink, int32_t grid,
                          hipStream_t stream);
int pagedkv_read_probe_chunked_nt(const void* buf, size_t bytes, uint32_t* sink, int32_t grid,
                                  hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_PROBE_H */
