/*
 * spa_probe.h -- a measurement aid shipped in libspa.so next to the sparse
 * paged decode-attention entry points (spa.h). Not part of the method: the
 * benchmark uses it to measure, on the GPU it runs on, how fast whole 4 KiB
 * pieces scattered over a large buffer can be read -- the access shape of the
 * attention kernel's logical-page reads (one logical page of one head is a
 * contiguous 4 KiB of keys and 4 KiB of values at 16 tokens) -- so that the
 * attention's achieved bandwidth can be set against a measured ceiling as
 * well as against the HBM peak.
 */
#ifndef SPA_PROBE_H
#define SPA_PROBE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads chunks chunk_ids[0 .. n_chunks) of 4096 bytes each (chunk c is bytes
 * [4096 c, 4096 c + 4096) of `base`), every byte once, one 64-lane wave per
 * `chunks_per_wave` chunks (4, 8 or 16) with all of a wave's loads in flight
 * together; writes one folded word per wave to sink[0 .. ceil(n_chunks /
 * chunks_per_wave)). All pointers are device pointers owned by the caller;
 * chunk ids must lie in [0, base_bytes / 4096) (not checked on the device).
 * Returns 0, 1 for bad arguments (nothing launched), 5 for a launch failure.
 * Asynchronous on `stream`. */
int spa_probe_read_chunks(const void* base, size_t base_bytes, const int32_t* chunk_ids, int32_t n_chunks,
                          int32_t chunks_per_wave, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SPA_PROBE_H */
