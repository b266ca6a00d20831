/*
 * pa_probe.h -- bandwidth probe of libpa.so, a measurement aid beside the
 * attention library (include/pa.h), not part of the attention path.
 *
 * Paged decode reads, for every (sequence, KV head), the K tile and the V
 * tile of each block in the sequence's table: tiles of block_size * head_dim
 * elements at scattered places of two cache arrays ([aiqz] section 块表映射机制:
 * a sequence's blocks are anywhere in the pool; [cf-1] 2.2: the lookup costs
 * an indirection per block). pa_probe_read_tiles reads exactly such a list of
 * tiles with the decode's loads (nontemporal 16-byte vector loads, one tile
 * pair per step of a wave) and does no arithmetic on them beyond folding the
 * bytes into a checksum, so its rate is the most the access pattern itself
 * allows on the device: the ceiling the decode is measured against next to
 * the HBM peak.
 *
 * [aiqz]  aiqz.cc/article/paged-attention-mechanism.html
 * [cf-1]  cf-1.com/news/5879632
 */
#ifndef PA_PROBE_H
#define PA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read tile pairs: for i in [0, num_tiles), the tile_bytes bytes at
 * k_cache + t * tile_bytes and at v_cache + t * tile_bytes, t = tiles[i]
 * (an index of a (block, KV head) tile: block * num_kv_heads + kv_head).
 * Indices outside [0, num_cache_tiles) are clamped into it. The list is split
 * into equal contiguous runs, one per wave of `workgroups` workgroups of 256
 * threads; each wave keeps `tiles_in_flight` (1, 2 or 4) tile pairs loading
 * at once. sink (device memory, 16 * 256 * workgroups bytes) receives each
 * thread's checksum so that no load can be dropped.
 * tile_bytes: a multiple of 1024 up to 8192. Pointers 16-byte aligned,
 * device memory owned by the caller; enqueued on `stream`.
 * Errors: PA_ERR_INVALID_ARG / PA_ERR_UNSUPPORTED before any launch,
 * PA_ERR_HIP for a launch failure.
 */
pa_status_t pa_probe_read_tiles(const void* k_cache, const void* v_cache, const int32_t* tiles, int num_tiles,
                                int num_cache_tiles, int tile_bytes, int tiles_in_flight, int workgroups,
                                void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H */
