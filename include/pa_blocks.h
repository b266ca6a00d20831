/*
 * pa_blocks.h -- C ABI of the host-side block manager: the bookkeeping that
 * produces the block tables, slot mappings and copy-on-write pairs the device
 * calls of pa.h consume.
 *
 * Pages the behaviour follows (cited by the short names of pa.h):
 *   [aiqz] 分页核心思想: a sequence takes a new block only when its last block
 *          is full (the block count is the ceiling of tokens / block size);
 *   [aiqz] 前缀共享机制 and [cf-1] 4.2: sequences share prefix blocks by
 *          reference count; the first write into a shared block takes a new
 *          block, copies the old one into it, writes the token there and
 *          drops one reference from the old block;
 *   [cf-1] 3.2: a freed sequence's mapping is removed, then each of its
 *          blocks loses one reference and returns to the free list at zero;
 *   [cf-1] 4.3: a consistency check of every reference count against the
 *          tables;
 *   [aiqz] Python 演示: with the default free order the lowest free id is
 *          handed out first, and the demo's script ends in the state the demo
 *          describes (11 blocks without sharing, 5 with it).
 *
 * The manager is plain host memory and host code; it never touches the GPU.
 * It is not thread-safe: calls on one manager must not overlap. Sequence ids
 * are any 64-bit integers chosen by the caller. Statuses and pa_last_error()
 * are those of pa.h; a failing call leaves the manager unchanged.
 */
#ifndef PA_BLOCKS_H
#define PA_BLOCKS_H

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager_t;

/*
 * A manager of num_blocks blocks of block_size tokens. free_order (nullable)
 * lists every block id once, in the order the free list hands them out;
 * NULL means 0, 1, 2, ... Blocks freed later go to the back of the list.
 * PA_ERR_INVALID_ARG for sizes <= 0, for num_blocks * block_size above
 * INT32_MAX (slots are int32), or a free_order that is not a permutation of
 * [0, num_blocks).
 */
pa_status_t pa_bm_create(int num_blocks, int block_size, const int32_t* free_order,
                         pa_block_manager_t** out);
void pa_bm_destroy(pa_block_manager_t* bm);

/* A new sequence holding num_tokens >= 0 tokens in ceil(num_tokens /
 * block_size) fresh blocks. PA_ERR_INVALID_ARG if seq exists,
 * PA_ERR_NO_BLOCKS if the free list is too short. */
pa_status_t pa_bm_prefill(pa_block_manager_t* bm, int64_t seq, int num_tokens);

/* A new sequence holding the first num_tokens tokens of src: it takes the
 * first ceil(num_tokens / block_size) blocks of src by reference (a fork for
 * parallel sampling, or a shared prompt prefix). */
pa_status_t pa_bm_share(pa_block_manager_t* bm, int64_t seq, int64_t src, int num_tokens);

/*
 * Reserve the slot of the next token of each of the n distinct sequences
 * seqs[0..n), in order: slots[i] = pid * block_size + offset. A sequence
 * whose last block is full takes a new block; one whose last block is
 * shared (reference count > 1) takes a new block, and the pair (old, new)
 * -- the copy the caller must make before writing the token -- is appended
 * to pairs (int32 [n][2]); *num_pairs gets their count. Of R sequences that
 * share a partly filled last block, the first R - 1 to append copy it and
 * the last one writes in place. All or nothing: PA_ERR_NO_BLOCKS (nothing
 * reserved) when the batch needs more free blocks than there are,
 * PA_ERR_INVALID_ARG for an unknown or repeated sequence.
 */
pa_status_t pa_bm_append(pa_block_manager_t* bm, const int64_t* seqs, int n, int32_t* slots,
                         int32_t* pairs, int* num_pairs);

/* Forget a sequence and release its blocks. */
pa_status_t pa_bm_free(pa_block_manager_t* bm, int64_t seq);

/*
 * Block tables and context lengths of n sequences, ready for pa_decode:
 * row i of tables (int32 [n][max_blocks]) gets the sequence's blocks and
 * `pad` in the rest; context_lens[i] its token count. PA_ERR_INVALID_ARG for
 * an unknown sequence or one with more than max_blocks blocks.
 */
pa_status_t pa_bm_block_tables(const pa_block_manager_t* bm, const int64_t* seqs, int n,
                               int32_t* tables, int max_blocks, int32_t pad, int32_t* context_lens);

/* Counts (-1 for a bad block id or an unknown sequence). */
int pa_bm_num_free(const pa_block_manager_t* bm);
int pa_bm_blocks_in_use(const pa_block_manager_t* bm);
int pa_bm_refcount(const pa_block_manager_t* bm, int block);
int64_t pa_bm_seq_tokens(const pa_block_manager_t* bm, int64_t seq);
/* Blocks the live sequences would need without sharing. */
int64_t pa_bm_blocks_without_sharing(const pa_block_manager_t* bm);

/* [cf-1] 4.3: every reference count equals the number of table entries that
 * name the block, and exactly the blocks with count 0 are on the free list,
 * once each. PA_OK, or PA_ERR_INVALID_ARG with the first violation. */
pa_status_t pa_bm_check(const pa_block_manager_t* bm);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCKS_H */
