/*
 * The library's C ABI driven from plain C99, with no GPU: version, status
 * strings, the host-side default partition, argument rejection before any
 * launch, and the block manager's copy-on-write append on a shared partly
 * filled block (aiqz.cc tutorial, section 前缀共享机制: of the sequences that
 * share a partly filled block, each writer but the last copies it first).
 * Prints "ok" and exits 0 when every check holds.
 */
#include <stdio.h>
#include <string.h>

#include "pa.h"
#include "pa_blocks.h"
#include "pa_probe.h"

#define CHECK(cond)                                                     \
    do {                                                                \
        if (!(cond)) {                                                  \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            return 1;                                                   \
        }                                                               \
    } while (0)

int main(void) {
    pa_block_manager_t* bm = NULL;
    int64_t seqs[2] = {0, 1};
    int32_t slots[2], pairs[4], tables[2 * 3], lens[2];
    int npairs = -1;

    CHECK(pa_abi_version() == PA_ABI_VERSION);
    CHECK(pa_status_string(PA_OK) != NULL && pa_status_string(PA_ERR_INVALID_ARG) != NULL);
    /* 256 sequences, 32 query and 8 KV heads, up to 8192 tokens, blocks of 16, bf16 */
    CHECK(pa_default_partition_size(256, 32, 8, 8192, 16, PA_BF16) == 2048);

    /* a null pointer is rejected on the host, before anything is launched */
    CHECK(pa_write_cache(NULL, NULL, NULL, NULL, NULL, 4, 8, 128, 16, 64, PA_BF16, NULL) == PA_ERR_INVALID_ARG);
    CHECK(strstr(pa_last_error(), "null") != NULL);
    CHECK(pa_probe_read_tiles(NULL, NULL, NULL, 4, 64, 4096, 2, 256, NULL, NULL) == PA_ERR_INVALID_ARG);

    /* the host-only launch plan of the GQA batch-256 shape: the stream split */
    {
        pa_decode_plan_t plan;
        CHECK(pa_decode_plan(256, 32, 8, 128, 8192, 16, 0, PA_BF16, 163840, 163840, 1, &plan) == PA_OK);
        CHECK(plan.kernel == PA_DECODE_MFMA_STREAM && plan.partition_size == 2048);
        CHECK(plan.lds_bytes > 0 && plan.lds_bytes <= 163840 && plan.ring_slots >= 4);
    }

    /* 8 blocks of 4 tokens; sequence 0 holds 10 tokens (blocks 0, 1, 2, the
     * last with 2 of 4 slots used), sequence 1 shares all 10 */
    CHECK(pa_bm_create(8, 4, NULL, &bm) == PA_OK);
    CHECK(pa_bm_prefill(bm, 0, 10) == PA_OK);
    CHECK(pa_bm_share(bm, 1, 0, 10) == PA_OK);
    CHECK(pa_bm_refcount(bm, 2) == 2 && pa_bm_num_free(bm) == 5);
    /* one append each: sequence 0 copies the shared block 2 into block 3 and
     * writes there (slot 3 * 4 + 2); sequence 1, now its only holder, writes
     * in place (slot 2 * 4 + 2) */
    CHECK(pa_bm_append(bm, seqs, 2, slots, pairs, &npairs) == PA_OK);
    CHECK(npairs == 1 && pairs[0] == 2 && pairs[1] == 3);
    CHECK(slots[0] == 14 && slots[1] == 10);
    CHECK(pa_bm_block_tables(bm, seqs, 2, tables, 3, -1, lens) == PA_OK);
    CHECK(tables[0] == 0 && tables[1] == 1 && tables[2] == 3);
    CHECK(tables[3] == 0 && tables[4] == 1 && tables[5] == 2);
    CHECK(lens[0] == 11 && lens[1] == 11);
    CHECK(pa_bm_refcount(bm, 0) == 2 && pa_bm_refcount(bm, 2) == 1 && pa_bm_refcount(bm, 3) == 1);
    CHECK(pa_bm_check(bm) == PA_OK);
    pa_bm_destroy(bm);
    printf("ok\n");
    return 0;
}
