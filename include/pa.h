/*
 * pa.h -- C ABI of the MI355X (gfx950) paged KV-cache decode library.
 *
 * Device operations, each enqueued on the caller's HIP stream:
 *   pa_decode       single-query attention of every sequence over its KV
 *                   cache, read through its block table (pa_decode_ex: with
 *                   a hint that the batch shares blocks);
 *   pa_prefill      attention of several new tokens per sequence, each over
 *                   the cached tokens up to its own position;
 *   pa_write_cache  write each new token's K and V rows into the slot given by
 *                   a slot mapping;
 *   pa_copy_blocks  whole-block copies, the copy half of copy-on-write;
 *   pa_append_block_tables  record each sequence's newest block in its
 *                   device block-table row after a decode append.
 *   pa_append_block_tables_host  the same, taking the step's lengths and
 *                   slots from host memory in the launch arguments;
 *   pa_write_cache_append_host  that append and the step's cache write in
 *                   one launch.
 *
 * Pages the operations are defined by (cited below by short name):
 *   [aiqz]     aiqz.cc/article/paged-attention-mechanism.html (PagedAttention
 *              tutorial: block table equation, prefix sharing, copy-on-write)
 *   [lihaoran] lihaoran.work/auto-20261007-1900 (mechanism note: the
 *              [5, 1, 7] example, tail-slot count)
 *   [cf-1]     cf-1.com/news/5879632 (engineering blog: block table in shared
 *              memory, prefetch, copy-on-write steps)
 *   [ipipp]    ipipp.com/html/20260817/41684.html ("PagedAttention原理是什么？")
 *
 * Memory layout (all arrays dense, row-major, in device memory owned by the
 * caller; the library never allocates, frees or synchronizes):
 *   k_cache           [num_blocks][num_kv_heads][block_size][head_dim]    elements of `dtype`
 *   v_cache           [num_blocks][num_kv_heads][block_size / T][head_dim][T], T = min(block_size, 16):
 *                     each block's V rows stored as tiles of T tokens, head_dim-major, so
 *                     the V row of (block pid, offset off) is v_cache[pid][kv][off / T][:][off % T]
 *   q, out            [num_seqs][num_heads][head_dim]                   elements of `dtype`
 *                     (pa_prefill: [num_tokens][num_heads][head_dim], the new tokens of
 *                     every sequence in order, delimited by query_start)
 *   query_start       int32 [num_seqs + 1] (pa_prefill only)
 *   k, v (new tokens) [num_tokens][num_kv_heads][head_dim]              elements of `dtype`
 *   block_tables      int32 [num_seqs][max_blocks_per_seq]
 *   context_lens      int32 [num_seqs]
 *   slot_mapping      int32 [num_tokens]; slot = physical_block * block_size + offset
 *   src_dst_pairs     int32 [num_pairs][2]
 * Every data pointer must be 16-byte aligned. `stream` is a hipStream_t
 * (NULL = the null stream) passed as void* so this header needs no HIP header.
 *
 * Errors: every check below is made on the host before anything is launched;
 * a failing call launches nothing and returns a status, and pa_last_error()
 * gives a message for the calling thread. A launch failure returns
 * PA_ERR_HIP. Index contents live in device memory and are not checked on the
 * host; the kernels clamp what they read so that a bad index can never make
 * them touch memory outside the arrays (see each call).
 *
 * Thread safety: the library keeps no state besides two caches filled under a
 * lock: per device, the compute-unit count and LDS sizes; per (device, decode
 * kernel, LDS request), the runtime's occupancy figure. Calls that share a
 * workspace must not overlap.
 *
 * Graph capture: the device calls enqueue kernels only (no allocation,
 * memset, copy or synchronization), so a caller may record them into a HIP
 * graph and replay it. Make one call of each kind and shape on the device
 * before capturing: a call whose cache entries are missing fills them through
 * host queries of the runtime; later calls of the same shape make none. The
 * calls that take host arrays (pa_append_block_tables_host,
 * pa_write_cache_append_host) carry their values in the launch arguments,
 * so a captured call replays the values it was captured with.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 10

typedef enum pa_dtype {
    PA_F32 = 0,  /* IEEE binary32 */
    PA_BF16 = 1, /* bfloat16 */
    PA_F16 = 2   /* IEEE binary16 */
} pa_dtype_t;

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = 1, /* null pointer, negative or inconsistent size, misalignment */
    PA_ERR_UNSUPPORTED = 2, /* valid request the library has no kernel for */
    PA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than pa_decode_workspace_size */
    PA_ERR_HIP = 4,         /* the HIP runtime reported an error */
    PA_ERR_NO_BLOCKS = 5    /* block manager (pa_blocks.h): not enough free blocks */
} pa_status_t;

/* The decode partition kernels (see pa_decode_plan). */
typedef enum pa_decode_kernel {
    PA_DECODE_VALU = 0,      /* vector ALU; one item per workgroup (float32, or one query head per KV head
                                outside the stream split) */
    PA_DECODE_MFMA = 1,      /* matrix cores; one item per workgroup (partitions of more than 128 blocks) */
    PA_DECODE_MFMA_WAVE = 2,  /* matrix cores; one item per wave (partitions of at most 128 blocks, 2 or
                                 more query heads per KV head, when the stream split's cost positions
                                 could pass 2^31: see pa_decode) */
    PA_DECODE_MFMA_STREAM = 3 /* matrix cores; the batch's tiles split evenly over the waves (16-bit
                                 elements, partitions of at most 128 blocks) */
} pa_decode_kernel_t;

/* How pa_decode launches its partition kernel for one shape. */
typedef struct pa_decode_plan {
    pa_decode_kernel_t kernel;
    int partition_size;     /* tokens per partition (partition_size = 0 resolved) */
    int lds_bytes;          /* dynamic LDS per workgroup; the kernels hold no static LDS */
    int ring_slots;         /* item results a workgroup buffers in that LDS before storing them */
    int workgroups_per_cu;  /* resident workgroups per compute unit the LDS allows */
} pa_decode_plan_t;

/* ABI version of the loaded library (PA_ABI_VERSION it was built with). */
int pa_abi_version(void);

/* Static description of a status code. */
const char* pa_status_string(pa_status_t status);

/* Message of the last failed call on the calling thread ("" if none). */
const char* pa_last_error(void);

/*
 * Tokens per context partition that pa_decode uses when the caller passes
 * partition_size = 0, a function of the batch's shape only (host code, no
 * device query). With items = num_seqs * num_kv_heads *
 * ceil(max_context_len / size):
 *   - bfloat16 / float16 (the stream split, or one wave per item):
 *     min(2048, 128 * block_size), halved while items < 2048 (two per wave
 *     of MI355X's 256 compute units);
 *   - float32 (a workgroup reduces an item): 256 * block_size, halved
 *     while items < 512;
 * in both cases not below 512 tokens. Long partitions cost the fewest item
 * switches and merges; the item count keeps every compute unit fed.
 * Returns 0 for invalid arguments (sizes below zero, num_heads,
 * num_kv_heads or block_size not positive, num_heads not a multiple of
 * num_kv_heads, unknown dtype).
 */
int pa_default_partition_size(int num_seqs, int num_heads, int num_kv_heads, int max_context_len, int block_size,
                              pa_dtype_t dtype);

/*
 * Bytes of device workspace pa_decode needs. For the item kernels: one
 * (max, sum, output row) record in float32 per sequence, query head and
 * partition, or 0 when no sequence can span more than one partition
 * (max_context_len <= partition_size). For the stream split (see
 * pa_decode): per wave of its grid (at most 1024), a tail and a head record
 * of every query head of a group and four ints naming the pair of the tail
 * record, whatever the batch (about 4.3 MB at 4 query heads per KV head and
 * head_dim 128). Returns 0 for invalid arguments too. partition_size = 0
 * selects pa_default_partition_size(num_seqs, num_heads, num_kv_heads,
 * max_context_len, block_size, dtype). The workspace is caller-owned device
 * memory with no required contents; calls that share one must not overlap.
 */
size_t pa_decode_workspace_size(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                int max_context_len, int block_size, int partition_size, pa_dtype_t dtype);

/*
 * Host-only planning query: fills *plan with the partition kernel, LDS request
 * and result ring pa_decode would use for this shape on a device whose
 * compute units hold lds_per_cu bytes of LDS, with at most lds_per_workgroup
 * per workgroup (163840 and 163840 on MI355X), when the registers of the
 * kernel allow max_workgroups_per_cu workgroups of 256 threads per compute
 * unit (the matrix-core kernels always run one per compute unit; 1 is always
 * a valid value). No device is queried: pa_decode runs this same computation
 * with its device's values (hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
 * hipDeviceAttributeMaxSharedMemoryPerBlock and the runtime's occupancy).
 * Returns PA_ERR_UNSUPPORTED when no kernel for the shape fits the LDS (the
 * batch's schedule grows with num_seqs); pa_decode then returns the same
 * status without launching. Other arguments and errors as pa_decode's shape
 * checks; the sizes must be positive.
 */
pa_status_t pa_decode_plan(int num_seqs, int num_heads, int num_kv_heads, int head_dim, int max_context_len,
                           int block_size, int partition_size, pa_dtype_t dtype, int lds_per_cu,
                           int lds_per_workgroup, int max_workgroups_per_cu, pa_decode_plan_t* plan);

/*
 * Paged decode attention.
 *
 * For sequence s with L = context_lens[s] and query head h (KV head
 * kv = h / (num_heads / num_kv_heads)), token t in [0, L) lives at physical
 * block pid = block_tables[s][t / block_size], offset off = t % block_size
 * ([aiqz] section 块表映射机制, equation pid/off; [lihaoran] section
 * 块表把逻辑顺序映射到物理位置). With x_t = scale * <q[s][h], k_cache[pid][kv][off]>,
 *     out[s][h] = sum_t exp(x_t - max x) v_cache[pid][kv][off] / sum_t exp(x_t - max x),
 * i.e. ordinary softmax attention over all L visible tokens: the paging
 * changes where the rows live, not the value ([aiqz] 常见误区; [ipipp]
 * 分页式KV缓存的底层设计). L = 0 gives a zero row. Slots at or past L in the
 * last block and table entries past ceil(L / block_size) are never read.
 * Arithmetic is float32; out is rounded to `dtype` (round to nearest even).
 *
 * The context is split into partitions of partition_size tokens that are
 * reduced separately and merged by log-sum-exp; the split changes rounding
 * only. A sequence with a single partition is written directly.
 *
 * Arguments: num_heads must be a multiple of num_kv_heads; num_heads /
 * num_kv_heads must be 1, 2, 4 or 8 (also 16 for bfloat16 / float16);
 * head_dim 64, 128 or 256; block_size a power of two from 4 to 256; with one
 * query head per KV head or float32 elements the block must also hold at
 * least max(1024 / (head_dim * sizeof(dtype)), 4, 16 * head_dim * sizeof(dtype) / 1024)
 * tokens (PA_ERR_UNSUPPORTED names the bound);
 * partition_size (0 = pa_default_partition_size) a multiple of 16 and of block_size with
 * partition_size / block_size <= 512; num_seqs <= 8192;
 * max_blocks_per_seq * block_size >= max_context_len. workspace must hold
 * pa_decode_workspace_size(...) bytes for the same arguments.
 * max_context_len must be >= every context_lens[s]; a longer sequence is
 * clamped to max_context_len tokens. Table entries outside [0, num_blocks)
 * are clamped into that range (wrong values, no fault). q/out must not alias.
 *
 * Work: with 16-bit elements and partitions of at most 128 blocks
 * (pa_decode_plan names the kernel), the batch's 16-key tiles form one
 * stream that a persistent grid divides evenly among its waves; a wave
 * merges the partitions of its stretch of a (sequence, KV head) pair
 * itself, and only pairs split between waves leave records for the merge.
 * The division depends on the batch and on the device's compute-unit count:
 * results repeat bit for bit on one device and differ in rounding only
 * between devices. The stream's cost positions are 32-bit: a batch with
 * num_seqs * num_kv_heads * (4 * ceil(max_context_len / 16) + 3) >= 2^31 - 1
 * runs the item kernels instead. Otherwise the work is split into items of
 * (sequence, KV head, partition) that a persistent grid processes largest
 * first; an item's result does not depend on which workgroup (or wave) ran
 * it.
 */
pa_status_t pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, float scale,
                      int block_size, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                      int num_blocks, int max_blocks_per_seq, int max_context_len,
                      int partition_size, pa_dtype_t dtype, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * The two stages pa_decode runs, exposed with the same arguments so a caller
 * can time them apart: pa_decode == pa_decode_partitions then
 * pa_decode_merge on the same stream. The merge combines per-partition
 * records (m_p, l_p, o_p) of a sequence as M = max m_p, w_p = l_p e^(m_p - M),
 * out = sum w_p o_p / sum w_p, and does nothing for single-partition
 * sequences (with the stream split: the records of the pairs split between
 * waves, and nothing for pairs one wave held whole). Calling
 * pa_decode_merge without a preceding pa_decode_partitions on the same
 * workspace leaves `out` undefined.
 */
pa_status_t pa_decode_partitions(void* out, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_tables,
                                 const int32_t* context_lens, float scale, int block_size,
                                 int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                 int num_blocks, int max_blocks_per_seq, int max_context_len,
                                 int partition_size, pa_dtype_t dtype, void* workspace,
                                 size_t workspace_bytes, void* stream);
pa_status_t pa_decode_merge(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            float scale, int block_size, int num_seqs, int num_heads,
                            int num_kv_heads, int head_dim, int num_blocks,
                            int max_blocks_per_seq, int max_context_len, int partition_size,
                            pa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * pa_decode and pa_decode_partitions with flags; flags = 0 is the plain
 * call. PA_DECODE_SHARED_BLOCKS tells the library that some physical blocks
 * appear in several sequences' tables (prefix sharing, [aiqz] section
 * 前缀共享机制): the stream split then reads K/V tiles of blocks of 16 or
 * more tokens with ordinary loads, which the L2 keeps for the other
 * sequences that list the same blocks, instead of nontemporal (streaming)
 * loads. Results are bit for bit those of the plain call; only the load
 * policy changes. Without sharing the hint is slower (streaming loads suit a
 * batch read once), so pass it only for batches that share. The item
 * kernels ignore it. Unknown flag bits return PA_ERR_INVALID_ARG before any
 * launch.
 */
#define PA_DECODE_SHARED_BLOCKS 1u
pa_status_t pa_decode_ex(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens, float scale,
                         int block_size, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                         int num_blocks, int max_blocks_per_seq, int max_context_len,
                         int partition_size, pa_dtype_t dtype, void* workspace,
                         size_t workspace_bytes, unsigned flags, void* stream);
pa_status_t pa_decode_partitions_ex(void* out, const void* q, const void* k_cache,
                                    const void* v_cache, const int32_t* block_tables,
                                    const int32_t* context_lens, float scale, int block_size,
                                    int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                    int num_blocks, int max_blocks_per_seq, int max_context_len,
                                    int partition_size, pa_dtype_t dtype, void* workspace,
                                    size_t workspace_bytes, unsigned flags, void* stream);

/*
 * pa_decode for callers that cannot allocate: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments,
 * result and errors as pa_decode without the workspace: the split-K records
 * go to a scratch array the library holds in device memory (one copy per GPU
 * it runs on, PA_NOALLOC_SCRATCH_BYTES bytes, kept until the process ends).
 * The call allocates nothing: no hipMalloc or hipFree, no allocating library
 * routine. A shape whose records (pa_decode_workspace_size for the same
 * arguments) exceed the scratch is refused with PA_ERR_UNSUPPORTED before
 * anything is launched. The scratch needs no contents between calls (every
 * record the merge reads is written by the same call), but every call on one
 * GPU uses the same scratch: calls that overlap on one GPU (on different
 * streams, or from several threads) race and give undefined results. The
 * first call on a device looks up the scratch's device address once
 * (hipGetSymbolAddress); make it before capturing a graph.
 */
#define PA_NOALLOC_SCRATCH_BYTES (32u << 20)
pa_status_t pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens, float scale,
                              int block_size, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                              int num_blocks, int max_blocks_per_seq, int max_context_len, int partition_size,
                              pa_dtype_t dtype, void* stream);

/*
 * Paged prefill attention (several new tokens per sequence).
 *
 * Sequence s holds L = context_lens[s] tokens in its blocks; the last
 * M = query_start[s + 1] - query_start[s] of them are new, their K and V
 * already written (pa_write_cache), and their query rows are
 * q[query_start[s] + i], i in [0, M). New token i sits at position
 * p = L - M + i and attends to the tokens at positions 0..p -- everything
 * before it and itself ([lihaoran] section 块表把逻辑顺序映射到物理位置: causal
 * attention covers the visible history, whatever the blocks). With token t
 * read at block_tables[s][t / block_size], offset t % block_size ([aiqz]
 * 块表映射机制) and x_t = scale * <q_row[h], k_t[kv]>,
 *     out[query_start[s] + i][h] = sum_{t <= p} exp(x_t - max x) v_t[kv] / sum_{t <= p} exp(x_t - max x),
 * kv = h / (num_heads / num_kv_heads). M = 1 is the decode of the same
 * sequence. A row whose position would be negative (M > L, an invalid input)
 * is written as zeros. Arithmetic is float32 on MFMA; for bfloat16 and
 * float16 the probabilities are rounded to `dtype` before they weight V (the
 * softmax denominator sums the rounded values), and out is rounded to
 * `dtype`.
 *
 * Arguments: q and out hold num_tokens rows; query_start must be
 * non-decreasing from 0 to at most num_tokens (entries are clamped into
 * [0, num_tokens]). dtype float32, bfloat16 or float16; head_dim 64, 128 or 256;
 * num_heads / num_kv_heads 1, 2, 4, 8 or 16; block_size a power of two from
 * 4 to 256; max_blocks_per_seq * block_size >= max_context_len.
 * max_query_len must be >= every M and max_context_len >= every L: a longer
 * sequence has only its last max_query_len rows computed, over at most
 * max_context_len tokens. Table entries past ceil(L / block_size) are never
 * read; entries outside [0, num_blocks) are clamped. q/out must not alias.
 * No workspace is needed. num_seqs = 0 or max_query_len = 0 is a no-op.
 *
 * Work is split into (query tile, sequence, KV head) workgroups; a tile's
 * result does not depend on the others.
 */
pa_status_t pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens,
                       const int32_t* query_start, float scale, int block_size, int num_seqs,
                       int num_tokens, int num_heads, int num_kv_heads, int head_dim,
                       int num_blocks, int max_blocks_per_seq, int max_query_len,
                       int max_context_len, pa_dtype_t dtype, void* stream);

/*
 * Cache write: for every token i with 0 <= slot_mapping[i] < num_blocks *
 * block_size, with pid = slot / block_size and off = slot % block_size,
 *     k_cache[pid][kv][off][:] = k[i][kv][:]  and  the V row of (pid, off) = v[i][kv][:]
 * for every KV head kv -- the step that stores a sequence's newest token after
 * any copy ([aiqz] 前缀共享机制), addressed as in [aiqz] 块表映射机制.
 * Elements are copied as raw bits (NaN payloads included). A negative slot
 * skips the token; a slot past the pool is skipped too. Slots must be
 * distinct (two tokens writing one slot leave either value). A K/V row
 * (head_dim * element size) must be a multiple of 16 bytes and at most
 * 32768 bytes (PA_ERR_UNSUPPORTED otherwise). num_tokens = 0 is a no-op.
 * Tokens at consecutive offsets of a block are written fastest. The stores
 * bypass the cache, so a decode launched right after reads them from memory.
 */
pa_status_t pa_write_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                           const int32_t* slot_mapping, int num_tokens, int num_kv_heads,
                           int head_dim, int block_size, int num_blocks, pa_dtype_t dtype,
                           void* stream);

/*
 * Block copy: for every pair (src, dst) = src_dst_pairs[i], copy the whole
 * block -- all KV heads, all block_size slots (stale ones too) -- of both
 * caches: k_cache[dst] = k_cache[src], v_cache[dst] = v_cache[src], as raw
 * bits. This is the copy of copy-on-write ([aiqz] 前缀共享机制: allocate, copy
 * the old block, then write; [cf-1] 4.2). Pairs act as if applied at once:
 * every dst must be distinct and no dst may also be a src (otherwise the
 * result is unspecified). A pair with an id outside [0, num_blocks) is
 * skipped. num_pairs = 0 is a no-op.
 */
pa_status_t pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_dst_pairs,
                           int num_pairs, int num_kv_heads, int block_size, int head_dim,
                           int num_blocks, pa_dtype_t dtype, void* stream);

/*
 * Multi-layer forms: one launch applies the same slot mapping, or the same
 * copy pairs, to the caches of num_layers layers -- a token's K/V rows go
 * into every layer's cache at its one slot, and a copy-on-write duplicates a
 * block in every layer ([aiqz] 前缀共享机制: the copy is of the whole block).
 * Layer l's caches follow layer l - 1's in one allocation:
 *   k_cache  [num_layers][num_blocks][num_kv_heads][block_size][head_dim]
 *   v_cache  [num_layers][num_blocks][num_kv_heads][block_size / T][head_dim][T]
 *   k, v     [num_layers][num_tokens][num_kv_heads][head_dim]   (write only)
 * Each layer's result is exactly what pa_write_cache / pa_copy_blocks would
 * give on that layer's slice, with the same argument rules; num_layers = 1
 * is those calls, num_layers = 0 a no-op, at most 65535 layers
 * (PA_ERR_UNSUPPORTED beyond).
 */
/*
 * Keep device block tables in step with a decode append, without sending
 * rows from the host: for each sequence i with L = context_lens[i] >= 1 and
 * slot_mapping[i] >= 0, block_tables[i][(L - 1) / block_size] =
 * slot_mapping[i] / block_size -- the physical block of its newest token
 * (token L - 1) in its table row ([aiqz] section 块表映射机制: a sequence
 * takes a new block when its last one is full; [aiqz] section 前缀共享机制:
 * a copy-on-write replaces the block the write goes to). Every other entry
 * is left as it is. block_tables is int32 [num_seqs][max_blocks_per_seq],
 * context_lens and slot_mapping int32 [num_seqs] (lengths including the new
 * token), all device memory. A column past max_blocks_per_seq skips the
 * sequence. block_size a power of two up to 256.
 */
pa_status_t pa_append_block_tables(int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                                   const int32_t* slot_mapping, int num_seqs, int block_size, void* stream);

/*
 * pa_append_block_tables with the step's lengths and slots read from HOST
 * memory: host_context_lens and host_slot_mapping (int32 [num_seqs], any host
 * memory) are read during the call and reach the device inside the kernel's
 * launch arguments, so no copy command or staging buffer is involved and the
 * caller may reuse both arrays as soon as the call returns. The kernel also
 * stores them to context_lens_out and slot_mapping_out (int32 [num_seqs],
 * device memory), where the step's cache write and decode read them. Same
 * table update, argument rules and errors as pa_append_block_tables (the
 * host arrays need no particular alignment); one launch per 448 sequences.
 */
pa_status_t pa_append_block_tables_host(int32_t* block_tables, int max_blocks_per_seq,
                                        const int32_t* host_context_lens, const int32_t* host_slot_mapping,
                                        int32_t* context_lens_out, int32_t* slot_mapping_out, int num_seqs,
                                        int block_size, void* stream);

/*
 * A decode step's table append and cache write in one launch (per 448
 * sequences): the same result as
 *     pa_append_block_tables_host(block_tables, max_blocks_per_seq, host_context_lens, host_slot_mapping,
 *                                 context_lens_out, slot_mapping_out, num_seqs, block_size, stream)
 * followed by
 *     pa_write_cache(k, v, k_cache, v_cache, slot_mapping_out, num_seqs, num_kv_heads, head_dim,
 *                    block_size, num_blocks, dtype, stream)
 * ([aiqz] 块表映射机制 and 前缀共享机制: the newest token's block enters its
 * table row, the token is written into its slot). k, v are
 * [num_seqs][num_kv_heads][head_dim], row i sequence i's newest token. The
 * host arrays are read during the call and travel in the launch arguments
 * (the write takes its slots from there), so the caller may reuse them as
 * soon as the call returns. Argument rules and errors as those two calls'.
 */
pa_status_t pa_write_cache_append_host(const void* k, const void* v, void* k_cache, void* v_cache,
                                       int32_t* block_tables, int max_blocks_per_seq,
                                       const int32_t* host_context_lens, const int32_t* host_slot_mapping,
                                       int32_t* context_lens_out, int32_t* slot_mapping_out, int num_seqs,
                                       int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                       pa_dtype_t dtype, void* stream);

pa_status_t pa_write_cache_layers(const void* k, const void* v, void* k_cache, void* v_cache,
                                  const int32_t* slot_mapping, int num_tokens, int num_layers,
                                  int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                  pa_dtype_t dtype, void* stream);
pa_status_t pa_copy_blocks_layers(void* k_cache, void* v_cache, const int32_t* src_dst_pairs,
                                  int num_pairs, int num_layers, int num_kv_heads, int block_size,
                                  int head_dim, int num_blocks, pa_dtype_t dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
