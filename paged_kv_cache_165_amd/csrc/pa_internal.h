// Internal launch interface between the C-ABI entry points (pa_api.hip) and
// the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include "pa.h"

namespace pa {

// Set the calling thread's pa_last_error() message and return `st`.
pa_status_t fail(pa_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Table entries (blocks) one decode partition may span: an item stages that
// slice of its block table in LDS.
constexpr int kMaxTableSlice = 512;
// Partitions of at most this many blocks run on the MFMA kernels that give
// each wave items of its own (bfloat16 / float16 with grouped query heads).
constexpr int kWaveSlice = 128;
// Waves of the stream kernel's grid at most (256 compute units x 4 waves on
// MI355X); its workspace holds one extra record per wave.
constexpr int kMaxStreamWaves = 1024;

// Everything one decode launch needs. Pointers are device pointers.
struct DecodeParams {
    void* out;
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    const int32_t* context_lens;
    float* ws_m;        // [S][Hq][pmax]  running max per partition (log2 units)
    float* ws_l;        // [S][Hq][pmax]  softmax denominator per partition
    float* ws_o;        // [S][Hq][pmax][D] normalised partial output
    int* ws_meta;       // stream kernel: [kMaxStreamWaves][4] (sequence, KV head, later waves, 0) of the
                        //   pair each wave's tail record belongs to (later waves = 0: no tail record)
    float* ws_xm;       // stream kernel: [2][kMaxStreamWaves][G] records of pairs split between
    float* ws_xl;       //   waves (a wave's tail, then its head): max, sum,
    float* ws_xo;       //   and [2][kMaxStreamWaves][G][D] normalised output
    int stream;         // 1: the records are the stream kernel's
    float scale_log2;   // scale * log2(e): logits are kept in base-2 units
    int num_seqs;
    int num_heads;
    int num_kv_heads;
    int group;          // num_heads / num_kv_heads
    int num_blocks;
    int max_blocks;     // max_blocks_per_seq (row stride of block_tables)
    int max_ctx;        // host bound on context lengths
    int part;           // tokens per partition
    int pmax;           // ceil(max_ctx / part), >= 1
    int log2_bs;        // block size = 1 << log2_bs
    int log2_vt;        // tokens per transposed V tile = min(block size, 16)
    int ring_slots;     // item results a workgroup buffers in LDS before storing them
    int keep_tiles;     // 1: the stream kernel reads K/V tiles with ordinary loads, which the L2 keeps for
                        //   other readers of shared blocks; 0: nontemporal (streaming) loads
};

// Everything one prefill launch needs. Pointers are device pointers.
struct PrefillParams {
    void* out;
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    const int32_t* context_lens;
    const int32_t* query_start;  // [num_seqs + 1]
    float scale_log2;            // scale * log2(e)
    int num_seqs;
    int num_heads;
    int num_kv_heads;
    int num_blocks;
    int max_blocks;     // max_blocks_per_seq (row stride of block_tables)
    int max_ctx;        // host bound on context lengths
    int max_q;          // host bound on new tokens per sequence
    int num_tokens;     // rows of q and out
    int log2_bs;
    int log2_vt;
    int pair_major;     // 1: each XCD runs all query tiles of a (sequence, KV head) pair together
};

// Tokens per transposed V tile: V rows of a block are stored as tiles of
// this many tokens, head_dim-major.
inline int v_tile_tokens(int block_size) { return block_size < 16 ? block_size : 16; }

// log2 of a power of two
inline int ilog2(int x) {
    int r = 0;
    while ((1 << r) < x) ++r;
    return r;
}

// Launch `kern` and return the status of this launch alone. hipLaunchKernel
// reports its own error; checking hipGetLastError() after a launch would also
// return (and clear) an error left behind by an earlier, unrelated HIP call
// on the thread. The arguments are converted to the kernel's parameter types
// first and passed by address, as hipLaunchKernel expects.
template <typename... P, typename... A>
hipError_t launch_kernel(void (*kern)(P...), dim3 grid, dim3 block, size_t smem, hipStream_t stream,
                         A&&... a) {
    static_assert(sizeof...(P) == sizeof...(A), "one argument per kernel parameter");
    std::tuple<P...> args(std::forward<A>(a)...);
    return std::apply(
        [&](auto&... x) {
            void* ptrs[] = {static_cast<void*>(&x)...};
            return hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, ptrs, smem, stream);
        },
        args);
}

// What a launch needs to know of the current device (read once per device).
struct DeviceInfo {
    int id;
    int cus;            // compute units
    size_t lds_per_cu;  // LDS bytes of one compute unit
    size_t lds_per_wg;  // LDS bytes one workgroup may hold
};

// The decode partition kernel a launch runs and its LDS (see pa_decode_plan
// in pa.h): which kernel, the dynamic LDS per workgroup (the kernels hold no
// static LDS), the result-ring slots inside it and the workgroups per compute
// unit.
struct DecodePlan {
    pa_decode_kernel_t kernel;
    size_t smem;
    int ring_slots;
    int resident;
};

// Host-only: no device is queried. max_per_cu is the most workgroups per
// compute unit the registers of the VALU kernel allow (ignored for the MFMA
// kernels, which run one per compute unit). PA_ERR_UNSUPPORTED if no kernel
// for the shape fits the LDS.
pa_status_t plan_decode(pa_dtype_t dt, int head_dim, int group, int num_seqs, int part_blocks, bool stream,
                        size_t lds_per_cu, size_t lds_per_wg, int max_per_cu, DecodePlan* out);

// Return hipSuccess or the launch error.
hipError_t launch_decode_partitions(const DecodeParams& p, pa_dtype_t dt, int head_dim, const DeviceInfo& dv,
                                    hipStream_t stream);
hipError_t launch_decode_merge(const DecodeParams& p, pa_dtype_t dt, int head_dim,
                               hipStream_t stream);
bool decode_supported(pa_dtype_t dt, int head_dim, int group);
// Whether a shape runs the stream kernel, which splits the batch's tiles
// evenly over the grid's waves (its workspace layout differs): 16-bit
// elements, any group and block size (decode_stream_shape), partitions of at
// most a wave's table slice and cost positions in 31 bits.
bool decode_stream_shape(pa_dtype_t dt, int block_size);
bool decode_stream(pa_dtype_t dt, int group, int block_size, int part, int num_seqs, int num_kv_heads, int max_ctx);
bool decode_uses_mfma(pa_dtype_t dt, int group);
// Whether a partition of `part_blocks` blocks runs one item per wave.
bool decode_wave_items(pa_dtype_t dt, int group, int part_blocks);
int decode_min_block_size(pa_dtype_t dt, int head_dim, int group);

bool prefill_supported(pa_dtype_t dt, int head_dim, int group);
hipError_t launch_prefill(const PrefillParams& p, pa_dtype_t dt, int head_dim, int group,
                          hipStream_t stream);

// num_layers caches laid out one after another (see pa_write_cache_layers)
hipError_t launch_write_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                              const int32_t* slots, int num_tokens, int num_layers, int num_kv_heads,
                              int head_dim, int elem_bytes, int block_size, int num_blocks,
                              hipStream_t stream);
hipError_t launch_table_append(int32_t* tables, int max_blocks, const int32_t* lens, const int32_t* slots,
                               int num_seqs, int block_size, hipStream_t stream);
// Sequences per launch of the append that carries lengths and slots in its
// launch arguments (two int32 arrays of this size fit in the 4 KB limit).
constexpr int kStageSeqs = 448;
hipError_t launch_stage_append(int32_t* tables, int max_blocks, const int32_t* host_lens,
                               const int32_t* host_slots, int32_t* lens_out, int32_t* slots_out, int num_seqs,
                               int block_size, hipStream_t stream);
// launch_stage_append followed by launch_write_cache of the step's one token
// per sequence, in one launch per kStageSeqs sequences
hipError_t launch_write_stage(const void* k, const void* v, void* k_cache, void* v_cache, int32_t* tables,
                              int max_blocks, const int32_t* host_lens, const int32_t* host_slots, int32_t* lens_out,
                              int32_t* slots_out, int num_seqs, int num_kv_heads, int head_dim, int elem_bytes,
                              int block_size, int num_blocks, hipStream_t stream);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int num_pairs,
                              int num_layers, size_t block_bytes, int num_blocks, hipStream_t stream);

}  // namespace pa
