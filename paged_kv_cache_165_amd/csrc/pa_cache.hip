// Cache maintenance kernels for gfx950: the per-token write through a slot
// mapping and the whole-block copy of copy-on-write.
//
// Both move raw bits and never convert, so the result is bit-exact whatever
// the element type (NaN payloads included): K rows and whole blocks as 16-byte
// vectors, V elements one by one into their transposed tile. The write
// stores a sequence's newest token; the copy duplicates a shared block into a
// freshly allocated one before a sharer writes into it, the copy half of
// copy-on-write (aiqz.cc tutorial, section 前缀共享机制; cf-1.com blog, 4.2).
// The slot of a token is its (physical block, offset) pair of the block-table
// equation (aiqz.cc, section 块表映射机制) flattened as pid * B + off.

#include <algorithm>
#include <cstring>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// LDS row of the write kernel's V staging, in elements: head_dim plus
// padding that makes the row an odd number of 32-bit words, so that lanes
// reading one element of 16 consecutive rows hit 16 different banks.
__host__ __device__ constexpr int write_lds_row(int head_dim, int elem_bytes) {
    return head_dim + (elem_bytes == 2 ? 2 : 1);
}

// One workgroup per (chunk of up to 16 consecutive tokens, KV head, layer).
// Layer z reads its new rows at k + z * num_tokens * Hkv * D (the same for v)
// and writes the caches at kc + z * layer_blocks * Hkv * B * D (the same for
// vc); with one layer the strides are never used.
// K: each token's row is one contiguous run in the cache, copied as 16-byte
// vectors. V: the cache holds each block's rows as tiles of vt tokens stored
// head_dim-major ([NB][Hkv][B/vt][D][vt]), so element d of a token at offset
// off goes to row d, column off % vt of its tile, and a tile row is only
// vt elements (32 bytes for 16 bf16 tokens). HBM writes such a row at full
// speed only when it is written whole: two workgroups writing two parts of
// one row at different times cost nearly twice as much (measured on MI355X:
// 64k tokens in runs that start at a tile boundary, 80 us; the same runs
// shifted by a few slots, 144 us). The V rows therefore go by runs: a run is
// a stretch of slot-mapping entries whose slots are consecutive within one
// tile (at most vt tokens), and the workgroup whose chunk holds a run's
// first entry writes the whole run, reaching up to vt - 1 entries into the
// next chunk, whose workgroup skips them. The V rows of those tokens are
// staged in LDS and written with the token index fastest across lanes, so a
// run that fills a tile leaves the wave as whole tile rows (the staging
// window holds 2^log2_win = 32 tokens). Rows too wide for 32 staged tokens
// in 64 KB of LDS go by plain chunks instead: log2_win = log2_chunk, 16
// entries or fewer so that a chunk's rows fit in 32 KB, and every workgroup
// writes exactly its chunk's V rows. Slots outside [0, pool_slots) skip the
// token (and end any run).

template <typename EW>
__device__ __forceinline__ void write_tokens(const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                                             u32x4* __restrict__ kc, EW* __restrict__ vc,
                                             const int32_t* __restrict__ slots, int num_tokens, int num_kv_heads,
                                             int head_dim, int row16, int log2_bs, int log2_vt, int log2_chunk,
                                             int log2_win, long long pool_slots) {
    constexpr int E = sizeof(EW);
    {
        // this workgroup's layer: pool_slots is also the cache's layer
        // stride in slots (num_blocks * B)
        const size_t z = blockIdx.z;
        const size_t new_el = static_cast<size_t>(num_tokens) * num_kv_heads * row16;  // in 16-byte vectors
        const size_t cache_el = static_cast<size_t>(pool_slots) * num_kv_heads * row16;
        k += z * new_el;
        v += z * new_el;
        kc += z * cache_el;
        vc += z * cache_el * (16 / E);
    }
    extern __shared__ __align__(16) unsigned char smem[];
    const int chunk = 1 << log2_chunk;
    const bool runs = log2_win > log2_chunk;
    const int ld = write_lds_row(head_dim, E);  // padded row (elements): odd dword stride
    EW* vs = reinterpret_cast<EW*>(smem);      // [2^log2_win][ld]
    const int i0 = blockIdx.x << log2_chunk;
    const int kvh = blockIdx.y;
    const int n = min(chunk, num_tokens - i0);
    const int bs = 1 << log2_bs, vt = 1 << log2_vt;
    const int lane = threadIdx.x & 63;

    // Every wave holds the slot window in its lanes: lane j has the slot of
    // entry i0 - 1 + j (j <= chunk + 16; -1 outside the mapping or the pool).
    int my_slot = -1;
    if (lane <= chunk + 16) {
        const int i = i0 - 1 + lane;
        const int sv = i >= 0 && i < num_tokens ? slots[i] : -1;
        my_slot = (sv < 0 || static_cast<long long>(sv) >= pool_slots) ? -1 : sv;
    }
    auto slot_of = [&](int j) { return __shfl(my_slot, j); };  // slot of entry i0 - 1 + j
    // This chunk's V tokens: from its first run start (skipping p entries
    // that continue a run of the chunk before) to the end of its last run
    // (q entries into the next chunk). One ballot evaluates whether entry
    // i0 - 1 + j continues the run of the entry before it, for every j at
    // once; the next workgroup finds p = q on the same slots.
    int p = 0, q = 0;
    {
        const int prev = __shfl_up(my_slot, 1);
        const bool c = lane >= 1 && lane <= chunk + 16 && prev >= 0 && my_slot >= 0 && my_slot == prev + 1 &&
                       (my_slot & (vt - 1)) != 0;
        const unsigned long long mask = __ballot(c);
        if (runs) {
            p = min(n, __builtin_ctzll(~(mask >> 1)));
            if (n == chunk && p < n) q = min(vt - 1, __builtin_ctzll(~(mask >> (1 + n))));
        }
    }
    const int m = n - p + q;  // V tokens, at most chunk + vt - 1 <= 2^log2_win

    // their rows, staged in LDS (row t: entry i0 + p + t)
    for (int c = threadIdx.x; c < m * row16; c += blockDim.x) {
        const int t = c / row16;
        const int r = c - t * row16;
        const u32x4 w = v[(static_cast<size_t>(i0 + p + t) * num_kv_heads + kvh) * row16 + r];
        uint32_t* dst = reinterpret_cast<uint32_t*>(vs + static_cast<size_t>(t) * ld) + 4 * r;
        dst[0] = w.x;
        dst[1] = w.y;
        dst[2] = w.z;
        dst[3] = w.w;
    }

    // All stores are nontemporal. A token's V elements touch every line of
    // its tile, each partially; left dirty in L2, such lines slow down the
    // decode that reads them next (measured: +12 us on the batch-256
    // grouped-query decode after its 256 one-token writes). Measured on
    // MI355X against ordinary stores, and against K rows loaded before the
    // barrier, this is the fastest both for one new token per sequence and
    // for long runs of consecutive tokens.
    for (int c = threadIdx.x; c < ((n * row16 + 63) & ~63); c += blockDim.x) {
        const int t = c / row16;
        const int slot = slot_of(1 + min(t, n - 1));  // every lane takes part in the shuffle
        if (c >= n * row16 || slot < 0) continue;
        const int r = c - t * row16;
        const int pid = slot >> log2_bs;
        const int off = slot & (bs - 1);
        __builtin_nontemporal_store(k[(static_cast<size_t>(i0 + t) * num_kv_heads + kvh) * row16 + r],
                                    kc + ((static_cast<size_t>(pid) * num_kv_heads + kvh) * bs + off) * row16 + r);
    }
    // lanes per token group: 16 unless more than 16 tokens are to be
    // written (a group of 16 lanes stores a whole tile row of 16 tokens, and
    // a wave four consecutive rows); this thread's token is the same in
    // every pass below (blockDim is a multiple of the group)
    const int log2_tw = m > 16 ? log2_win : min(log2_win, 4);
    const int t = threadIdx.x & ((1 << log2_tw) - 1);
    const int slot = slot_of(1 + p + min(t, chunk + 15 - p));
    __syncthreads();
    if (t >= m || slot < 0) return;
    const EW* vsrc = vs + static_cast<size_t>(t) * ld;
    const int pid = slot >> log2_bs;
    const int off = slot & (bs - 1);
    EW* vrow = vc + (static_cast<size_t>(pid) * num_kv_heads + kvh) * bs * head_dim +
               static_cast<size_t>(off >> log2_vt) * head_dim * vt + (off & (vt - 1));
    for (int e = threadIdx.x; e < (head_dim << log2_tw); e += blockDim.x) {
        const int d = e >> log2_tw;
        __builtin_nontemporal_store(vsrc[d], vrow + static_cast<size_t>(d) * vt);
    }
}

template <typename EW>
__global__ __launch_bounds__(256) void pa_write_kernel(const u32x4* __restrict__ k,
                                                       const u32x4* __restrict__ v,
                                                       u32x4* __restrict__ kc,
                                                       EW* __restrict__ vc,
                                                       const int32_t* __restrict__ slots,
                                                       int num_tokens, int num_kv_heads, int head_dim,
                                                       int row16, int log2_bs, int log2_vt, int log2_chunk,
                                                       int log2_win, long long pool_slots) {
    write_tokens<EW>(k, v, kc, vc, slots, num_tokens, num_kv_heads, head_dim, row16, log2_bs, log2_vt, log2_chunk,
                     log2_win, pool_slots);
}

// grid (pairs, 2, layers): y = 0 copies K, y = 1 copies V, z is the layer
// (its caches start z * num_blocks * block16 vectors in). A block is
// contiguous ([Hkv][B][D]), so the copy is one linear run of block16 vectors.
__global__ __launch_bounds__(256) void pa_copy_kernel(u32x4* __restrict__ kc, u32x4* __restrict__ vc,
                                                      const int32_t* __restrict__ pairs,
                                                      size_t block16, int num_blocks) {
    const int i = blockIdx.x;
    const int src = pairs[2 * i];
    const int dst = pairs[2 * i + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
    u32x4* c = (blockIdx.y == 0 ? kc : vc) + static_cast<size_t>(blockIdx.z) * num_blocks * block16;
    const u32x4* from = c + static_cast<size_t>(src) * block16;
    u32x4* to = c + static_cast<size_t>(dst) * block16;
    size_t x = threadIdx.x;
    // nontemporal stores: the copies are read by the next decode, which
    // should find them in memory rather than dirty in L2
    for (; x + 3 * 256 < block16; x += 4 * 256) {
        const u32x4 a0 = from[x], a1 = from[x + 256], a2 = from[x + 512], a3 = from[x + 768];
        __builtin_nontemporal_store(a0, to + x);
        __builtin_nontemporal_store(a1, to + x + 256);
        __builtin_nontemporal_store(a2, to + x + 512);
        __builtin_nontemporal_store(a3, to + x + 768);
    }
    for (; x < block16; x += 256) __builtin_nontemporal_store(from[x], to + x);
}

// One thread per sequence: the block that holds the sequence's newest token
// (token L - 1, at the slot the append gave it) goes into its table row, at
// column (L - 1) / B. The entry changes only when the token opened a block or
// a copy-on-write moved it; writing it every step keeps the table in step
// with the slots without the host sending rows.
__global__ __launch_bounds__(256) void pa_table_append_kernel(int32_t* __restrict__ tables, int max_blocks,
                                                              const int32_t* __restrict__ lens,
                                                              const int32_t* __restrict__ slots, int num_seqs,
                                                              int log2_bs) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= num_seqs) return;
    const int L = lens[i];
    const int slot = slots[i];
    if (L <= 0 || slot < 0) return;
    const int col = (L - 1) >> log2_bs;
    if (col >= max_blocks) return;
    tables[static_cast<size_t>(i) * max_blocks + col] = slot >> log2_bs;
}

hipError_t launch_table_append(int32_t* tables, int max_blocks, const int32_t* lens, const int32_t* slots,
                               int num_seqs, int block_size, hipStream_t stream) {
    if (num_seqs == 0) return hipSuccess;
    return launch_kernel(pa_table_append_kernel, dim3(static_cast<unsigned>((num_seqs + 255) / 256)), dim3(256), 0,
                         stream, tables, max_blocks, lens, slots, num_seqs, ilog2(block_size));
}

// The same append with the step's lengths and slots carried in the launch
// arguments (host values copied into the dispatch's argument buffer by the
// runtime): each thread stores its sequence's length and slot to the device
// arrays the step's later kernels read, then updates the table row. One
// launch covers kStageSeqs sequences.
struct StageArgs {
    int32_t* tables;
    int32_t* lens_out;
    int32_t* slots_out;
    int max_blocks;
    int num_seqs;
    int log2_bs;
    int32_t lens[kStageSeqs];
    int32_t slots[kStageSeqs];
};
static_assert(sizeof(StageArgs) <= 4000, "kernel arguments are limited to 4 KB");

__global__ __launch_bounds__(kStageSeqs) void pa_stage_append_kernel(StageArgs a) {
    const int i = threadIdx.x;
    if (i >= a.num_seqs) return;
    const int L = a.lens[i];
    const int slot = a.slots[i];
    a.lens_out[i] = L;
    a.slots_out[i] = slot;
    if (L <= 0 || slot < 0) return;
    const int col = (L - 1) >> a.log2_bs;
    if (col >= a.max_blocks) return;
    a.tables[static_cast<size_t>(i) * a.max_blocks + col] = slot >> a.log2_bs;
}

// The table append of pa_stage_append_kernel and the cache write of the
// step's new tokens in one launch: the lengths and slots travel in the
// launch arguments, and the write reads its slots from there too (no slot
// load from memory). Workgroup (x, 0) also does the append for its chunk of
// sequences; every workgroup then writes as pa_write_kernel does.
struct WriteGeom {
    const u32x4* k;
    const u32x4* v;
    u32x4* kc;
    void* vc;
    long long pool_slots;
    int num_kv_heads;
    int head_dim;
    int row16;
    int log2_vt;
    int log2_chunk;
    int log2_win;
};
static_assert(sizeof(StageArgs) + sizeof(WriteGeom) <= 4000, "kernel arguments are limited to 4 KB");

template <typename EW>
__global__ __launch_bounds__(256) void pa_write_stage_kernel(StageArgs a, WriteGeom g) {
    if (blockIdx.y == 0 && threadIdx.x < (1u << g.log2_chunk)) {
        const int i = (blockIdx.x << g.log2_chunk) + threadIdx.x;
        if (i < a.num_seqs) {
            const int L = a.lens[i];
            const int slot = a.slots[i];
            a.lens_out[i] = L;
            a.slots_out[i] = slot;
            if (L > 0 && slot >= 0) {
                const int col = (L - 1) >> a.log2_bs;
                if (col < a.max_blocks) a.tables[static_cast<size_t>(i) * a.max_blocks + col] = slot >> a.log2_bs;
            }
        }
    }
    write_tokens<EW>(g.k, g.v, g.kc, static_cast<EW*>(g.vc), a.slots, a.num_seqs, g.num_kv_heads, g.head_dim,
                     g.row16, a.log2_bs, g.log2_vt, g.log2_chunk, g.log2_win, g.pool_slots);
}

hipError_t launch_stage_append(int32_t* tables, int max_blocks, const int32_t* host_lens,
                               const int32_t* host_slots, int32_t* lens_out, int32_t* slots_out, int num_seqs,
                               int block_size, hipStream_t stream) {
    const int log2_bs = ilog2(block_size);
    for (int i0 = 0; i0 < num_seqs; i0 += kStageSeqs) {
        StageArgs a;
        const int n = std::min(kStageSeqs, num_seqs - i0);
        a.tables = tables + static_cast<size_t>(i0) * max_blocks;
        a.lens_out = lens_out + i0;
        a.slots_out = slots_out + i0;
        a.max_blocks = max_blocks;
        a.num_seqs = n;
        a.log2_bs = log2_bs;
        std::memcpy(a.lens, host_lens + i0, sizeof(int32_t) * n);
        std::memcpy(a.slots, host_slots + i0, sizeof(int32_t) * n);
        const hipError_t e = launch_kernel(pa_stage_append_kernel, dim3(1), dim3(kStageSeqs), 0, stream, a);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// The write's chunking: run mode is 16 entries per workgroup, with V
// staging for up to 31 tokens (the chunk and the rest of its last run) when
// 32 rows fit in 64 KB of LDS. Otherwise plain chunks of 16 entries, fewer
// for rows so wide that 16 would not fit in 32 KB. Returns false if no
// chunk fits.
static bool write_geometry(int head_dim, int elem_bytes, int* log2_chunk, int* log2_win, size_t* smem) {
    const int ld = write_lds_row(head_dim, elem_bytes);
    int c = 4, w = 5;
    if ((static_cast<size_t>(1) << w) * ld * elem_bytes > 64 * 1024) {
        while (c > 0 && (static_cast<size_t>(1) << c) * ld * elem_bytes > 32 * 1024) --c;
        w = c;
    }
    *log2_chunk = c;
    *log2_win = w;
    *smem = (static_cast<size_t>(1) << w) * ld * elem_bytes;
    return *smem <= 64 * 1024;
}

hipError_t launch_write_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                              const int32_t* slots, int num_tokens, int num_layers, int num_kv_heads,
                              int head_dim, int elem_bytes, int block_size, int num_blocks,
                              hipStream_t stream) {
    if (num_tokens == 0 || num_layers == 0) return hipSuccess;
    const int row16 = head_dim * elem_bytes / 16;
    int log2_chunk = 0, log2_win = 0;
    size_t smem = 0;
    if (!write_geometry(head_dim, elem_bytes, &log2_chunk, &log2_win, &smem)) return hipErrorInvalidConfiguration;
    const int log2_bs = ilog2(block_size);
    const int log2_vt = ilog2(v_tile_tokens(block_size));
    const long long pool_slots = static_cast<long long>(num_blocks) * block_size;
    const unsigned chunks = static_cast<unsigned>((num_tokens + (1 << log2_chunk) - 1) >> log2_chunk);
    const dim3 grid(chunks, static_cast<unsigned>(num_kv_heads), static_cast<unsigned>(num_layers));
    if (elem_bytes == 2)
        return launch_kernel(pa_write_kernel<uint16_t>, grid, dim3(256), smem, stream,
                             static_cast<const u32x4*>(k), static_cast<const u32x4*>(v),
                             static_cast<u32x4*>(k_cache), static_cast<uint16_t*>(v_cache), slots, num_tokens,
                             num_kv_heads, head_dim, row16, log2_bs, log2_vt, log2_chunk, log2_win, pool_slots);
    return launch_kernel(pa_write_kernel<uint32_t>, grid, dim3(256), smem, stream,
                         static_cast<const u32x4*>(k), static_cast<const u32x4*>(v),
                         static_cast<u32x4*>(k_cache), static_cast<uint32_t*>(v_cache), slots, num_tokens,
                         num_kv_heads, head_dim, row16, log2_bs, log2_vt, log2_chunk, log2_win, pool_slots);
}

hipError_t launch_write_stage(const void* k, const void* v, void* k_cache, void* v_cache, int32_t* tables,
                              int max_blocks, const int32_t* host_lens, const int32_t* host_slots, int32_t* lens_out,
                              int32_t* slots_out, int num_seqs, int num_kv_heads, int head_dim, int elem_bytes,
                              int block_size, int num_blocks, hipStream_t stream) {
    const int row16 = head_dim * elem_bytes / 16;
    int log2_chunk = 0, log2_win = 0;
    size_t smem = 0;
    if (!write_geometry(head_dim, elem_bytes, &log2_chunk, &log2_win, &smem)) return hipErrorInvalidConfiguration;
    const int log2_bs = ilog2(block_size);
    WriteGeom g;
    g.kc = static_cast<u32x4*>(k_cache);
    g.vc = v_cache;
    g.pool_slots = static_cast<long long>(num_blocks) * block_size;
    g.num_kv_heads = num_kv_heads;
    g.head_dim = head_dim;
    g.row16 = row16;
    g.log2_vt = ilog2(v_tile_tokens(block_size));
    g.log2_chunk = log2_chunk;
    g.log2_win = log2_win;
    for (int i0 = 0; i0 < num_seqs; i0 += kStageSeqs) {
        StageArgs a;
        const int n = std::min(kStageSeqs, num_seqs - i0);
        a.tables = tables + static_cast<size_t>(i0) * max_blocks;
        a.lens_out = lens_out + i0;
        a.slots_out = slots_out + i0;
        a.max_blocks = max_blocks;
        a.num_seqs = n;
        a.log2_bs = log2_bs;
        std::memcpy(a.lens, host_lens + i0, sizeof(int32_t) * n);
        std::memcpy(a.slots, host_slots + i0, sizeof(int32_t) * n);
        const size_t row0 = static_cast<size_t>(i0) * num_kv_heads * row16;
        g.k = static_cast<const u32x4*>(k) + row0;
        g.v = static_cast<const u32x4*>(v) + row0;
        const dim3 grid(static_cast<unsigned>((n + (1 << log2_chunk) - 1) >> log2_chunk),
                        static_cast<unsigned>(num_kv_heads), 1);
        const hipError_t e = elem_bytes == 2
                                 ? launch_kernel(pa_write_stage_kernel<uint16_t>, grid, dim3(256), smem, stream, a, g)
                                 : launch_kernel(pa_write_stage_kernel<uint32_t>, grid, dim3(256), smem, stream, a, g);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int num_pairs,
                              int num_layers, size_t block_bytes, int num_blocks, hipStream_t stream) {
    if (num_pairs == 0 || num_layers == 0) return hipSuccess;
    return launch_kernel(pa_copy_kernel, dim3(static_cast<unsigned>(num_pairs), 2, static_cast<unsigned>(num_layers)),
                         dim3(256), 0, stream, static_cast<u32x4*>(k_cache), static_cast<u32x4*>(v_cache), pairs,
                         block_bytes / 16, num_blocks);
}

}  // namespace pa
