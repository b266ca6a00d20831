// Cache maintenance kernels for gfx950: the per-token write through a slot
// mapping and the whole-block copy of copy-on-write.
//
// Both move raw bits and never convert, so the result is bit-exact whatever
// the element type (NaN payloads included): K rows and whole blocks as 16-byte
// vectors, V elements one by one into their transposed tile. The write
// stores a sequence's newest token; the copy duplicates a shared block into a
// freshly allocated one before a sharer writes into it, the copy half of
// copy-on-write (aiqz.cc tutorial, section 前缀共享机制; cf-1.com blog, 4.2).
// The slot of a
// token is its (physical block, offset) pair of the block-table equation
// (aiqz.cc, section 块表映射机制) flattened as pid * B + off.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// One workgroup per new token. K: thread c moves 16-byte chunk c of the
// token's [Hkv][D] rows into k_cache[pid][kv][off][:]. V: the cache holds each
// block's rows as tiles of vt tokens stored head_dim-major
// ([NB][Hkv][B/vt][D][vt]), so element d of head kv goes to
// v_cache[pid][kv][off / vt][d][off % vt], one element per thread.
template <typename EW>
__global__ __launch_bounds__(256) void pa_write_kernel(const u32x4* __restrict__ k,
                                                       const EW* __restrict__ v,
                                                       u32x4* __restrict__ kc,
                                                       EW* __restrict__ vc,
                                                       const int32_t* __restrict__ slots,
                                                       int num_kv_heads, int head_dim, int row16,
                                                       int block_size, int vt, long long pool_slots) {
    const int i = blockIdx.x;
    const int slot = slots[i];
    if (slot < 0 || static_cast<long long>(slot) >= pool_slots) return;
    const int pid = slot / block_size;
    const int off = slot - pid * block_size;
    const int chunks = num_kv_heads * row16;
    for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
        const int kvh = c / row16;
        const int r = c - kvh * row16;
        const size_t dst = ((static_cast<size_t>(pid) * num_kv_heads + kvh) * block_size + off) * row16 + r;
        kc[dst] = k[static_cast<size_t>(i) * chunks + c];
    }
    const int elems = num_kv_heads * head_dim;
    const size_t tile_off = static_cast<size_t>(off / vt) * head_dim * vt + (off % vt);
    for (int c = threadIdx.x; c < elems; c += blockDim.x) {
        const int kvh = c / head_dim;
        const int d = c - kvh * head_dim;
        const size_t dst = (static_cast<size_t>(pid) * num_kv_heads + kvh) * block_size * head_dim + tile_off +
                           static_cast<size_t>(d) * vt;
        vc[dst] = v[static_cast<size_t>(i) * elems + c];
    }
}

// grid (pairs, 2): y = 0 copies K, y = 1 copies V. A block is contiguous
// ([Hkv][B][D]), so the copy is one linear run of block16 vectors.
__global__ __launch_bounds__(256) void pa_copy_kernel(u32x4* __restrict__ kc, u32x4* __restrict__ vc,
                                                      const int32_t* __restrict__ pairs,
                                                      size_t block16, int num_blocks) {
    const int i = blockIdx.x;
    const int src = pairs[2 * i];
    const int dst = pairs[2 * i + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
    u32x4* c = blockIdx.y == 0 ? kc : vc;
    const u32x4* from = c + static_cast<size_t>(src) * block16;
    u32x4* to = c + static_cast<size_t>(dst) * block16;
    size_t x = threadIdx.x;
    for (; x + 3 * 256 < block16; x += 4 * 256) {
        const u32x4 a0 = from[x], a1 = from[x + 256], a2 = from[x + 512], a3 = from[x + 768];
        to[x] = a0; to[x + 256] = a1; to[x + 512] = a2; to[x + 768] = a3;
    }
    for (; x < block16; x += 256) to[x] = from[x];
}

hipError_t launch_write_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                              const int32_t* slots, int num_tokens, int num_kv_heads,
                              int head_dim, int elem_bytes, int block_size, int num_blocks,
                              hipStream_t stream) {
    if (num_tokens == 0) return hipSuccess;
    const int row16 = head_dim * elem_bytes / 16;
    const int work = num_kv_heads * head_dim;
    const int threads = work < 256 ? ((work + 63) / 64) * 64 : 256;
    const int vt = v_tile_tokens(block_size);
    const long long pool_slots = static_cast<long long>(num_blocks) * block_size;
    const dim3 grid(static_cast<unsigned>(num_tokens));
    if (elem_bytes == 2) {
        hipLaunchKernelGGL(pa_write_kernel<uint16_t>, grid, dim3(threads), 0, stream,
                           static_cast<const u32x4*>(k), static_cast<const uint16_t*>(v),
                           static_cast<u32x4*>(k_cache), static_cast<uint16_t*>(v_cache), slots,
                           num_kv_heads, head_dim, row16, block_size, vt, pool_slots);
    } else {
        hipLaunchKernelGGL(pa_write_kernel<uint32_t>, grid, dim3(threads), 0, stream,
                           static_cast<const u32x4*>(k), static_cast<const uint32_t*>(v),
                           static_cast<u32x4*>(k_cache), static_cast<uint32_t*>(v_cache), slots,
                           num_kv_heads, head_dim, row16, block_size, vt, pool_slots);
    }
    return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int num_pairs,
                              size_t block_bytes, int num_blocks, hipStream_t stream) {
    if (num_pairs == 0) return hipSuccess;
    hipLaunchKernelGGL(pa_copy_kernel, dim3(static_cast<unsigned>(num_pairs), 2), dim3(256), 0, stream,
                       static_cast<u32x4*>(k_cache), static_cast<u32x4*>(v_cache), pairs,
                       block_bytes / 16, num_blocks);
    return hipGetLastError();
}

}  // namespace pa
