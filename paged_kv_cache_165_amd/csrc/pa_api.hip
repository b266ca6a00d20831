// C-ABI entry points: argument validation, workspace layout and dispatch.
// Every check happens before any launch; a failing call launches nothing.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <unordered_map>

#include "pa.h"
#include "pa_internal.h"

namespace {

// Shape of the default split.
// Workgroup items (float32): at most 256 blocks, and at least 512 items per
// launch (two per compute unit of
// MI355X). The default stops at 256 blocks although an item can stage 512:
// on a skewed batch (lognormal lengths up to 8192) the largest items then
// take most of a launch and the static deal cannot even them out (measured
// on MI355X: 285 us against 255 us at 256 blocks for 256 sequences of 8 KV
// heads, and 562 against 465 us for 8 sequences of 32k-131k tokens).
// 16-bit elements (the stream split, or one item per wave where its cost
// positions would not fit 31 bits): one wave reduces an item alone, four
// times slower than a workgroup, so items stay at 2048 tokens or less (and
// within the wave's table slice), at least 2048 of them (two per wave); the
// stream split needs partitions within that slice and is indifferent to
// their size.
// Neither goes below 512 tokens, the shortest partition worth its item
// switch and merge.
constexpr int kAutoMaxBlocks = 256;
constexpr int kTargetItems = 512;
constexpr int kWaveMaxPartition = 2048;
constexpr int kWaveTargetItems = 2048;
constexpr int kMinAutoPartition = 512;
constexpr int kMaxSeqs = 8192;
using pa::kMaxTableSlice;

thread_local std::string g_last_error;

// Scratch of pa_decode_noalloc: the split-K records live here instead of in a
// caller's workspace. Each GPU the library runs on holds its own copy until
// the process ends. Host code must not use the array's name as an address:
// it is a host-side stand-in; the device address comes from
// hipGetSymbolAddress (noalloc_scratch below).
constexpr size_t kNoAllocScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

}  // namespace

namespace pa {

pa_status_t fail(pa_status_t st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

}  // namespace pa

namespace {

using pa::fail;

pa_status_t hip_fail(hipError_t e, const char* what) {
    return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

pa_status_t lds_fail(int num_seqs, int head_dim, int group, size_t lds_per_cu, size_t lds_per_wg) {
    return fail(PA_ERR_UNSUPPORTED, "num_seqs %d with head_dim %d and group %d needs more LDS than one "
                "workgroup can hold (%zu bytes per compute unit, %zu per workgroup)", num_seqs, head_dim, group,
                lds_per_cu, lds_per_wg);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(pa_dtype_t dt) { return dt == PA_F32 ? 4 : 2; }

bool valid_dtype(int dt) { return dt == PA_F32 || dt == PA_BF16 || dt == PA_F16; }

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int log2i(int x) {
    int r = 0;
    while ((1 << r) < x) ++r;
    return r;
}

// What the launches need to know of the current device, read once per
// device: compute units and LDS sizes.
pa_status_t device_info(pa::DeviceInfo* out) {
    static std::mutex mu;
    static std::unordered_map<int, pa::DeviceInfo> cache;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(dev);
    if (it != cache.end()) {
        *out = it->second;
        return PA_OK;
    }
    int cus = 0, lds_cu = 0, lds_wg = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&lds_wg, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    if (cus < 1 || lds_cu < 1 || lds_wg < 1)
        return fail(PA_ERR_HIP, "device %d reports %d compute units, %d bytes of LDS per compute unit, %d per "
                    "workgroup", dev, cus, lds_cu, lds_wg);
    pa::DeviceInfo d{dev, cus, static_cast<size_t>(lds_cu), static_cast<size_t>(lds_wg)};
    cache[dev] = d;
    *out = d;
    return PA_OK;
}

// Device address of this device's copy of `scratch`, looked up once per
// device with that device current and kept.
pa_status_t noalloc_scratch(void** out) {
    static std::mutex mu;
    static std::unordered_map<int, void*> cache;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(dev);
    if (it != cache.end()) {
        *out = it->second;
        return PA_OK;
    }
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(PA_ERR_HIP, "hipGetSymbolAddress(scratch) returned a null address");
    cache[dev] = ptr;
    *out = ptr;
    return PA_OK;
}

// The default split (pa_default_partition_size): start from the longest
// default partition of the kernel the shape runs on and halve it while the
// batch has too few items to fill the chip. Block sizes are powers of two
// up to 256, so every halving down to 512 stays a multiple of 16 and of
// block_size.
int auto_partition(int num_seqs, int num_heads, int num_kv_heads, int max_context_len, int block_size,
                   pa_dtype_t dtype) {
    const bool wave = pa::decode_uses_mfma(dtype, num_heads / num_kv_heads) ||
                      pa::decode_stream_shape(dtype, block_size);
    int part = wave ? std::min(kWaveMaxPartition, pa::kWaveSlice * block_size) : kAutoMaxBlocks * block_size;
    const long long target = wave ? kWaveTargetItems : kTargetItems;
    while (part > kMinAutoPartition) {
        const long long items = static_cast<long long>(num_seqs) * num_kv_heads *
                                ((static_cast<long long>(max_context_len) + part - 1) / part);
        if (items >= target) break;
        part /= 2;
    }
    return part;
}

int resolve_partition(int partition_size, int num_seqs, int num_heads, int num_kv_heads, int max_context_len,
                      int block_size, pa_dtype_t dtype) {
    return partition_size == 0
               ? auto_partition(num_seqs, num_heads, num_kv_heads, max_context_len, block_size, dtype)
               : partition_size;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Workspace: the per-partition records m, l and o, needed only when some
// sequence can span several partitions. The stream kernel keeps no
// per-partition records (a wave merges the partitions of its stretch of a
// pair itself): per wave of its grid, a tail and a head record of every
// query head of a group, and which pair the tail record belongs to.
struct WsLayout {
    size_t m_off, l_off, o_off, meta_off, xm_off, xl_off, xo_off, total;
};

WsLayout ws_layout(int num_seqs, int num_heads, int num_kv_heads, int head_dim, int pmax, bool stream) {
    WsLayout w{};
    if (stream) {
        const size_t xrecs = 2 * static_cast<size_t>(pa::kMaxStreamWaves) * (num_heads / num_kv_heads);
        w.meta_off = 0;
        w.xm_off = align256(static_cast<size_t>(pa::kMaxStreamWaves) * 4 * sizeof(int));
        w.xl_off = w.xm_off + align256(xrecs * sizeof(float));
        w.xo_off = w.xl_off + align256(xrecs * sizeof(float));
        w.total = w.xo_off + align256(xrecs * head_dim * sizeof(float));
        return w;
    }
    if (pmax <= 1) return w;  // single-partition sequences never write records
    const size_t recs = static_cast<size_t>(num_seqs) * num_heads * pmax;
    w.m_off = 0;
    w.l_off = align256(recs * sizeof(float));
    w.o_off = w.l_off + align256(recs * sizeof(float));
    w.total = w.o_off + align256(recs * head_dim * sizeof(float));
    return w;
}

int pmax_of(int max_context_len, int part) {
    const int p = (max_context_len + part - 1) / part;
    return p < 1 ? 1 : p;
}

// Shape checks shared by the decode entry points and the planning query;
// sets *part to the resolved partition size.
pa_status_t check_decode_shape(int num_seqs, int num_heads, int num_kv_heads, int head_dim, int max_context_len,
                               int block_size, int partition_size, pa_dtype_t dtype, int* part_out) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_context_len < 0 ||
        block_size <= 0 || partition_size < 0)
        return fail(PA_ERR_INVALID_ARG, "negative or zero size (num_seqs=%d num_heads=%d num_kv_heads=%d "
                    "head_dim=%d max_context_len=%d block_size=%d partition_size=%d)", num_seqs, num_heads,
                    num_kv_heads, head_dim, max_context_len, block_size, partition_size);
    if (!valid_dtype(dtype)) return fail(PA_ERR_INVALID_ARG, "unknown dtype %d", static_cast<int>(dtype));
    if (num_heads % num_kv_heads != 0)
        return fail(PA_ERR_INVALID_ARG, "num_heads %d is not a multiple of num_kv_heads %d", num_heads, num_kv_heads);
    const int group = num_heads / num_kv_heads;
    if (!pa::decode_supported(dtype, head_dim, group))
        return fail(PA_ERR_UNSUPPORTED, "no kernel for dtype=%d head_dim=%d group=%d "
                    "(head_dim 64/128/256; group 1/2/4/8, or 16 for 16-bit types)", static_cast<int>(dtype), head_dim, group);
    if (num_seqs > kMaxSeqs) return fail(PA_ERR_UNSUPPORTED, "num_seqs %d > %d", num_seqs, kMaxSeqs);
    if (!is_pow2(block_size) || block_size < 4 || block_size > 256)
        return fail(PA_ERR_UNSUPPORTED, "block_size %d is not a power of two in [4, 256]", block_size);
    const int min_bs = pa::decode_min_block_size(dtype, head_dim, group);
    if (block_size < min_bs)
        return fail(PA_ERR_UNSUPPORTED, "block_size %d < %d, the smallest block this dtype/head_dim/group supports",
                    block_size, min_bs);
    const int part =
        resolve_partition(partition_size, num_seqs, num_heads, num_kv_heads, max_context_len, block_size, dtype);
    if (part % 16 != 0 || part % block_size != 0 || part / block_size > kMaxTableSlice)
        return fail(PA_ERR_INVALID_ARG, "partition_size %d must be a multiple of 16 and of block_size %d "
                    "spanning at most %d blocks", part, block_size, kMaxTableSlice);
    *part_out = part;
    return PA_OK;
}

// Shared validation of the decode entry points; fills `p`.
pa_status_t prepare_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens, float scale,
                           int block_size, int num_seqs, int num_heads, int num_kv_heads,
                           int head_dim, int num_blocks, int max_blocks_per_seq,
                           int max_context_len, int partition_size, pa_dtype_t dtype,
                           void* workspace, size_t workspace_bytes, pa::DecodeParams* p) {
    int part = 0;
    pa_status_t st = check_decode_shape(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, block_size,
                                        partition_size, dtype, &part);
    if (st != PA_OK) return st;
    if (num_blocks <= 0 || max_blocks_per_seq <= 0)
        return fail(PA_ERR_INVALID_ARG, "num_blocks %d and max_blocks_per_seq %d must be positive", num_blocks,
                    max_blocks_per_seq);
    if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale is not finite");
    const int group = num_heads / num_kv_heads;
    if (static_cast<long long>(max_blocks_per_seq) * block_size < max_context_len)
        return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq * block_size = %lld < max_context_len %d",
                    static_cast<long long>(max_blocks_per_seq) * block_size, max_context_len);
    if (num_seqs > 0) {
        if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
            return fail(PA_ERR_INVALID_ARG, "null pointer argument");
        if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
            return fail(PA_ERR_INVALID_ARG, "q, out, k_cache and v_cache must be 16-byte aligned");
        if (out == q) return fail(PA_ERR_INVALID_ARG, "out aliases q");
    }
    const int pmax = pmax_of(max_context_len, part);
    const bool stream = pa::decode_stream(dtype, group, block_size, part, num_seqs, num_kv_heads, max_context_len);
    const WsLayout ws = ws_layout(num_seqs, num_heads, num_kv_heads, head_dim, pmax, stream);
    if (ws.total > 0 && num_seqs > 0) {
        if (!workspace) return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes required", ws.total);
        if (workspace_bytes < ws.total)
            return fail(PA_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", workspace_bytes, ws.total);
        if (!aligned16(workspace)) return fail(PA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    }
    char* wsb = static_cast<char*>(workspace);
    p->out = out;
    p->q = q;
    p->k_cache = k_cache;
    p->v_cache = v_cache;
    p->block_tables = block_tables;
    p->context_lens = context_lens;
    p->ws_m = ws.total && !stream ? reinterpret_cast<float*>(wsb + ws.m_off) : nullptr;
    p->ws_l = ws.total && !stream ? reinterpret_cast<float*>(wsb + ws.l_off) : nullptr;
    p->ws_o = ws.total && !stream ? reinterpret_cast<float*>(wsb + ws.o_off) : nullptr;
    p->ws_meta = stream && ws.total ? reinterpret_cast<int*>(wsb + ws.meta_off) : nullptr;
    p->ws_xm = stream && ws.total ? reinterpret_cast<float*>(wsb + ws.xm_off) : nullptr;
    p->ws_xl = stream && ws.total ? reinterpret_cast<float*>(wsb + ws.xl_off) : nullptr;
    p->ws_xo = stream && ws.total ? reinterpret_cast<float*>(wsb + ws.xo_off) : nullptr;
    p->stream = stream ? 1 : 0;
    p->keep_tiles = 0;
    p->scale_log2 = scale * 1.4426950408889634f;
    p->num_seqs = num_seqs;
    p->num_heads = num_heads;
    p->num_kv_heads = num_kv_heads;
    p->group = group;
    p->num_blocks = num_blocks;
    p->max_blocks = max_blocks_per_seq;
    p->max_ctx = max_context_len;
    p->part = part;
    p->pmax = pmax;
    p->log2_bs = log2i(block_size);
    p->log2_vt = log2i(pa::v_tile_tokens(block_size));
    p->ring_slots = 1;  // set per kernel at launch
    return PA_OK;
}

constexpr int kMaxLayers = 65535;  // grid z

pa_status_t write_cache_layers(const void* k, const void* v, void* k_cache, void* v_cache,
                               const int32_t* slot_mapping, int num_tokens, int num_layers, int num_kv_heads,
                               int head_dim, int block_size, int num_blocks, pa_dtype_t dtype, void* stream) {
    if (num_tokens < 0 || num_layers < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_blocks <= 0)
        return fail(PA_ERR_INVALID_ARG, "negative or zero size (num_tokens=%d num_layers=%d num_kv_heads=%d "
                    "head_dim=%d block_size=%d num_blocks=%d)", num_tokens, num_layers, num_kv_heads, head_dim,
                    block_size, num_blocks);
    if (num_layers > kMaxLayers) return fail(PA_ERR_UNSUPPORTED, "num_layers %d > %d", num_layers, kMaxLayers);
    if (!valid_dtype(dtype)) return fail(PA_ERR_INVALID_ARG, "unknown dtype %d", static_cast<int>(dtype));
    const int row_bytes = head_dim * elem_bytes(dtype);
    if (row_bytes % 16 != 0)
        return fail(PA_ERR_UNSUPPORTED, "head_dim * element size = %d bytes is not a multiple of 16", row_bytes);
    if (row_bytes > 32 * 1024)
        return fail(PA_ERR_UNSUPPORTED, "head_dim * element size = %d bytes is more than 32768", row_bytes);
    if (!is_pow2(block_size) || block_size < 4)
        return fail(PA_ERR_UNSUPPORTED, "block_size %d is not a power of two >= 4", block_size);
    if (num_tokens == 0 || num_layers == 0) return PA_OK;
    if (!k || !v || !k_cache || !v_cache || !slot_mapping) return fail(PA_ERR_INVALID_ARG, "null pointer argument");
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
        return fail(PA_ERR_INVALID_ARG, "k, v, k_cache and v_cache must be 16-byte aligned");
    hipError_t e = pa::launch_write_cache(k, v, k_cache, v_cache, slot_mapping, num_tokens, num_layers, num_kv_heads,
                                          head_dim, elem_bytes(dtype), block_size, num_blocks,
                                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "cache write kernel launch");
    return PA_OK;
}

pa_status_t copy_blocks_layers(void* k_cache, void* v_cache, const int32_t* src_dst_pairs, int num_pairs,
                               int num_layers, int num_kv_heads, int block_size, int head_dim, int num_blocks,
                               pa_dtype_t dtype, void* stream) {
    if (num_pairs < 0 || num_layers < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
        return fail(PA_ERR_INVALID_ARG, "negative or zero size (num_pairs=%d num_layers=%d num_kv_heads=%d "
                    "block_size=%d head_dim=%d num_blocks=%d)", num_pairs, num_layers, num_kv_heads, block_size,
                    head_dim, num_blocks);
    if (num_layers > kMaxLayers) return fail(PA_ERR_UNSUPPORTED, "num_layers %d > %d", num_layers, kMaxLayers);
    if (!valid_dtype(dtype)) return fail(PA_ERR_INVALID_ARG, "unknown dtype %d", static_cast<int>(dtype));
    if (!is_pow2(block_size) || block_size < 4)
        return fail(PA_ERR_UNSUPPORTED, "block_size %d is not a power of two >= 4", block_size);
    const size_t block_bytes = static_cast<size_t>(num_kv_heads) * block_size * head_dim * elem_bytes(dtype);
    if (block_bytes % 16 != 0)
        return fail(PA_ERR_UNSUPPORTED, "block of %zu bytes is not a multiple of 16", block_bytes);
    if (num_pairs == 0 || num_layers == 0) return PA_OK;
    if (!k_cache || !v_cache || !src_dst_pairs) return fail(PA_ERR_INVALID_ARG, "null pointer argument");
    if (!aligned16(k_cache) || !aligned16(v_cache))
        return fail(PA_ERR_INVALID_ARG, "k_cache and v_cache must be 16-byte aligned");
    hipError_t e = pa::launch_copy_blocks(k_cache, v_cache, src_dst_pairs, num_pairs, num_layers, block_bytes,
                                          num_blocks, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "block copy kernel launch");
    return PA_OK;
}

}  // namespace

extern "C" {

int pa_abi_version(void) { return PA_ABI_VERSION; }

const char* pa_status_string(pa_status_t status) {
    switch (status) {
        case PA_OK: return "ok";
        case PA_ERR_INVALID_ARG: return "invalid argument";
        case PA_ERR_UNSUPPORTED: return "unsupported configuration";
        case PA_ERR_WORKSPACE: return "workspace missing or too small";
        case PA_ERR_HIP: return "HIP runtime error";
        case PA_ERR_NO_BLOCKS: return "not enough free blocks";
    }
    return "unknown status";
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

int pa_default_partition_size(int num_seqs, int num_heads, int num_kv_heads, int max_context_len, int block_size,
                              pa_dtype_t dtype) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 ||
        max_context_len < 0 || block_size <= 0 || !valid_dtype(dtype))
        return 0;
    return auto_partition(num_seqs, num_heads, num_kv_heads, max_context_len, block_size, dtype);
}

size_t pa_decode_workspace_size(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                int max_context_len, int block_size, int partition_size, pa_dtype_t dtype) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 || head_dim <= 0 ||
        max_context_len < 0 || block_size <= 0 || partition_size < 0 || !valid_dtype(dtype))
        return 0;
    const int part =
        resolve_partition(partition_size, num_seqs, num_heads, num_kv_heads, max_context_len, block_size, dtype);
    const bool stream = pa::decode_stream(dtype, num_heads / num_kv_heads, block_size, part, num_seqs, num_kv_heads,
                                          max_context_len);
    return ws_layout(num_seqs, num_heads, num_kv_heads, head_dim, pmax_of(max_context_len, part), stream).total;
}

pa_status_t pa_decode_plan(int num_seqs, int num_heads, int num_kv_heads, int head_dim, int max_context_len,
                           int block_size, int partition_size, pa_dtype_t dtype, int lds_per_cu,
                           int lds_per_workgroup, int max_workgroups_per_cu, pa_decode_plan_t* plan) {
    if (!plan) return fail(PA_ERR_INVALID_ARG, "null plan");
    if (lds_per_cu <= 0 || lds_per_workgroup <= 0 || max_workgroups_per_cu <= 0)
        return fail(PA_ERR_INVALID_ARG, "lds_per_cu %d, lds_per_workgroup %d and max_workgroups_per_cu %d must be "
                    "positive", lds_per_cu, lds_per_workgroup, max_workgroups_per_cu);
    int part = 0;
    const pa_status_t st = check_decode_shape(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len,
                                              block_size, partition_size, dtype, &part);
    if (st != PA_OK) return st;
    const int group = num_heads / num_kv_heads;
    const bool stream =
        pa::decode_stream(dtype, group, block_size, part, num_seqs, num_kv_heads, max_context_len);
    pa::DecodePlan pl;
    if (pa::plan_decode(dtype, head_dim, group, num_seqs, part / block_size, stream, static_cast<size_t>(lds_per_cu),
                        static_cast<size_t>(lds_per_workgroup), max_workgroups_per_cu, &pl) != PA_OK)
        return lds_fail(num_seqs, head_dim, group, static_cast<size_t>(lds_per_cu),
                        static_cast<size_t>(lds_per_workgroup));
    plan->kernel = pl.kernel;
    plan->partition_size = part;
    plan->lds_bytes = static_cast<int>(pl.smem);
    plan->ring_slots = pl.ring_slots;
    plan->workgroups_per_cu = pl.resident;
    return PA_OK;
}

#define PA_DECODE_ARGS                                                                              \
    out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size, num_seqs, num_heads, \
        num_kv_heads, head_dim, num_blocks, max_blocks_per_seq, max_context_len, partition_size,  \
        dtype, workspace, workspace_bytes

namespace {

pa_status_t apply_decode_flags(unsigned flags, pa::DecodeParams* p) {
    if (flags & ~static_cast<unsigned>(PA_DECODE_SHARED_BLOCKS))
        return fail(PA_ERR_INVALID_ARG, "unknown decode flags 0x%x", flags & ~static_cast<unsigned>(PA_DECODE_SHARED_BLOCKS));
    p->keep_tiles = (flags & PA_DECODE_SHARED_BLOCKS) ? 1 : 0;
    return PA_OK;
}

}  // namespace

pa_status_t pa_decode_partitions_ex(void* out, const void* q, const void* k_cache,
                                    const void* v_cache, const int32_t* block_tables,
                                    const int32_t* context_lens, float scale, int block_size,
                                    int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                    int num_blocks, int max_blocks_per_seq, int max_context_len,
                                    int partition_size, pa_dtype_t dtype, void* workspace,
                                    size_t workspace_bytes, unsigned flags, void* stream) {
    pa::DecodeParams p;
    pa_status_t st = prepare_decode(PA_DECODE_ARGS, &p);
    if (st != PA_OK) return st;
    st = apply_decode_flags(flags, &p);
    if (st != PA_OK) return st;
    if (num_seqs == 0) return PA_OK;
    pa::DeviceInfo dv;
    st = device_info(&dv);
    if (st != PA_OK) return st;
    hipError_t e = pa::launch_decode_partitions(p, dtype, head_dim, dv, static_cast<hipStream_t>(stream));
    if (e == hipErrorInvalidConfiguration)
        return lds_fail(num_seqs, head_dim, num_heads / num_kv_heads, dv.lds_per_cu, dv.lds_per_wg);
    if (e != hipSuccess) return hip_fail(e, "decode partition kernel launch");
    return PA_OK;
}

pa_status_t pa_decode_partitions(void* out, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_tables,
                                 const int32_t* context_lens, float scale, int block_size,
                                 int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                 int num_blocks, int max_blocks_per_seq, int max_context_len,
                                 int partition_size, pa_dtype_t dtype, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    return pa_decode_partitions_ex(PA_DECODE_ARGS, 0u, stream);
}

pa_status_t pa_decode_merge(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            float scale, int block_size, int num_seqs, int num_heads,
                            int num_kv_heads, int head_dim, int num_blocks,
                            int max_blocks_per_seq, int max_context_len, int partition_size,
                            pa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                            void* stream) {
    pa::DecodeParams p;
    pa_status_t st = prepare_decode(PA_DECODE_ARGS, &p);
    if (st != PA_OK) return st;
    if (num_seqs == 0) return PA_OK;
    hipError_t e = pa::launch_decode_merge(p, dtype, head_dim, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "decode merge kernel launch");
    return PA_OK;
}

pa_status_t pa_decode_ex(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens, float scale,
                         int block_size, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                         int num_blocks, int max_blocks_per_seq, int max_context_len,
                         int partition_size, pa_dtype_t dtype, void* workspace,
                         size_t workspace_bytes, unsigned flags, void* stream) {
    pa::DecodeParams p;
    pa_status_t st = prepare_decode(PA_DECODE_ARGS, &p);
    if (st != PA_OK) return st;
    st = apply_decode_flags(flags, &p);
    if (st != PA_OK) return st;
    if (num_seqs == 0) return PA_OK;
    pa::DeviceInfo dv;
    st = device_info(&dv);
    if (st != PA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = pa::launch_decode_partitions(p, dtype, head_dim, dv, s);
    if (e == hipErrorInvalidConfiguration)
        return lds_fail(num_seqs, head_dim, num_heads / num_kv_heads, dv.lds_per_cu, dv.lds_per_wg);
    if (e != hipSuccess) return hip_fail(e, "decode partition kernel launch");
    e = pa::launch_decode_merge(p, dtype, head_dim, s);
    if (e != hipSuccess) return hip_fail(e, "decode merge kernel launch");
    return PA_OK;
}

pa_status_t pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, float scale,
                      int block_size, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                      int num_blocks, int max_blocks_per_seq, int max_context_len,
                      int partition_size, pa_dtype_t dtype, void* workspace,
                      size_t workspace_bytes, void* stream) {
    return pa_decode_ex(PA_DECODE_ARGS, 0u, stream);
}

pa_status_t pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens, float scale,
                              int block_size, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                              int num_blocks, int max_blocks_per_seq, int max_context_len, int partition_size,
                              pa_dtype_t dtype, void* stream) {
    // the same shape checks and record sizing as pa_decode (no device query)
    int part = 0;
    pa_status_t st = check_decode_shape(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, block_size,
                                        partition_size, dtype, &part);
    if (st != PA_OK) return st;
    const bool split = pa::decode_stream(dtype, num_heads / num_kv_heads, block_size, part, num_seqs, num_kv_heads,
                                         max_context_len);
    const size_t need =
        ws_layout(num_seqs, num_heads, num_kv_heads, head_dim, pmax_of(max_context_len, part), split).total;
    if (need > kNoAllocScratchBytes)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode_noalloc: %d sequences x %d heads x %d partitions of %d tokens "
                    "need %zu bytes of split-K records, more than the %zu bytes of its static scratch (use "
                    "pa_decode with a workspace, or longer partitions)", num_seqs, num_heads,
                    pmax_of(max_context_len, part), part, need, kNoAllocScratchBytes);
    void* ws = nullptr;
    if (need > 0 && num_seqs > 0) {
        st = noalloc_scratch(&ws);
        if (st != PA_OK) return st;
    }
    return pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size, num_seqs, num_heads,
                     num_kv_heads, head_dim, num_blocks, max_blocks_per_seq, max_context_len, part, dtype, ws,
                     ws ? kNoAllocScratchBytes : 0, stream);
}

pa_status_t pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens,
                       const int32_t* query_start, float scale, int block_size, int num_seqs,
                       int num_tokens, int num_heads, int num_kv_heads, int head_dim,
                       int num_blocks, int max_blocks_per_seq, int max_query_len,
                       int max_context_len, pa_dtype_t dtype, void* stream) {
    if (num_seqs < 0 || num_tokens < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        num_blocks <= 0 || max_blocks_per_seq <= 0 || max_query_len < 0 || max_context_len < 0 ||
        block_size <= 0)
        return fail(PA_ERR_INVALID_ARG, "negative or zero size (num_seqs=%d num_tokens=%d num_heads=%d "
                    "num_kv_heads=%d head_dim=%d num_blocks=%d max_blocks_per_seq=%d max_query_len=%d "
                    "max_context_len=%d block_size=%d)", num_seqs, num_tokens, num_heads, num_kv_heads,
                    head_dim, num_blocks, max_blocks_per_seq, max_query_len, max_context_len, block_size);
    if (!valid_dtype(dtype)) return fail(PA_ERR_INVALID_ARG, "unknown dtype %d", static_cast<int>(dtype));
    if (num_heads % num_kv_heads != 0)
        return fail(PA_ERR_INVALID_ARG, "num_heads %d is not a multiple of num_kv_heads %d", num_heads, num_kv_heads);
    if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale is not finite");
    const int group = num_heads / num_kv_heads;
    if (!pa::prefill_supported(dtype, head_dim, group))
        return fail(PA_ERR_UNSUPPORTED, "no prefill kernel for dtype=%d head_dim=%d group=%d "
                    "(float32, bfloat16 or float16; head_dim 64/128/256; group 1/2/4/8/16)",
                    static_cast<int>(dtype), head_dim, group);
    if (!is_pow2(block_size) || block_size < 4 || block_size > 256)
        return fail(PA_ERR_UNSUPPORTED, "block_size %d is not a power of two in [4, 256]", block_size);
    if (static_cast<long long>(max_blocks_per_seq) * block_size < max_context_len)
        return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq * block_size = %lld < max_context_len %d",
                    static_cast<long long>(max_blocks_per_seq) * block_size, max_context_len);
    if (num_seqs == 0 || max_query_len == 0) return PA_OK;
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
        return fail(PA_ERR_INVALID_ARG, "null pointer argument");
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return fail(PA_ERR_INVALID_ARG, "q, out, k_cache and v_cache must be 16-byte aligned");
    if (out == q) return fail(PA_ERR_INVALID_ARG, "out aliases q");
    pa::PrefillParams p;
    p.out = out;
    p.q = q;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.query_start = query_start;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.num_seqs = num_seqs;
    p.num_heads = num_heads;
    p.num_kv_heads = num_kv_heads;
    p.num_blocks = num_blocks;
    p.max_blocks = max_blocks_per_seq;
    p.max_ctx = max_context_len;
    p.max_q = max_query_len;
    p.num_tokens = num_tokens;
    p.log2_bs = log2i(block_size);
    p.log2_vt = log2i(pa::v_tile_tokens(block_size));
    // The K/V rows the batch attends to, at most: when they cannot stay in
    // half of MI355X's 256 MB last-level cache, the query tiles of one
    // (sequence, KV head) pair are kept together on one XCD so that they
    // share its L2 (measured: 455-459 against 562 us on 32 chunks of 512
    // tokens after histories of up to 3072; whole 2048-token prompts, whose
    // 67 MB stay in the last-level cache, run within noise of each other in
    // both orders, tile-major fetching about three times their K/V and
    // queries past the L2).
    const double kv_bound = static_cast<double>(num_seqs) * num_kv_heads * max_context_len * head_dim *
                            elem_bytes(dtype) * 2.0;
    p.pair_major = kv_bound > 128.0 * (1 << 20) ? 1 : 0;
    hipError_t e = pa::launch_prefill(p, dtype, head_dim, group, static_cast<hipStream_t>(stream));
    if (e == hipErrorInvalidConfiguration)
        return fail(PA_ERR_UNSUPPORTED, "num_seqs %d x num_kv_heads %d x query tiles of max_query_len %d "
                    "exceeds the grid limit", num_seqs, num_kv_heads, max_query_len);
    if (e != hipSuccess) return hip_fail(e, "prefill kernel launch");
    return PA_OK;
}

pa_status_t pa_write_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                           const int32_t* slot_mapping, int num_tokens, int num_kv_heads,
                           int head_dim, int block_size, int num_blocks, pa_dtype_t dtype,
                           void* stream) {
    return write_cache_layers(k, v, k_cache, v_cache, slot_mapping, num_tokens, 1, num_kv_heads, head_dim,
                              block_size, num_blocks, dtype, stream);
}

pa_status_t pa_write_cache_layers(const void* k, const void* v, void* k_cache, void* v_cache,
                                  const int32_t* slot_mapping, int num_tokens, int num_layers,
                                  int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                  pa_dtype_t dtype, void* stream) {
    return write_cache_layers(k, v, k_cache, v_cache, slot_mapping, num_tokens, num_layers, num_kv_heads,
                              head_dim, block_size, num_blocks, dtype, stream);
}

pa_status_t pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_dst_pairs,
                           int num_pairs, int num_kv_heads, int block_size, int head_dim,
                           int num_blocks, pa_dtype_t dtype, void* stream) {
    return copy_blocks_layers(k_cache, v_cache, src_dst_pairs, num_pairs, 1, num_kv_heads, block_size, head_dim,
                              num_blocks, dtype, stream);
}

pa_status_t pa_copy_blocks_layers(void* k_cache, void* v_cache, const int32_t* src_dst_pairs,
                                  int num_pairs, int num_layers, int num_kv_heads, int block_size,
                                  int head_dim, int num_blocks, pa_dtype_t dtype, void* stream) {
    return copy_blocks_layers(k_cache, v_cache, src_dst_pairs, num_pairs, num_layers, num_kv_heads, block_size,
                              head_dim, num_blocks, dtype, stream);
}

pa_status_t pa_append_block_tables(int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                                   const int32_t* slot_mapping, int num_seqs, int block_size, void* stream) {
    if (num_seqs < 0 || max_blocks_per_seq <= 0 || block_size <= 0)
        return fail(PA_ERR_INVALID_ARG, "negative or zero size (num_seqs=%d max_blocks_per_seq=%d block_size=%d)",
                    num_seqs, max_blocks_per_seq, block_size);
    if (!is_pow2(block_size) || block_size > 256)
        return fail(PA_ERR_UNSUPPORTED, "block_size %d is not a power of two up to 256", block_size);
    if (num_seqs == 0) return PA_OK;
    if (!block_tables || !context_lens || !slot_mapping) return fail(PA_ERR_INVALID_ARG, "null pointer argument");
    hipError_t e = pa::launch_table_append(block_tables, max_blocks_per_seq, context_lens, slot_mapping, num_seqs,
                                           block_size, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "table append kernel launch");
    return PA_OK;
}

pa_status_t pa_append_block_tables_host(int32_t* block_tables, int max_blocks_per_seq,
                                        const int32_t* host_context_lens, const int32_t* host_slot_mapping,
                                        int32_t* context_lens_out, int32_t* slot_mapping_out, int num_seqs,
                                        int block_size, void* stream) {
    if (num_seqs < 0 || max_blocks_per_seq <= 0 || block_size <= 0)
        return fail(PA_ERR_INVALID_ARG, "negative or zero size (num_seqs=%d max_blocks_per_seq=%d block_size=%d)",
                    num_seqs, max_blocks_per_seq, block_size);
    if (!is_pow2(block_size) || block_size > 256)
        return fail(PA_ERR_UNSUPPORTED, "block_size %d is not a power of two up to 256", block_size);
    if (num_seqs == 0) return PA_OK;
    if (!block_tables || !host_context_lens || !host_slot_mapping || !context_lens_out || !slot_mapping_out)
        return fail(PA_ERR_INVALID_ARG, "null pointer argument");
    hipError_t e = pa::launch_stage_append(block_tables, max_blocks_per_seq, host_context_lens, host_slot_mapping,
                                           context_lens_out, slot_mapping_out, num_seqs, block_size,
                                           static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "table append kernel launch");
    return PA_OK;
}

pa_status_t pa_write_cache_append_host(const void* k, const void* v, void* k_cache, void* v_cache,
                                       int32_t* block_tables, int max_blocks_per_seq,
                                       const int32_t* host_context_lens, const int32_t* host_slot_mapping,
                                       int32_t* context_lens_out, int32_t* slot_mapping_out, int num_seqs,
                                       int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                       pa_dtype_t dtype, void* stream) {
    if (num_seqs < 0 || max_blocks_per_seq <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_blocks <= 0)
        return fail(PA_ERR_INVALID_ARG, "negative or zero size (num_seqs=%d max_blocks_per_seq=%d num_kv_heads=%d "
                    "head_dim=%d block_size=%d num_blocks=%d)", num_seqs, max_blocks_per_seq, num_kv_heads, head_dim,
                    block_size, num_blocks);
    if (!valid_dtype(dtype)) return fail(PA_ERR_INVALID_ARG, "unknown dtype %d", static_cast<int>(dtype));
    const int row_bytes = head_dim * elem_bytes(dtype);
    if (row_bytes % 16 != 0)
        return fail(PA_ERR_UNSUPPORTED, "head_dim * element size = %d bytes is not a multiple of 16", row_bytes);
    if (row_bytes > 32 * 1024)
        return fail(PA_ERR_UNSUPPORTED, "head_dim * element size = %d bytes is more than 32768", row_bytes);
    if (!is_pow2(block_size) || block_size < 4 || block_size > 256)
        return fail(PA_ERR_UNSUPPORTED, "block_size %d is not a power of two in [4, 256]", block_size);
    if (num_seqs == 0) return PA_OK;
    if (!k || !v || !k_cache || !v_cache || !block_tables || !host_context_lens || !host_slot_mapping ||
        !context_lens_out || !slot_mapping_out)
        return fail(PA_ERR_INVALID_ARG, "null pointer argument");
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
        return fail(PA_ERR_INVALID_ARG, "k, v, k_cache and v_cache must be 16-byte aligned");
    hipError_t e = pa::launch_write_stage(k, v, k_cache, v_cache, block_tables, max_blocks_per_seq,
                                          host_context_lens, host_slot_mapping, context_lens_out, slot_mapping_out,
                                          num_seqs, num_kv_heads, head_dim, elem_bytes(dtype), block_size,
                                          num_blocks, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "table append and cache write kernel launch");
    return PA_OK;
}

}  // extern "C"
