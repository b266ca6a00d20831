// Bandwidth probe: read the (K tile, V tile) pairs paged decode reads, with
// its loads and no arithmetic (see include/pa_probe.h). A measurement aid for
// the benchmark's pattern ceiling; nothing in the attention path uses it.

#include <hip/hip_runtime.h>

#include "pa_device.h"
#include "pa_internal.h"
#include "pa_probe.h"

namespace pa {
namespace {

// One wave per contiguous run of the tile list, the runs dealt to the XCDs as
// the decode's stream split deals its runs; U tile pairs loading at once,
// each CH KB of K and CH KB of V as 16-byte nontemporal lane loads (one 1 KB
// row of the wave per load instruction), folded into a checksum after all U
// have arrived. Past the run's end a group repeats the run's last tile.
template <int U, int CH>
__global__ __launch_bounds__(256) void pa_probe_tiles_kernel(const char* __restrict__ k, const char* __restrict__ v,
                                                             const int32_t* __restrict__ tiles, int n,
                                                             int num_cache_tiles, u32x4* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int W = gridDim.x * 4;
    const int w = __builtin_amdgcn_readfirstlane(xcd_run_id<4>(W, static_cast<int>(threadIdx.x >> 6)));
    const int lo = static_cast<int>(static_cast<long long>(n) * w / W);
    const int hi = static_cast<int>(static_cast<long long>(n) * (w + 1) / W);
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int i = lo; i < hi; i += U) {
        u32x4 a[U][2 * CH];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int t = tiles[min(i + u, hi - 1)];
            t = t < 0 ? 0 : (t >= num_cache_tiles ? num_cache_tiles - 1 : t);
            const size_t off = static_cast<size_t>(t) * (CH * 1024) + lane * 16;
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                a[u][c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k + off + 1024 * c));
                a[u][CH + c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + off + 1024 * c));
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int c = 0; c < 2 * CH; ++c) acc ^= a[u][c];
    }
    sink[static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x] = acc;
}

template <int U>
hipError_t launch_u(const char* k, const char* v, const int32_t* tiles, int n, int num_cache_tiles, int ch,
                    unsigned grid, u32x4* sink, hipStream_t s) {
    switch (ch) {
        case 1: return launch_kernel(pa_probe_tiles_kernel<U, 1>, dim3(grid), dim3(256), 0, s, k, v, tiles, n,
                                     num_cache_tiles, sink);
        case 2: return launch_kernel(pa_probe_tiles_kernel<U, 2>, dim3(grid), dim3(256), 0, s, k, v, tiles, n,
                                     num_cache_tiles, sink);
        case 4: return launch_kernel(pa_probe_tiles_kernel<U, 4>, dim3(grid), dim3(256), 0, s, k, v, tiles, n,
                                     num_cache_tiles, sink);
        case 8: return launch_kernel(pa_probe_tiles_kernel<U, 8>, dim3(grid), dim3(256), 0, s, k, v, tiles, n,
                                     num_cache_tiles, sink);
    }
    return hipErrorInvalidValue;
}

}  // namespace
}  // namespace pa

extern "C" pa_status_t pa_probe_read_tiles(const void* k_cache, const void* v_cache, const int32_t* tiles,
                                           int num_tiles, int num_cache_tiles, int tile_bytes, int tiles_in_flight,
                                           int workgroups, void* sink, void* stream) {
    using pa::fail;
    if (num_tiles < 0 || num_cache_tiles <= 0 || workgroups <= 0 || workgroups > 65535)
        return fail(PA_ERR_INVALID_ARG, "num_tiles %d, num_cache_tiles %d, workgroups %d out of range", num_tiles,
                    num_cache_tiles, workgroups);
    const int ch = tile_bytes / 1024;
    if (tile_bytes % 1024 != 0 || !(ch == 1 || ch == 2 || ch == 4 || ch == 8))
        return fail(PA_ERR_UNSUPPORTED, "tile_bytes %d: 1, 2, 4 or 8 KB", tile_bytes);
    if (!(tiles_in_flight == 1 || tiles_in_flight == 2 || tiles_in_flight == 4))
        return fail(PA_ERR_UNSUPPORTED, "tiles_in_flight %d: 1, 2 or 4", tiles_in_flight);
    if (num_tiles == 0) return PA_OK;
    if (!k_cache || !v_cache || !tiles || !sink) return fail(PA_ERR_INVALID_ARG, "null pointer argument");
    if ((reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache) |
         reinterpret_cast<uintptr_t>(sink)) & 15u)
        return fail(PA_ERR_INVALID_ARG, "k_cache, v_cache and sink must be 16-byte aligned");
    const char* k = static_cast<const char*>(k_cache);
    const char* v = static_cast<const char*>(v_cache);
    auto* out = static_cast<pa::u32x4*>(sink);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const unsigned grid = static_cast<unsigned>(workgroups);
    hipError_t e = hipErrorInvalidValue;
    switch (tiles_in_flight) {
        case 1: e = pa::launch_u<1>(k, v, tiles, num_tiles, num_cache_tiles, ch, grid, out, s); break;
        case 2: e = pa::launch_u<2>(k, v, tiles, num_tiles, num_cache_tiles, ch, grid, out, s); break;
        case 4: e = pa::launch_u<4>(k, v, tiles, num_tiles, num_cache_tiles, ch, grid, out, s); break;
    }
    if (e != hipSuccess) return fail(PA_ERR_HIP, "probe kernel launch: %s", hipGetErrorString(e));
    return PA_OK;
}
