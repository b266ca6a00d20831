// Paged decode attention kernels for gfx950 (MI355X).
//
// Operation (aiqz.cc tutorial, section 块表映射机制, equation pid/off; the
// lihaoran.work note, section 块表把逻辑顺序映射到物理位置): token t of a sequence
// lives at block_table[t / B], offset t % B; attention over all visible tokens
// is ordinary softmax attention, only the addressing differs.
//
// Work decomposition. An item is (sequence, KV head, partition of `part`
// tokens). A persistent grid of 256-thread workgroups walks the item list;
// every workgroup first builds, in LDS, the prefix sum of partition counts
// over the batch so that an item index maps to its sequence by binary search.
// The four waves of a workgroup share one item and take its steps of
// 4 x (rows per load) tokens round robin.
//
// Per item: the slice of the block table the partition reads is staged in
// LDS (cf-1.com blog, 2.2 and 5.4: table lookups served from shared memory,
// not global memory). Per step every lane loads four 16-byte pieces of K and
// of V -- each wave load instruction covers whole rows, 1 KiB contiguous for
// bf16 D=128 at B=16 -- while the previous step is being reduced, so the next
// block is always in flight (cf-1.com 5.1 and 6.2: prefetch the next
// physical block). q.k is a per-lane partial dot product finished by a DPP
// butterfly inside the lanes that hold one row; each lane keeps an online
// softmax (running max m, sum l, weighted V sum) over the rows it saw.
// Lanes, then waves (through LDS), are merged by the log-sum-exp rule.
// A sequence that fits one partition is written straight to `out`; longer
// ones leave one (m, l, o) record per partition for the merge kernel.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxTableSlice = 256;  // table entries one partition may span

__device__ __forceinline__ int clamp_ctx(int L, const DecodeParams& p) {
    L = L < 0 ? 0 : L;
    L = L > p.max_ctx ? p.max_ctx : L;
    return L;
}

template <int DT, int D, int G>
__global__ __launch_bounds__(kThreads) void pa_partition_valu(DecodeParams p) {
    using EL = Elem<DT>;
    constexpr int E = EL::E;
    constexpr int EPL = 16 / E;        // elements per lane per 16-byte load
    constexpr int LPR = D / EPL;       // lanes holding one row
    constexpr int RPI = 64 / LPR;      // rows per wave load instruction
    constexpr int U = 4;               // row chunks per step
    constexpr int STEP = U * RPI;      // tokens per step
    static_assert(LPR >= 8 && LPR <= 64 && RPI * LPR == 64, "row mapping");

    extern __shared__ __align__(16) unsigned char smem[];
    const int S = p.num_seqs;
    int* prefix = reinterpret_cast<int*>(smem);                  // S + 1
    int* tbl = prefix + ((S + 4) & ~3);                           // kMaxTableSlice
    float* red = reinterpret_cast<float*>(tbl + kMaxTableSlice);  // kWaves * G * (D + 2)
    __shared__ int wave_tot[kWaves];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int rg = lane / LPR;             // row inside a load instruction
    const int dsl = (lane % LPR) * EPL;    // first head-dim element of the lane
    const int bs = 1 << p.log2_bs;
    const int hkv = p.num_kv_heads;

    // ---- prefix sum of partition counts (every workgroup builds its own copy)
    if (tid == 0) prefix[0] = 0;
    int carry = 0;
    for (int base = 0; base < S; base += kThreads) {
        const int i = base + tid;
        int n = 0;
        if (i < S) {
            const int L = clamp_ctx(p.context_lens[i], p);
            n = L > 0 ? ceil_div(L, p.part) : 1;
        }
        int x = n;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (lane == 63) wave_tot[wave] = x;
        __syncthreads();
        int add = carry;
        for (int w = 0; w < wave; ++w) add += wave_tot[w];
        if (i < S) prefix[i + 1] = x + add;
        carry += wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
        __syncthreads();
    }
    const int total_items = prefix[S] * hkv;

    const size_t kv_head_stride = static_cast<size_t>(bs) * D;  // elements
    const char* kbase = static_cast<const char*>(p.k_cache);
    const char* vbase = static_cast<const char*>(p.v_cache);

    for (int item = blockIdx.x; item < total_items; item += gridDim.x) {
        const int j = item / hkv;
        const int kv = item - j * hkv;
        int lo = 0, hi = S;  // prefix[lo] <= j < prefix[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (prefix[mid] <= j) lo = mid; else hi = mid;
        }
        const int s = lo;
        const int pidx = j - prefix[s];
        const int nparts = prefix[s + 1] - prefix[s];
        const int L = clamp_ctx(p.context_lens[s], p);
        const int t0 = pidx * p.part;
        const int t1 = min(L, t0 + p.part);
        const int ntok = t1 - t0;  // 0 only for an empty sequence
        const int b0 = t0 >> p.log2_bs;
        const int nblk = (ntok + bs - 1) >> p.log2_bs;

        if (tid < nblk) {
            int pid = p.block_tables[static_cast<size_t>(s) * p.max_blocks + b0 + tid];
            pid = pid < 0 ? 0 : (pid >= p.num_blocks ? p.num_blocks - 1 : pid);
            tbl[tid] = pid;
        }
        __syncthreads();

        // query rows of the G heads sharing this KV head, widened to float
        float qv[G][EPL];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const size_t qoff = (static_cast<size_t>(s) * p.num_heads + kv * G + h) * D + dsl;
            const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const char*>(p.q) + qoff * E);
            EL::to_float(w, qv[h]);
        }

        float m[G], l[G], acc[G][EPL];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            m[h] = -INFINITY;
            l[h] = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
        }

        const int nsteps = ntok > 0 ? (ntok + STEP - 1) / STEP : 0;

        auto load_step = [&](int step, u32x4 (&kb)[U], u32x4 (&vb)[U]) {
#pragma unroll
            for (int c = 0; c < U; ++c) {
                const int tc = t0 + step * STEP + c * RPI;  // first token of the chunk
                const int tcc = min(tc, t1 - 1);
                const int trow = min(tc + rg, t1 - 1);       // this lane's row (clamped)
                const int pid = __builtin_amdgcn_readfirstlane(tbl[(tcc >> p.log2_bs) - b0]);
                const size_t tile = (static_cast<size_t>(pid) * hkv + kv) * kv_head_stride;
                const size_t el = tile + static_cast<size_t>(trow & (bs - 1)) * D + dsl;
                kb[c] = *reinterpret_cast<const u32x4*>(kbase + el * E);
                vb[c] = *reinterpret_cast<const u32x4*>(vbase + el * E);
            }
        };

        auto compute_step = [&](int step, const u32x4 (&kb)[U], const u32x4 (&vb)[U]) {
            float x[U][G];
#pragma unroll
            for (int c = 0; c < U; ++c) {
                float kf[EPL];
                EL::to_float(kb[c], kf);
                const bool valid = (t0 + step * STEP + c * RPI + rg) < t1;
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    float d = 0.f;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) d = fmaf(qv[h][e], kf[e], d);
                    d = group_sum<LPR>(d);
                    x[c][h] = valid ? d * p.scale_log2 : -INFINITY;
                }
            }
            float pw[U][G];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float mx = x[0][h];
#pragma unroll
                for (int c = 1; c < U; ++c) mx = fmaxf(mx, x[c][h]);
                const float mnew = fmaxf(m[h], mx);
                const float mu = mnew == -INFINITY ? 0.f : mnew;
                const float alpha = fast_exp2(m[h] - mu);
                float ps = 0.f;
#pragma unroll
                for (int c = 0; c < U; ++c) {
                    pw[c][h] = fast_exp2(x[c][h] - mu);
                    ps += pw[c][h];
                }
                l[h] = l[h] * alpha + ps;
                m[h] = mnew;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
            }
#pragma unroll
            for (int c = 0; c < U; ++c) {
                float vf[EPL];
                EL::to_float(vb[c], vf);
#pragma unroll
                for (int h = 0; h < G; ++h) {
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pw[c][h], vf[e], acc[h][e]);
                }
            }
        };

        // double-buffered walk over this wave's steps
        int s0 = wave;
        if (s0 < nsteps) {
            u32x4 ka[U], va[U], kb2[U], vb2[U];
            load_step(s0, ka, va);
            while (true) {
                const int s1 = s0 + kWaves;
                if (s1 < nsteps) load_step(s1, kb2, vb2);
                compute_step(s0, ka, va);
                if (s1 >= nsteps) break;
                s0 = s1 + kWaves;
                if (s0 < nsteps) load_step(s0, ka, va);
                compute_step(s1, kb2, vb2);
                if (s0 >= nsteps) break;
            }
        }

        // merge the row groups of the wave (lanes LPR apart)
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float mo = __shfl_xor(m[h], off);
                const float lo2 = __shfl_xor(l[h], off);
                const float mn = fmaxf(m[h], mo);
                const float mu = mn == -INFINITY ? 0.f : mn;
                const float a = fast_exp2(m[h] - mu);
                const float b = fast_exp2(mo - mu);
                l[h] = l[h] * a + lo2 * b;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[h][e] = acc[h][e] * a + __shfl_xor(acc[h][e], off) * b;
                m[h] = mn;
            }
        }
        if (lane < LPR) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float* r = red + (wave * G + h) * (D + 2);
#pragma unroll
                for (int e = 0; e < EPL; ++e) r[dsl + e] = acc[h][e];
                if (lane == 0) {
                    r[D] = m[h];
                    r[D + 1] = l[h];
                }
            }
        }
        __syncthreads();

        // merge the waves and write the partition's result
        for (int idx = tid; idx < G * D; idx += kThreads) {
            const int h = idx / D;
            const int d = idx - h * D;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red[(w * G + h) * (D + 2) + D]);
            const float Mu = M == -INFINITY ? 0.f : M;
            float lsum = 0.f, o = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float* r = red + (w * G + h) * (D + 2);
                const float f = fast_exp2(r[D] - Mu);
                lsum += r[D + 1] * f;
                o += r[d] * f;
            }
            const float res = lsum > 0.f ? o / lsum : 0.f;
            const int hq = kv * G + h;
            if (nparts == 1) {
                EL::store(p.out, (static_cast<size_t>(s) * p.num_heads + hq) * D + d, res);
            } else {
                const size_t rec = (static_cast<size_t>(s) * p.num_heads + hq) * p.pmax + pidx;
                p.ws_o[rec * D + d] = res;
                if (d == 0) {
                    p.ws_m[rec] = M;
                    p.ws_l[rec] = lsum;
                }
            }
        }
        __syncthreads();
    }
}

// Log-sum-exp merge of the partition records of one (sequence, query head).
template <int DT, int D>
__global__ __launch_bounds__(64) void pa_merge(DecodeParams p) {
    using EL = Elem<DT>;
    constexpr int PER = D / 64;
    const int hq = blockIdx.x;
    const int s = blockIdx.y;
    const int lane = threadIdx.x;
    const int L = clamp_ctx(p.context_lens[s], p);
    const int P = L > 0 ? ceil_div(L, p.part) : 1;
    if (P == 1) return;
    const size_t rec0 = (static_cast<size_t>(s) * p.num_heads + hq) * p.pmax;
    const float* mrow = p.ws_m + rec0;
    const float* lrow = p.ws_l + rec0;
    float M = -INFINITY;
    for (int i = lane; i < P; i += 64) M = fmaxf(M, mrow[i]);
    M = wave_max(M);
    const float Mu = M == -INFINITY ? 0.f : M;
    float acc[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = 0.f;
    float W = 0.f;
    const float* o = p.ws_o + rec0 * D;
#pragma unroll 4
    for (int i = 0; i < P; ++i) {
        const float w = lrow[i] * fast_exp2(mrow[i] - Mu);
        W += w;
#pragma unroll
        for (int k = 0; k < PER; ++k) acc[k] = fmaf(w, o[static_cast<size_t>(i) * D + lane + 64 * k], acc[k]);
    }
    const float inv = W > 0.f ? 1.f / W : 0.f;
#pragma unroll
    for (int k = 0; k < PER; ++k)
        EL::store(p.out, (static_cast<size_t>(s) * p.num_heads + hq) * D + lane + 64 * k, acc[k] * inv);
}

// ---------------------------------------------------------------------------
// Host-side dispatch
// ---------------------------------------------------------------------------

namespace {

template <int DT, int D, int G>
hipError_t launch_part(const DecodeParams& p, int num_cus, hipStream_t stream) {
    const size_t smem = (static_cast<size_t>((p.num_seqs + 4) & ~3) + kMaxTableSlice) * sizeof(int) +
                        static_cast<size_t>(kWaves) * G * (D + 2) * sizeof(float);
    auto kern = pa_partition_valu<DT, D, G>;
    int occ = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, kThreads, smem);
    if (e != hipSuccess) return e;
    if (occ < 1) occ = 1;
    const long long upper = static_cast<long long>(p.num_seqs) * p.num_kv_heads * p.pmax;
    long long grid = static_cast<long long>(num_cus) * occ;
    if (grid > upper) grid = upper;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kThreads), smem, stream, p);
    return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_part_g(const DecodeParams& p, int num_cus, hipStream_t stream) {
    switch (p.group) {
        case 1: return launch_part<DT, D, 1>(p, num_cus, stream);
        case 2: return launch_part<DT, D, 2>(p, num_cus, stream);
        case 4: return launch_part<DT, D, 4>(p, num_cus, stream);
        case 8: return launch_part<DT, D, 8>(p, num_cus, stream);
    }
    return hipErrorInvalidValue;
}

template <int DT>
hipError_t launch_part_d(const DecodeParams& p, int head_dim, int num_cus, hipStream_t stream) {
    switch (head_dim) {
        case 64: return launch_part_g<DT, 64>(p, num_cus, stream);
        case 128: return launch_part_g<DT, 128>(p, num_cus, stream);
        case 256: return launch_part_g<DT, 256>(p, num_cus, stream);
    }
    return hipErrorInvalidValue;
}

template <int DT>
hipError_t launch_merge_d(const DecodeParams& p, int head_dim, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(p.num_heads), static_cast<unsigned>(p.num_seqs));
    switch (head_dim) {
        case 64: hipLaunchKernelGGL((pa_merge<DT, 64>), grid, dim3(64), 0, stream, p); break;
        case 128: hipLaunchKernelGGL((pa_merge<DT, 128>), grid, dim3(64), 0, stream, p); break;
        case 256: hipLaunchKernelGGL((pa_merge<DT, 256>), grid, dim3(64), 0, stream, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

bool decode_supported(pa_dtype_t dt, int head_dim, int group) {
    const bool d_ok = head_dim == 64 || head_dim == 128 || head_dim == 256;
    const bool g_ok = group == 1 || group == 2 || group == 4 || group == 8;
    const bool t_ok = dt == PA_F32 || dt == PA_BF16 || dt == PA_F16;
    return d_ok && g_ok && t_ok;
}

hipError_t launch_decode_partitions(const DecodeParams& p, pa_dtype_t dt, int head_dim,
                                    int num_cus, hipStream_t stream) {
    switch (dt) {
        case PA_F32: return launch_part_d<PA_F32>(p, head_dim, num_cus, stream);
        case PA_BF16: return launch_part_d<PA_BF16>(p, head_dim, num_cus, stream);
        case PA_F16: return launch_part_d<PA_F16>(p, head_dim, num_cus, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_decode_merge(const DecodeParams& p, pa_dtype_t dt, int head_dim,
                               hipStream_t stream) {
    if (p.pmax <= 1) return hipSuccess;  // every sequence was written directly
    switch (dt) {
        case PA_F32: return launch_merge_d<PA_F32>(p, head_dim, stream);
        case PA_BF16: return launch_merge_d<PA_BF16>(p, head_dim, stream);
        case PA_F16: return launch_merge_d<PA_F16>(p, head_dim, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace pa
