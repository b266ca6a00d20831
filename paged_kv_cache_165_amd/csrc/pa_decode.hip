// Paged decode attention kernels for gfx950 (MI355X).
//
// Operation (aiqz.cc tutorial, section 块表映射机制, equation pid/off; the
// lihaoran.work note, section 块表把逻辑顺序映射到物理位置): token t of a sequence
// lives at block_table[t / B], offset t % B; attention over all visible tokens
// is ordinary softmax attention, only the addressing differs.
//
// Cache layout. K: [NB][Hkv][B][D] (one 16-byte lane load = part of a row).
// V: [NB][Hkv][B/T][D][T] with T = min(B, 16): every block holds its V rows
// as tiles of T tokens stored head_dim-major, so the token index -- the axis
// P.V contracts over -- is contiguous. Each 16-token step therefore reads one
// contiguous run of V bytes, and the MFMA operand of P.V is a plain load.
//
// Work decomposition. An item is (sequence, KV head, partition of `part`
// tokens). A persistent grid of 256-thread workgroups walks the items largest
// first; every workgroup first builds that order in LDS (a prefix sum of full
// partitions, searched by bisection, then the partial partitions sorted by
// size: see "Work order and assignment" below). Either the four waves of a
// workgroup share one item and take its steps round robin, or (the
// wave-item kernel) each wave reduces whole items alone. The slice of the
// block table the partition reads is staged in LDS (cf-1.com blog, 2.2 and
// 5.4: table lookups served from shared memory, not global memory). K/V are
// streamed with nontemporal 16-byte loads, the next step always in flight
// while the current one is reduced (cf-1.com 5.1 and 6.2: prefetch the next
// physical block).
//
// Two inner loops, four kernels:
//  * pa_decode_valu (float32, and one query head per KV head where the
//    stream split below does not run): q.k is a per-lane partial dot product
//    finished by a DPP butterfly over the lanes that hold one K row; each
//    lane keeps an online softmax over its rows and accumulates P.V with FMAs.
//  * the MFMA tile code (bfloat16/float16): the heads sharing a KV head form
//    a small dense product (one distinct column with one head). Per 16-token
//    tile, S^T = K Q^T is D/32 v_mfma_f32_16x16x32 (K rows as A, the group's
//    query rows as B columns), and O^T += V^T P^T is D/16 v_mfma_f32_16x16x16
//    whose B operand is exactly the lane layout of S^T after exp2, so P never
//    leaves registers. The softmax max is rescaled lazily (only when a tile's
//    max exceeds the running max by more than 2^8). pa_decode_stream deals
//    the batch's 16-key tiles evenly over a persistent grid's waves, each
//    merging the partitions of its stretch in registers (partitions of at
//    most kWaveSlice blocks, any group and block size); pa_decode_mfma_wave
//    runs the same tile code with one item per wave where the stream's
//    32-bit cost positions could overflow; pa_decode_mfma shares an item
//    among the workgroup's waves, for longer partitions.
// Lanes, then (workgroup items) waves through LDS, are merged by the
// log-sum-exp rule.
// A sequence that fits one partition is written straight to `out`; longer
// ones leave one (m, l, o) record per partition for the merge kernel.

#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kTblPerThread = kMaxTableSlice / kThreads;  // table entries each thread stages
static_assert(kTblPerThread * kThreads == kMaxTableSlice, "whole table entries per thread");

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int clamp_ctx(int L, const DecodeParams& p) {
    L = L < 0 ? 0 : L;
    return L > p.max_ctx ? p.max_ctx : L;
}

struct Item {
    int s, kv, pidx, nparts, t0, t1, b0, nblk;
};

__host__ __device__ constexpr size_t red_stride(int d) { return static_cast<size_t>(d) + 4; }

// ---------------------------------------------------------------------------
// Work order and assignment
// ---------------------------------------------------------------------------
//
// Items are ordered largest first: every full partition of every sequence
// (sequence-major), then the partial last partitions sorted by size from
// largest to smallest (stable counting sort into kBuckets size classes), then
// empty sequences; the KV heads of one (sequence, partition) are consecutive
// items. Each workgroup builds this order in LDS (fullpre: prefix sum of full
// partitions per sequence; plist: sequences with a partial partition, in
// order) and takes items in a snake: round r gives item r * G + g to
// workgroup g for even r and to workgroup G - 1 - g for odd r. Over a
// largest-first order this balances about as well as a shared queue, without
// the device-scope atomic per item that a queue costs.

constexpr int kBuckets = 256;

// LDS ints of the schedule: fullpre[S + 1] | plist[S] | lens[S] | bucket[kBuckets]
// | the build's scratch: wave_tot[kWaves] | wave_cnt[kWaves][kBuckets]. All of
// it is dynamic LDS, so that the kernels hold no static LDS and a launch's
// LDS is exactly what the host plan computes.
__host__ __device__ constexpr size_t sched_ints(int num_seqs) {
    return static_cast<size_t>((num_seqs + 4) & ~3) + 2 * static_cast<size_t>((num_seqs + 3) & ~3) + kBuckets +
           kWaves + static_cast<size_t>(kWaves) * kBuckets;
}

struct Sched {
    int* fullpre;
    int* plist;
    int* lens;   // context lengths, clamped to [0, max_ctx]
    int* bucket;
    int* wave_tot;  // scratch of build_schedule
    int* wave_cnt;  // [kWaves][kBuckets], scratch of build_schedule
    int full;    // number of full partitions
    int total;   // number of items
};

__device__ __forceinline__ Sched sched_lds(const DecodeParams& p, int* base) {
    Sched sc;
    sc.fullpre = base;
    sc.plist = sc.fullpre + ((p.num_seqs + 4) & ~3);
    sc.lens = sc.plist + ((p.num_seqs + 3) & ~3);
    sc.bucket = sc.lens + ((p.num_seqs + 3) & ~3);
    sc.wave_tot = sc.bucket + kBuckets;
    sc.wave_cnt = sc.wave_tot + kWaves;
    sc.full = sc.total = 0;
    return sc;
}

// Size class of a partial partition of r tokens (r = 0: empty sequence):
// larger partials get smaller classes.
__device__ __forceinline__ int size_class(int r, int part) {
    if (r == 0) return kBuckets - 1;
    return static_cast<int>((static_cast<long long>(part - 1 - r) * kBuckets) / part);
}

// Every thread of the workgroup takes part; fills sc.full and sc.total.
// Every workgroup must derive the same order, so the partial list is a
// stable counting sort: sequences of one size class keep their index order
// (ranks inside a wave come from ballots, not from atomics).
__device__ void build_schedule(const DecodeParams& p, Sched& sc) {
    static_assert(kBuckets == kThreads, "one size class per thread");
    int* wave_tot = sc.wave_tot;
    int (*wave_cnt)[kBuckets] = reinterpret_cast<int (*)[kBuckets]>(sc.wave_cnt);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int S = p.num_seqs;
    sc.bucket[tid] = 0;
    if (tid == 0) sc.fullpre[0] = 0;
    __syncthreads();
    int carry = 0;
    for (int base = 0; base < S; base += kThreads) {
        const int i = base + tid;
        int nf = 0;
        if (i < S) {
            const int L = clamp_ctx(p.context_lens[i], p);
            sc.lens[i] = L;
            nf = L / p.part;
            const int r = L - nf * p.part;
            if (r != 0 || L == 0) atomicAdd(&sc.bucket[size_class(r, p.part)], 1);
        }
        int x = nf;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (lane == 63) wave_tot[wave] = x;
        __syncthreads();
        int add = carry;
        for (int w = 0; w < wave; ++w) add += wave_tot[w];
        if (i < S) sc.fullpre[i + 1] = x + add;
        carry += wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
        __syncthreads();
    }
    // exclusive scan of the class sizes: class c starts at bucket[c]
    int x = sc.bucket[tid];
    const int own = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) wave_tot[wave] = x;
    __syncthreads();
    int add = 0;
    for (int w = 0; w < wave; ++w) add += wave_tot[w];
    const int partials = wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
    sc.bucket[tid] = x + add - own;  // cursor of class tid
    __syncthreads();
    for (int base = 0; base < S; base += kThreads) {
        const int i = base + tid;
        int c = -1;
        if (i < S) {
            const int L = sc.lens[i];
            const int r = L - (L / p.part) * p.part;
            if (r != 0 || L == 0) c = size_class(r, p.part);
        }
        // lanes of this wave in the same class, from one ballot per class bit
        unsigned long long same = __ballot(c >= 0);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const unsigned long long m = __ballot((c >> b) & 1);
            same &= ((c >> b) & 1) ? m : ~m;
        }
        const int rank = __popcll(same & ((1ull << lane) - 1ull));
        for (int w = 0; w < kWaves; ++w) wave_cnt[w][tid] = 0;
        __syncthreads();
        if (c >= 0 && rank == 0) wave_cnt[wave][c] = __popcll(same);
        __syncthreads();
        if (c >= 0) {
            int pos = sc.bucket[c] + rank;
            for (int w = 0; w < wave; ++w) pos += wave_cnt[w][c];
            sc.plist[pos] = i;
        }
        __syncthreads();
        sc.bucket[tid] += wave_cnt[0][tid] + wave_cnt[1][tid] + wave_cnt[2][tid] + wave_cnt[3][tid];
        __syncthreads();
    }
    sc.full = sc.fullpre[S];
    sc.total = (sc.full + partials) * p.num_kv_heads;
}

__device__ __forceinline__ Item item_at(const DecodeParams& p, const Sched& sc, int item) {
    Item it;
    const int j = item / p.num_kv_heads;
    it.kv = item - j * p.num_kv_heads;
    int s, pidx;
    if (j < sc.full) {
        int lo = 0, hi = p.num_seqs;  // fullpre[lo] <= j < fullpre[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (sc.fullpre[mid] <= j) lo = mid; else hi = mid;
        }
        s = lo;
        pidx = j - sc.fullpre[lo];
    } else {
        s = sc.plist[j - sc.full];
        pidx = -1;
    }
    const int L = sc.lens[s];
    const int nf = L / p.part;
    const bool partial = L - nf * p.part != 0 || L == 0;
    if (pidx < 0) pidx = nf;
    it.s = s;
    it.pidx = pidx;
    it.nparts = nf + (partial ? 1 : 0);
    it.t0 = pidx * p.part;
    it.t1 = min(L, it.t0 + p.part);
    it.b0 = it.t0 >> p.log2_bs;
    it.nblk = (it.t1 - it.t0 + (1 << p.log2_bs) - 1) >> p.log2_bs;
    return it;
}

// Item of round r for this workgroup (snake order), or -1 past the end.
__device__ __forceinline__ int snake_item(const Sched& sc, int r) {
    const int g = blockIdx.x, G = gridDim.x;
    const int item = r * G + ((r & 1) ? (G - 1 - g) : g);
    return item < sc.total ? item : -1;
}

__device__ __forceinline__ void stage_table(const DecodeParams& p, const Item& it, int* tbl) {
    for (int i = threadIdx.x; i < it.nblk; i += kThreads) {
        int pid = p.block_tables[static_cast<size_t>(it.s) * p.max_blocks + it.b0 + i];
        pid = pid < 0 ? 0 : (pid >= p.num_blocks ? p.num_blocks - 1 : pid);
        tbl[i] = pid;
    }
}

// Item results are not stored as soon as they are known: every global store
// holds back the streaming loads issued after it (measured: about 4 us per
// item on MI355X), so each workgroup keeps the results of up to
// `ring_slots` items in an LDS ring and writes them out together.
// Slot layout (floats): o[G][D] | m[G] | l[G] | s, kv, pidx, nparts (as ints).
__host__ __device__ constexpr int ring_slot_floats(int g, int d) { return ((g * d + 2 * g + 4) + 3) & ~3; }

// The MFMA kernel double-buffers its wave partials (no barrier between an
// item's combine and the next item's writes) when they are small enough.
__host__ __device__ constexpr bool mfma_red_double(int g, int d) { return g * d <= 1024; }

// Merge the waves' partial results held in `red` (per wave and head: D
// weighted V sums, then the running max in log2 units, then the sum of
// weights) into one ring slot.
template <int D, int G>
__device__ __forceinline__ void combine_to_ring(const Item& it, const float* red, float* slot) {
    constexpr int RS = static_cast<int>(red_stride(D));
    for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
        const int h = idx / D;
        const int d = idx - h * D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red[(w * G + h) * RS + D]);
        const float Mu = M == -INFINITY ? 0.f : M;
        float lsum = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float* r = red + (w * G + h) * RS;
            const float f = fast_exp2(r[D] - Mu);
            lsum += r[D + 1] * f;
            o += r[d] * f;
        }
        slot[idx] = lsum > 0.f ? o / lsum : 0.f;
        if (d == 0) {
            slot[G * D + h] = M;
            slot[G * D + G + h] = lsum;
        }
    }
    if (threadIdx.x == 0) {
        int* meta = reinterpret_cast<int*>(slot + G * D + 2 * G);
        meta[0] = it.s;
        meta[1] = it.kv;
        meta[2] = it.pidx;
        meta[3] = it.nparts;
    }
}

// Write `n` ring slots: a single-partition sequence's rows go to `out`
// (rounded to the element type), a partition's record to the workspace.
template <int DT, int D, int G>
__device__ __forceinline__ void flush_ring(const DecodeParams& p, const float* ring, int n) {
    using EL = Elem<DT>;
    constexpr int SL = ring_slot_floats(G, D);
    for (int i = 0; i < n; ++i) {
        const float* slot = ring + i * SL;
        const int* meta = reinterpret_cast<const int*>(slot + G * D + 2 * G);
        const int s = meta[0], kv = meta[1], pidx = meta[2], nparts = meta[3];
        const size_t row0 = static_cast<size_t>(s) * p.num_heads + kv * G;  // first query head row
        if (nparts == 1) {
            for (int idx = threadIdx.x; idx < G * D; idx += kThreads) EL::store(p.out, row0 * D + idx, slot[idx]);
        } else {
            for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
                const int h = idx / D;
                const int d = idx - h * D;
                p.ws_o[((row0 + h) * p.pmax + pidx) * D + d] = slot[idx];
            }
            if (threadIdx.x < G) {
                const size_t rec = (row0 + threadIdx.x) * p.pmax + pidx;
                p.ws_m[rec] = slot[G * D + threadIdx.x];
                p.ws_l[rec] = slot[G * D + G + threadIdx.x];
            }
        }
    }
}

template <typename T>
__device__ __forceinline__ T nt_load(const char* base, size_t byte_off) {
    return __builtin_nontemporal_load(reinterpret_cast<const T*>(base + byte_off));
}

// ---------------------------------------------------------------------------
// VALU kernel
// ---------------------------------------------------------------------------

// Row-group geometry of the VALU kernel for one (element size, D): LPR lanes
// hold one K row (16 bytes each), RPI row groups per wave, U consecutive
// tokens per row group and step.
template <int E, int D>
struct ValuGeom {
    static constexpr int EPL = 16 / E;
    static constexpr int LPR = D / EPL;
    static constexpr int RPI = 64 / LPR;
    static constexpr int U = RPI >= 4 ? 4 : 16 / RPI;
    static constexpr int STEP = RPI * U;
    static constexpr int VW = U * E / 4;  // 32-bit words of one lane's V^T segment
};

template <int DT, int D, int G, bool BIGB>
__global__ __launch_bounds__(kThreads) void pa_decode_valu(DecodeParams p) {
    using EL = Elem<DT>;
    constexpr int E = EL::E;
    using GM = ValuGeom<E, D>;
    constexpr int EPL = GM::EPL, LPR = GM::LPR, U = GM::U, STEP = GM::STEP, VW = GM::VW;
    constexpr int RS = static_cast<int>(red_stride(D));
    static_assert(LPR >= 8 && LPR <= 64 && GM::RPI * LPR == 64, "row mapping");
    static_assert(VW == 2 || VW % 4 == 0, "V segment is 8 bytes or a multiple of 16");
    constexpr int NVL = VW == 2 ? 1 : VW / 4;  // loads per V^T segment

    // LDS: schedule | tbl[kMaxTableSlice] | red[kWaves * G * RS] | ring[ring_slots]
    extern __shared__ __align__(16) unsigned char smem[];
    Sched sc = sched_lds(p, reinterpret_cast<int*>(smem));
    int* tbl = reinterpret_cast<int*>(smem) + sched_ints(p.num_seqs);
    float* red = reinterpret_cast<float*>(tbl + kMaxTableSlice);
    float* ring = red + kWaves * G * RS;
    constexpr int SL = ring_slot_floats(G, D);
    int nring = 0;

    // the wave index is uniform: branches on it stay scalar
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rg = lane / LPR;           // row group: tokens U*rg .. U*rg+U-1 of a step
    const int li = lane % LPR;
    const int dsl = li * EPL;            // K side: first head-dim element of the lane
    const int bs = 1 << p.log2_bs;
    const int vt = 1 << p.log2_vt;
    const int hkv = p.num_kv_heads;
    const size_t blk_el = static_cast<size_t>(bs) * D;  // elements of one (block, head) tile
    const char* kbase = static_cast<const char*>(p.k_cache);
    const char* vbase = static_cast<const char*>(p.v_cache);

    build_schedule(p, sc);

    for (int r = 0, item = snake_item(sc, 0); item >= 0;) {
        const Item it = item_at(p, sc, item);
        stage_table(p, it, tbl);
        __syncthreads();

        float qv[G][EPL];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const size_t qoff = (static_cast<size_t>(it.s) * p.num_heads + it.kv * G + h) * D + dsl;
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
        const int t1 = it.t1;
        const int ntok = t1 - it.t0;
        const int nsteps = ntok > 0 ? (ntok + STEP - 1) / STEP : 0;
        const int last_u = ntok > 0 ? ((t1 - 1) / U) * U : 0;  // first token of the last valid U-group

        struct Buf {
            u32x4 k[U];
            uint32_t v[EPL][NVL * 4];
        };

        auto load_step = [&](int step, Buf& b) {
            const int g0 = it.t0 + step * STEP + U * rg;  // first token of this lane's row group
            const int vtok = min(g0, last_u);
            int pid;
            if constexpr (BIGB) {
                pid = __builtin_amdgcn_readfirstlane(tbl[(min(it.t0 + step * STEP, t1 - 1) >> p.log2_bs) - it.b0]);
            } else {
                pid = tbl[(vtok >> p.log2_bs) - it.b0];
            }
            const size_t tile = (static_cast<size_t>(pid) * hkv + it.kv) * blk_el;
#pragma unroll
            for (int c = 0; c < U; ++c) {
                const int trow = min(g0 + c, t1 - 1);
                b.k[c] = nt_load<u32x4>(kbase, (tile + static_cast<size_t>(trow & (bs - 1)) * D + dsl) * E);
            }
            const int voff = vtok & (bs - 1);
            const size_t vt0 = tile + static_cast<size_t>(voff >> p.log2_vt) * D * vt + (voff & (vt - 1));
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const size_t el = vt0 + static_cast<size_t>(li + LPR * e) * vt;
                if constexpr (VW == 2) {
                    const u32x2 w = nt_load<u32x2>(vbase, el * E);
                    b.v[e][0] = w.x;
                    b.v[e][1] = w.y;
                } else {
#pragma unroll
                    for (int x = 0; x < NVL; ++x) {
                        const u32x4 w = nt_load<u32x4>(vbase, el * E + 16 * x);
                        b.v[e][4 * x] = w.x; b.v[e][4 * x + 1] = w.y;
                        b.v[e][4 * x + 2] = w.z; b.v[e][4 * x + 3] = w.w;
                    }
                }
            }
        };

        auto compute_step = [&](int step, const Buf& b) {
            const int g0 = it.t0 + step * STEP + U * rg;
            float x[U][G];
#pragma unroll
            for (int c = 0; c < U; ++c) {
                float kf[EPL];
                EL::to_float(b.k[c], kf);
                const bool valid = g0 + c < t1;
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
            for (int e = 0; e < EPL; ++e) {
                float vf[U];
                // tokens of this lane's segment past the context may hold
                // anything (NaN included): zero them so 0 * v stays 0
                if constexpr (E == 4) {
#pragma unroll
                    for (int c = 0; c < U; ++c) vf[c] = g0 + c < t1 ? u32_as_f32(b.v[e][c]) : 0.f;
                } else {
#pragma unroll
                    for (int c = 0; c < U; ++c) {
                        const uint32_t w = b.v[e][c >> 1];
                        const uint32_t half = (c & 1) ? (w >> 16) : (w & 0xffffu);
                        float f;
                        if constexpr (DT == PA_BF16) f = u32_as_f32(half << 16);
                        else f = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(half)));
                        vf[c] = g0 + c < t1 ? f : 0.f;
                    }
                }
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    float a = acc[h][e];
#pragma unroll
                    for (int c = 0; c < U; ++c) a = fmaf(pw[c][h], vf[c], a);
                    acc[h][e] = a;
                }
            }
        };

        int s0 = wave;
        if (s0 < nsteps) {
            Buf ba, bb;
            load_step(s0, ba);
            while (true) {
                const int s1 = s0 + kWaves;
                if (s1 < nsteps) load_step(s1, bb);
                compute_step(s0, ba);
                if (s1 >= nsteps) break;
                s0 = s1 + kWaves;
                if (s0 < nsteps) load_step(s0, ba);
                compute_step(s1, bb);
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
                const float b2 = fast_exp2(mo - mu);
                l[h] = l[h] * a + lo2 * b2;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[h][e] = acc[h][e] * a + __shfl_xor(acc[h][e], off) * b2;
                m[h] = mn;
            }
        }
        if (lane < LPR) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float* r = red + (wave * G + h) * RS;
#pragma unroll
                for (int e = 0; e < EPL; ++e) r[li + LPR * e] = acc[h][e];
                if (lane == 0) {
                    r[D] = m[h];
                    r[D + 1] = l[h];
                }
            }
        }
        __syncthreads();
        combine_to_ring<D, G>(it, red, ring + nring * SL);
        item = snake_item(sc, ++r);
        ++nring;
        if (nring == p.ring_slots || item < 0) {
            __syncthreads();
            flush_ring<DT, D, G>(p, ring, nring);
            nring = 0;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// MFMA kernel (grouped query heads, bfloat16 / float16)
// ---------------------------------------------------------------------------

template <int DT>
__device__ __forceinline__ f32x4_t mfma_qk(const u32x4& a, const u32x4& b, f32x4_t c) {
    if constexpr (DT == PA_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

template <int DT>
__device__ __forceinline__ f32x4_t mfma_pv(const u32x2& a, const u32x2& b, f32x4_t c) {
    if constexpr (DT == PA_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                         __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                     __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
}

// Two probabilities packed as the MFMA element type (round to nearest even);
// ra / rb return the rounded values so that the softmax denominator sums
// exactly the weights the numerator multiplies.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b, float& ra, float& rb) {
    if constexpr (DT == PA_BF16) {
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        const bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
        const uint32_t w = __builtin_bit_cast(uint32_t, v);
        ra = u32_as_f32(w << 16);
        rb = u32_as_f32(w & 0xffff0000u);
        return w;
    } else {
        typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
        const f16x2_t v = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
        ra = static_cast<float>(v.x);
        rb = static_cast<float>(v.y);
        return __builtin_bit_cast(uint32_t, v);
    }
}

template <int DT, int D, int G, bool BIGB>
__global__ __launch_bounds__(kThreads) void pa_decode_mfma(DecodeParams p) {
    static_assert(DT == PA_BF16 || DT == PA_F16, "MFMA path is for 16-bit elements");
    static_assert(G == 2 || G == 4 || G == 8 || G == 16, "group size");
    constexpr int E = 2;
    constexpr int NK = D / 32;   // 16x16x32 products for S^T
    constexpr int NV = D / 16;   // 16x16x16 products for O^T
    constexpr int RS = static_cast<int>(red_stride(D));
    constexpr int QW = G * D / 2;                    // 32-bit words of one item's query block
    constexpr int QPT = (QW + kThreads - 1) / kThreads;
    constexpr float kLazy = 8.f;  // rescale only when the max grows by more than 2^8
    constexpr bool kRed2 = mfma_red_double(G, D);

    // LDS: schedule | tbl[2][kMaxTableSlice] | qs[2][QW] | red[1 or 2][kWaves * G * RS] | ring[ring_slots]
    extern __shared__ __align__(16) unsigned char smem[];
    Sched sc = sched_lds(p, reinterpret_cast<int*>(smem));
    int* tbl2 = reinterpret_cast<int*>(smem) + sched_ints(p.num_seqs);
    uint32_t* qs2 = reinterpret_cast<uint32_t*>(tbl2 + 2 * kMaxTableSlice);
    float* red2 = reinterpret_cast<float*>(qs2 + 2 * ((QW + 3) & ~3));
    float* ring = red2 + (kRed2 ? 2 : 1) * kWaves * G * RS;
    constexpr int SL = ring_slot_floats(G, D);
    int nring = 0;

    // the wave index is uniform: branches on it stay scalar
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15;  // K row of the tile (A) / head column (B, C)
    const int j = lane >> 4;    // 8-element chunk of K / 4-token group of V and S
    const int bs = 1 << p.log2_bs;
    const int vt = 1 << p.log2_vt;
    const int hkv = p.num_kv_heads;
    const size_t blk_el = static_cast<size_t>(bs) * D;
    const char* kbase = static_cast<const char*>(p.k_cache);
    const char* vbase = static_cast<const char*>(p.v_cache);
    const uint32_t* qwords = static_cast<const uint32_t*>(p.q);

    build_schedule(p, sc);
    const int item0 = snake_item(sc, 0);
    if (item0 < 0) return;

    struct Buf {
        u32x4 k[NK];
        u32x2 v[NV];
    };
    auto ntiles_of = [](const Item& x) { return x.t1 > x.t0 ? (x.t1 - x.t0 + 15) >> 4 : 0; };
    auto last4_of = [](const Item& x) { return x.t1 > x.t0 ? ((x.t1 - 1) >> 2) << 2 : 0; };
    auto q_word0 = [&](const Item& x) {
        return (static_cast<size_t>(x.s) * p.num_heads + x.kv * G) * (D / 2);
    };
    auto clamp_pid = [&](int pid) { return pid < 0 ? 0 : (pid >= p.num_blocks ? p.num_blocks - 1 : pid); };

    // K/V loads of one 16-token tile. `pk`/`pv` are this lane's physical
    // blocks for its K row and its 4-token V group.
    auto load_with = [&](const Item& x, int tile, int pk, int pv, Buf& b) {
        const int t1 = x.t1;
        const int tt0 = x.t0 + 16 * tile;
        const int krow = min(tt0 + r16, t1 - 1);
        const int vtok = min(tt0 + 4 * j, last4_of(x));
        if constexpr (BIGB) {
            // the tile lies in one block and one 16-token V tile: scalar
            // bases, 32-bit lane offsets, immediate offsets per load
            const int pid = __builtin_amdgcn_readfirstlane(pk);
            const size_t tile_el = (static_cast<size_t>(pid) * hkv + x.kv) * blk_el;
            const char* kt = kbase + tile_el * E;
            const char* vtp = vbase + (tile_el + static_cast<size_t>((tt0 & (bs - 1)) >> 4) * D * 16) * E;
            const uint32_t ko = static_cast<uint32_t>(((krow & (bs - 1)) * D + 8 * j) * E);
            const uint32_t vo = static_cast<uint32_t>(((vtok & 15) + 16 * r16) * E);
#pragma unroll
            for (int c = 0; c < NK; ++c) b.k[c] = nt_load<u32x4>(kt, ko + 64 * c);
#pragma unroll
            for (int v = 0; v < NV; ++v) b.v[v] = nt_load<u32x2>(vtp, vo + 512 * v);
        } else {
            const size_t kel = (static_cast<size_t>(pk) * hkv + x.kv) * blk_el +
                               static_cast<size_t>(krow & (bs - 1)) * D + 8 * j;
#pragma unroll
            for (int c = 0; c < NK; ++c) b.k[c] = nt_load<u32x4>(kbase, (kel + 32 * c) * E);
            const int voff = vtok & (bs - 1);
            const size_t vel = (static_cast<size_t>(pv) * hkv + x.kv) * blk_el +
                               static_cast<size_t>(voff >> p.log2_vt) * D * vt + (voff & (vt - 1)) +
                               static_cast<size_t>(r16) * vt;
#pragma unroll
            for (int v = 0; v < NV; ++v)
                b.v[v] = nt_load<u32x2>(vbase, (vel + static_cast<size_t>(16 * v) * vt) * E);
        }
    };
    // this lane's physical blocks (K row, 4-token V group) of `tile` of `x`,
    // from x's table slice in LDS
    auto tile_blocks = [&](const Item& x, const int* tbl, int tile, int& pk, int& pv) {
        const int tt0 = x.t0 + 16 * tile;
        if constexpr (BIGB) {
            pk = pv = tbl[(min(tt0, x.t1 - 1) >> p.log2_bs) - x.b0];
        } else {
            pk = tbl[(min(tt0 + r16, x.t1 - 1) >> p.log2_bs) - x.b0];
            pv = tbl[(min(tt0 + 4 * j, last4_of(x)) >> p.log2_bs) - x.b0];
        }
    };

    // Load schedule. The compiler waits for a load by counting the memory
    // operations issued after it, and where paths issue different numbers
    // of loads it must assume the fewest -- a conditional prefetch would make
    // the reduction of one tile wait for the next tile too. So every step of
    // every wave issues the same loads: the next tile of the item, else the
    // wave's first tile of the next item, else a dummy tile of block 0
    // (in bounds, and cached after its first read). The next item's table
    // slice, query block and first-tile block ids are likewise loaded raw on
    // every item, from a harmless address when there is nothing to load, and
    // are clamped only where they are used.

    // ---- prologue: the first item's table slice and query block, the next
    // item's descriptor, this wave's first tile
    Item cur = item_at(p, sc, item0);
    int next_item = snake_item(sc, 1);
    Item nxt = next_item >= 0 ? item_at(p, sc, next_item) : cur;
    stage_table(p, cur, tbl2);
    for (int w = tid; w < QW; w += kThreads) qs2[w] = qwords[q_word0(cur) + w];
    __syncthreads();
    Buf A, B;
    {
        int pk = 0, pv = 0;
        const bool real = wave < ntiles_of(cur);
        if (real) tile_blocks(cur, tbl2, wave, pk, pv);
        load_with(cur, real ? wave : 0, pk, pv, A);
    }

    for (int k = 0;; ++k) {
        const int buf = k & 1;
        const int* tbl = tbl2 + buf * kMaxTableSlice;
        const bool has_next = next_item >= 0;
        const bool next_tile = has_next && wave < ntiles_of(nxt);
        // raw metadata of the next item (see the load schedule above)
        const int* trow = p.block_tables + static_cast<size_t>(nxt.s) * p.max_blocks + nxt.b0;
        const int* safe = p.context_lens;
        int pk_raw, pv_raw;
        {
            const int tt0 = nxt.t0 + 16 * wave;
            if constexpr (BIGB) {
                pk_raw = *(next_tile ? trow + ((min(tt0, nxt.t1 - 1) >> p.log2_bs) - nxt.b0) : safe);
                pv_raw = pk_raw;
            } else {
                pk_raw = *(next_tile ? trow + ((min(tt0 + r16, nxt.t1 - 1) >> p.log2_bs) - nxt.b0) : safe);
                pv_raw = *(next_tile ? trow + ((min(tt0 + 4 * j, last4_of(nxt)) >> p.log2_bs) - nxt.b0) : safe);
            }
        }
        int tbl_raw[kTblPerThread];
#pragma unroll
        for (int i = 0; i < kTblPerThread; ++i)
            tbl_raw[i] = *(has_next && tid + i * kThreads < nxt.nblk ? trow + tid + i * kThreads : safe);
        uint32_t q_raw[QPT];
#pragma unroll
        for (int i = 0; i < QPT; ++i) q_raw[i] = qwords[q_word0(nxt) + min(tid + i * kThreads, QW - 1)];

        // query fragments of this item from LDS: column r16 is head (r16 % G)
        u32x4 qf[NK];
        {
            const uint32_t* qrow = qs2 + buf * ((QW + 3) & ~3) + (r16 % G) * (D / 2);
#pragma unroll
            for (int c = 0; c < NK; ++c) qf[c] = *reinterpret_cast<const u32x4*>(qrow + 16 * c + 4 * j);
        }
        f32x4_t acc[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[v] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        float m_run = -INFINITY, lsum = 0.f;
        const int t1 = cur.t1;
        const int ntiles = ntiles_of(cur);

        auto compute_tile = [&](int tile, const Buf& b) {
            const int tt0 = cur.t0 + 16 * tile;
            f32x4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NK; ++c) st = mfma_qk<DT>(b.k[c], qf[c], st);
            // st[r] = S^T[token tt0 + 4j + r][head column r16]
            float x[4];
            bool valid[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                valid[r] = tt0 + 4 * j + r < t1;
                x[r] = valid[r] ? st[r] * p.scale_log2 : -INFINITY;
            }
            float tmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
            const bool need = tmax > m_run + kLazy;
            if (__any(need)) {
                const float mn = need ? tmax : m_run;
                const float alpha = fast_exp2(m_run - mn);
#pragma unroll
                for (int v = 0; v < NV; ++v) acc[v] *= alpha;
                lsum *= alpha;
                m_run = mn;
            }
            float pr[4];
            u32x2 pb;
            pb.x = pack2<DT>(fast_exp2(x[0] - m_run), fast_exp2(x[1] - m_run), pr[0], pr[1]);
            pb.y = pack2<DT>(fast_exp2(x[2] - m_run), fast_exp2(x[3] - m_run), pr[2], pr[3]);
            lsum += (pr[0] + pr[1]) + (pr[2] + pr[3]);
            // V^T values of tokens past the context may hold anything: zero them
            const uint32_t mask0 = (valid[0] ? 0xffffu : 0u) | (valid[1] ? 0xffff0000u : 0u);
            const uint32_t mask1 = (valid[2] ? 0xffffu : 0u) | (valid[3] ? 0xffff0000u : 0u);
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                u32x2 a = b.v[v];
                a.x &= mask0;
                a.y &= mask1;
                acc[v] = mfma_pv<DT>(a, pb, acc[v]);
            }
        };

        auto load_tile = [&](int tile, Buf& b) {
            int pk, pv;
            tile_blocks(cur, tbl, tile, pk, pv);
            load_with(cur, tile, pk, pv, b);
        };
        // this wave's first tile of the next item, else a dummy. The empty
        // asm keeps the use of the raw block ids here: hoisted to the top of
        // the item, it would wait for loads issued just before.
        auto load_next = [&](Buf& b) {
            int pk = pk_raw, pv = pv_raw;
            asm volatile("" : "+v"(pk), "+v"(pv));
            if (next_tile) load_with(nxt, wave, clamp_pid(pk), clamp_pid(pv), b);
            else load_with(cur, 0, 0, 0, b);
        };

        // This wave's tiles of the item, two deep. A holds the wave's first
        // tile on entry and the next item's first tile on exit; B is loaded
        // and reduced within one pass. Only A (and the accumulators) live
        // across the loop, a plain counted loop over the pairs of tiles that
        // another tile follows, and the next item's first tile is loaded at
        // one point that every path reaches: the compiler then keeps A in
        // place instead of copying a buffer whose loads are in flight, and
        // each wait counts exactly the loads issued after what it waits for.
        // The scheduling barriers keep each load group ahead of the reduction
        // after it, and A's reads ahead of its refill.
        const int mine = wave < ntiles ? (ntiles - 1 - wave) / kWaves + 1 : 0;  // this wave's tiles
        int t = wave;
        if (mine > 0) {
            for (int i = 0; i < ((mine - 1) >> 1); ++i) {
                load_tile(t + kWaves, B);
                __builtin_amdgcn_sched_barrier(0);
                compute_tile(t, A);
                __builtin_amdgcn_sched_barrier(0);
                load_tile(t + 2 * kWaves, A);
                __builtin_amdgcn_sched_barrier(0);
                compute_tile(t + kWaves, B);
                t += 2 * kWaves;
            }
            if (mine & 1) {
                compute_tile(t, A);
            } else {
                load_tile(t + kWaves, B);
                __builtin_amdgcn_sched_barrier(0);
                compute_tile(t, A);
                compute_tile(t + kWaves, B);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        load_next(A);  // (a wave without a tile here replaces a dummy)
        // every path has used the raw block ids by now (the compiler cannot
        // tell): say so, so that no later reuse of their registers waits
        asm volatile("" ::"v"(pk_raw), "v"(pv_raw));

        // acc[v][r] = O^T[d = 16v + 4j + r][head column r16]; lsum covers this
        // lane's 4-token groups only: total it over the four lanes of the column
        lsum += __shfl_xor(lsum, 16);
        lsum += __shfl_xor(lsum, 32);
        float* red = red2 + (kRed2 ? buf : 0) * (kWaves * G * RS);
        if (r16 < G) {
            float* r = red + (wave * G + r16) * RS;
#pragma unroll
            for (int v = 0; v < NV; ++v) *reinterpret_cast<f32x4_t*>(r + 16 * v + 4 * j) = acc[v];
            if (j == 0) {
                r[D] = m_run;
                r[D + 1] = lsum;
            }
        }
        {
            // The next item's table slice and query block go to the other
            // buffers, which nobody reads during this item. The stores are
            // unconditional (entries past the slice are never read; lanes past
            // the query block repeat its last word) so that every path
            // consumes the raw loads.
#pragma unroll
            for (int i = 0; i < kTblPerThread; ++i)
                tbl2[(buf ^ 1) * kMaxTableSlice + tid + i * kThreads] = clamp_pid(tbl_raw[i]);
            uint32_t* qn = qs2 + (buf ^ 1) * ((QW + 3) & ~3);
#pragma unroll
            for (int i = 0; i < QPT; ++i) qn[min(tid + i * kThreads, QW - 1)] = q_raw[i];
        }
        __syncthreads();
        combine_to_ring<D, G>(cur, red, ring + nring * SL);
        ++nring;
        if constexpr (!kRed2) __syncthreads();  // the next item rewrites the single partials buffer
        if (nring == p.ring_slots || !has_next) {
            __syncthreads();
            flush_ring<DT, D, G>(p, ring, nring);
            nring = 0;
        }
        if (!has_next) break;
        cur = nxt;
        next_item = snake_item(sc, k + 2);
        if (next_item >= 0) nxt = item_at(p, sc, next_item);
    }
}

// ---------------------------------------------------------------------------
// MFMA kernel, one item per wave
// ---------------------------------------------------------------------------
//
// The per-tile products and softmax of pa_decode_mfma, but each wave reduces
// whole items on its own: after the schedule is built the waves of a
// workgroup never wait for each other, and an item ends without a
// cross-wave combine. Items are dealt to the waves of the grid (numbered
// workgroup-major) in the same largest-first snake. Each wave keeps in LDS
// its item's table slice and query block and its own result ring, which it
// flushes itself. The next item's slice and query block are loaded raw
// during the current item and stored over the current ones at its end,
// when the tile loop no longer reads the slice and the query fragments are
// in registers.

__host__ __device__ constexpr int wave_q_words(int g, int d) { return ((g * d / 2) + 3) & ~3; }

template <int DT, int D, int G, bool BIGB>
__global__ __launch_bounds__(kThreads) void pa_decode_mfma_wave(DecodeParams p) {
    static_assert(DT == PA_BF16 || DT == PA_F16, "MFMA path is for 16-bit elements");
    static_assert(G == 2 || G == 4 || G == 8 || G == 16, "group size");
    using EL = Elem<DT>;
    constexpr int E = 2;
    constexpr int NK = D / 32;
    constexpr int NV = D / 16;
    constexpr int QW = G * D / 2;
    constexpr int QWP = wave_q_words(G, D);
    constexpr int QPL = (QW + 63) / 64;
    constexpr int TPL = kWaveSlice / 64;
    constexpr float kLazy = 8.f;
    constexpr int SL = ring_slot_floats(G, D);

    // LDS: schedule | tbl[kWaves][kWaveSlice] | qs[kWaves][QWP] | ring[kWaves][wring]
    extern __shared__ __align__(16) unsigned char smem[];
    Sched sc = sched_lds(p, reinterpret_cast<int*>(smem));
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int* tbl_all = reinterpret_cast<int*>(smem) + sched_ints(p.num_seqs);
    uint32_t* qs_all = reinterpret_cast<uint32_t*>(tbl_all + kWaves * kWaveSlice);
    float* ring_all = reinterpret_cast<float*>(qs_all + kWaves * QWP);
    const int wring = p.ring_slots / kWaves;
    int* tbl = tbl_all + wave * kWaveSlice;
    uint32_t* qs = qs_all + wave * QWP;
    float* ring = ring_all + wave * wring * SL;
    int nring = 0;

    const int r16 = lane & 15;
    const int j = lane >> 4;
    const int bs = 1 << p.log2_bs;
    const int vt = 1 << p.log2_vt;
    const int hkv = p.num_kv_heads;
    const size_t blk_el = static_cast<size_t>(bs) * D;
    const char* kbase = static_cast<const char*>(p.k_cache);
    const char* vbase = static_cast<const char*>(p.v_cache);
    const uint32_t* qwords = static_cast<const uint32_t*>(p.q);

    build_schedule(p, sc);  // the last barrier of the kernel
    const int W = gridDim.x * kWaves;
    const int gw = blockIdx.x * kWaves + wave;
    auto wave_item = [&](int r) -> int {
        const int it = r * W + ((r & 1) ? (W - 1 - gw) : gw);
        return it < sc.total ? it : -1;
    };
    const int item0 = wave_item(0);
    if (item0 < 0) return;

    struct Buf {
        u32x4 k[NK];
        u32x2 v[NV];
    };
    auto ntiles_of = [](const Item& x) { return x.t1 > x.t0 ? (x.t1 - x.t0 + 15) >> 4 : 0; };
    auto last4_of = [](const Item& x) { return x.t1 > x.t0 ? ((x.t1 - 1) >> 2) << 2 : 0; };
    auto q_word0 = [&](const Item& x) {
        return (static_cast<size_t>(x.s) * p.num_heads + x.kv * G) * (D / 2);
    };
    auto clamp_pid = [&](int pid) { return pid < 0 ? 0 : (pid >= p.num_blocks ? p.num_blocks - 1 : pid); };

    auto load_with = [&](const Item& x, int tile, int pk, int pv, Buf& b) {
        const int t1 = x.t1;
        const int tt0 = x.t0 + 16 * tile;
        const int krow = min(tt0 + r16, t1 - 1);
        const int vtok = min(tt0 + 4 * j, last4_of(x));
        if constexpr (BIGB) {
            const int pid = __builtin_amdgcn_readfirstlane(pk);
            const size_t tile_el = (static_cast<size_t>(pid) * hkv + x.kv) * blk_el;
            const char* kt = kbase + tile_el * E;
            const char* vtp = vbase + (tile_el + static_cast<size_t>((tt0 & (bs - 1)) >> 4) * D * 16) * E;
            const uint32_t ko = static_cast<uint32_t>(((krow & (bs - 1)) * D + 8 * j) * E);
            const uint32_t vo = static_cast<uint32_t>(((vtok & 15) + 16 * r16) * E);
#pragma unroll
            for (int c = 0; c < NK; ++c) b.k[c] = nt_load<u32x4>(kt, ko + 64 * c);
#pragma unroll
            for (int v = 0; v < NV; ++v) b.v[v] = nt_load<u32x2>(vtp, vo + 512 * v);
        } else {
            const size_t kel = (static_cast<size_t>(pk) * hkv + x.kv) * blk_el +
                               static_cast<size_t>(krow & (bs - 1)) * D + 8 * j;
#pragma unroll
            for (int c = 0; c < NK; ++c) b.k[c] = nt_load<u32x4>(kbase, (kel + 32 * c) * E);
            const int voff = vtok & (bs - 1);
            const size_t vel = (static_cast<size_t>(pv) * hkv + x.kv) * blk_el +
                               static_cast<size_t>(voff >> p.log2_vt) * D * vt + (voff & (vt - 1)) +
                               static_cast<size_t>(r16) * vt;
#pragma unroll
            for (int v = 0; v < NV; ++v)
                b.v[v] = nt_load<u32x2>(vbase, (vel + static_cast<size_t>(16 * v) * vt) * E);
        }
    };
    auto tile_blocks = [&](const Item& x, const int* tbl, int tile, int& pk, int& pv) {
        const int tt0 = x.t0 + 16 * tile;
        if constexpr (BIGB) {
            pk = pv = tbl[(min(tt0, x.t1 - 1) >> p.log2_bs) - x.b0];
        } else {
            pk = tbl[(min(tt0 + r16, x.t1 - 1) >> p.log2_bs) - x.b0];
            pv = tbl[(min(tt0 + 4 * j, last4_of(x)) >> p.log2_bs) - x.b0];
        }
    };
    auto stage_slice = [&](const Item& x, int* tbl) {
        const int* trow = p.block_tables + static_cast<size_t>(x.s) * p.max_blocks + x.b0;
#pragma unroll
        for (int i = 0; i < TPL; ++i)
            if (lane + 64 * i < x.nblk) tbl[lane + 64 * i] = clamp_pid(trow[lane + 64 * i]);
    };

    // prologue: the first item's table slice and query block, its first tile
    Item cur = item_at(p, sc, item0);
    int next_item = wave_item(1);
    Item nxt = next_item >= 0 ? item_at(p, sc, next_item) : cur;
    stage_slice(cur, tbl);
    for (int w = lane; w < QW; w += 64) qs[w] = qwords[q_word0(cur) + w];
    Buf A, B;
    {
        int pk = 0, pv = 0;
        const bool real = ntiles_of(cur) > 0;
        if (real) tile_blocks(cur, tbl, 0, pk, pv);
        load_with(cur, 0, pk, pv, A);
    }

    for (int k = 0;; ++k) {
        const bool has_next = next_item >= 0;
        const bool next_tile = has_next && ntiles_of(nxt) > 0;
        // raw loads of the next item's metadata, consumed at the end
        const int* trow = p.block_tables + static_cast<size_t>(nxt.s) * p.max_blocks + nxt.b0;
        const int* safe = p.context_lens;
        int pk_raw, pv_raw;
        if constexpr (BIGB) {
            pk_raw = *(next_tile ? trow : safe);
            pv_raw = pk_raw;
        } else {
            pk_raw = *(next_tile ? trow + ((min(nxt.t0 + r16, nxt.t1 - 1) >> p.log2_bs) - nxt.b0) : safe);
            pv_raw = *(next_tile ? trow + ((min(nxt.t0 + 4 * j, last4_of(nxt)) >> p.log2_bs) - nxt.b0) : safe);
        }
        int tbl_raw[TPL];
#pragma unroll
        for (int i = 0; i < TPL; ++i)
            tbl_raw[i] = *(has_next && lane + 64 * i < nxt.nblk ? trow + lane + 64 * i : safe);
        uint32_t q_raw[QPL];
#pragma unroll
        for (int i = 0; i < QPL; ++i) q_raw[i] = qwords[q_word0(nxt) + min(lane + 64 * i, QW - 1)];

        u32x4 qf[NK];
        {
            const uint32_t* qrow = qs + (r16 % G) * (D / 2);
#pragma unroll
            for (int c = 0; c < NK; ++c) qf[c] = *reinterpret_cast<const u32x4*>(qrow + 16 * c + 4 * j);
        }
        f32x4_t acc[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[v] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        float m_run = -INFINITY, lsum = 0.f;
        const int t1 = cur.t1;
        const int ntiles = ntiles_of(cur);

        auto compute_tile = [&](int tile, const Buf& b) {
            const int tt0 = cur.t0 + 16 * tile;
            f32x4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NK; ++c) st = mfma_qk<DT>(b.k[c], qf[c], st);
            float x[4];
            bool valid[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                valid[r] = tt0 + 4 * j + r < t1;
                x[r] = valid[r] ? st[r] * p.scale_log2 : -INFINITY;
            }
            float tmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
            const bool need = tmax > m_run + kLazy;
            if (__any(need)) {
                const float mn = need ? tmax : m_run;
                const float alpha = fast_exp2(m_run - mn);
#pragma unroll
                for (int v = 0; v < NV; ++v) acc[v] *= alpha;
                lsum *= alpha;
                m_run = mn;
            }
            float pr[4];
            u32x2 pb;
            pb.x = pack2<DT>(fast_exp2(x[0] - m_run), fast_exp2(x[1] - m_run), pr[0], pr[1]);
            pb.y = pack2<DT>(fast_exp2(x[2] - m_run), fast_exp2(x[3] - m_run), pr[2], pr[3]);
            lsum += (pr[0] + pr[1]) + (pr[2] + pr[3]);
            const uint32_t mask0 = (valid[0] ? 0xffffu : 0u) | (valid[1] ? 0xffff0000u : 0u);
            const uint32_t mask1 = (valid[2] ? 0xffffu : 0u) | (valid[3] ? 0xffff0000u : 0u);
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                u32x2 a = b.v[v];
                a.x &= mask0;
                a.y &= mask1;
                acc[v] = mfma_pv<DT>(a, pb, acc[v]);
            }
        };
        auto load_tile = [&](int tile, Buf& b) {
            int pk, pv;
            tile_blocks(cur, tbl, tile, pk, pv);
            load_with(cur, tile, pk, pv, b);
        };
        auto load_next = [&](Buf& b) {
            int pk = pk_raw, pv = pv_raw;
            asm volatile("" : "+v"(pk), "+v"(pv));
            if (next_tile) load_with(nxt, 0, clamp_pid(pk), clamp_pid(pv), b);
            else load_with(cur, 0, 0, 0, b);
        };

        // the item's tiles, two deep (the structure of pa_decode_mfma with
        // one wave taking every tile)
        int t = 0;
        if (ntiles > 0) {
            for (int i = 0; i < ((ntiles - 1) >> 1); ++i) {
                load_tile(t + 1, B);
                __builtin_amdgcn_sched_barrier(0);
                compute_tile(t, A);
                __builtin_amdgcn_sched_barrier(0);
                load_tile(t + 2, A);
                __builtin_amdgcn_sched_barrier(0);
                compute_tile(t + 1, B);
                t += 2;
            }
            if (ntiles & 1) {
                compute_tile(t, A);
            } else {
                load_tile(t + 1, B);
                __builtin_amdgcn_sched_barrier(0);
                compute_tile(t, A);
                compute_tile(t + 1, B);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        load_next(A);
        asm volatile("" ::"v"(pk_raw), "v"(pv_raw));

        // acc[v][r] = O^T[d = 16v + 4j + r][head column r16]
        lsum += __shfl_xor(lsum, 16);
        lsum += __shfl_xor(lsum, 32);
        {
            float* slot = ring + nring * SL;
            if (r16 < G) {
                const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    f32x4_t o = acc[v] * inv;
                    *reinterpret_cast<f32x4_t*>(slot + r16 * D + 16 * v + 4 * j) = o;
                }
                if (j == 0) {
                    slot[G * D + r16] = m_run;
                    slot[G * D + G + r16] = lsum;
                }
            }
            if (lane == 0) {
                int* meta = reinterpret_cast<int*>(slot + G * D + 2 * G);
                meta[0] = cur.s;
                meta[1] = cur.kv;
                meta[2] = cur.pidx;
                meta[3] = cur.nparts;
            }
        }
        // the next item's table slice and query block (unconditional stores:
        // every path consumes the raw loads)
#pragma unroll
        for (int i = 0; i < TPL; ++i) tbl[lane + 64 * i] = clamp_pid(tbl_raw[i]);
#pragma unroll
        for (int i = 0; i < QPL; ++i) qs[min(lane + 64 * i, QW - 1)] = q_raw[i];
        ++nring;
        if (nring == wring || !has_next) {
            for (int i = 0; i < nring; ++i) {
                const float* sl = ring + i * SL;
                const int* meta = reinterpret_cast<const int*>(sl + G * D + 2 * G);
                const int s = meta[0], kv = meta[1], pidx = meta[2], nparts = meta[3];
                const size_t row0 = static_cast<size_t>(s) * p.num_heads + kv * G;
                if (nparts == 1) {
                    for (int idx = lane; idx < G * D; idx += 64) EL::store(p.out, row0 * D + idx, sl[idx]);
                } else {
                    for (int idx = lane; idx < G * D; idx += 64) {
                        const int h = idx / D;
                        const int d = idx - h * D;
                        p.ws_o[((row0 + h) * p.pmax + pidx) * D + d] = sl[idx];
                    }
                    if (lane < G) {
                        const size_t rec = (row0 + lane) * p.pmax + pidx;
                        p.ws_m[rec] = sl[G * D + lane];
                        p.ws_l[rec] = sl[G * D + G + lane];
                    }
                }
            }
            nring = 0;
        }
        if (!has_next) break;
        cur = nxt;
        next_item = wave_item(k + 2);
        if (next_item >= 0) nxt = item_at(p, sc, next_item);
    }
}

// ---------------------------------------------------------------------------
// MFMA kernel, even tile streams
// ---------------------------------------------------------------------------
//
// The per-tile products, softmax and two-deep load schedule of the wave-item
// kernel, with the work split evenly instead of dealt item by item. The
// batch's (sequence, KV head) pairs, in order, form one stream of 16-token
// tiles; every tile costs kStreamTileCost units and every pair
// kStreamPairCost more (its switch). Wave w of W takes the tiles whose cost
// position falls in [ceil(w C / W), ceil((w + 1) C / W)), C the total: one
// contiguous run per wave, equal to within a tile, with no queue, counter or
// barrier between waves.
//
// Within a run, each partition of a pair (partition_size tokens) is reduced
// on its own (running max, sum and weighted V rows), and the partitions of
// one pair that follow each other in the run are merged by the log-sum-exp
// rule as they end, in registers: split-K records exist only where the work
// is split between waves. A run therefore holds one segment per pair it
// touches: a pair it holds whole is written to `out` directly; a pair split
// between waves w0 < ... < w1 leaves the tail record of w0 (its first part)
// and the head records of w0 + 1 .. w1 (a run starts inside at most one pair
// and ends inside at most one), which the merge kernel combines. Every wave
// also states which pair its tail record belongs to and how many later waves
// continue it (none if it has no tail record), so that the merge runs one
// workgroup per wave. Results
// wait in an LDS ring and are stored when it is full or the run ends: a
// store between the streaming loads holds back the loads issued after it
// (measured on MI355X: storing each result as soon as it is known, by the
// reducing wave or by a fifth wave of the workgroup, cost 25-35 % more time
// on the long-context batch). Empty sequences count as one tile without
// loads and give zero rows.

constexpr int kStreamTileCost = 4;
constexpr int kStreamPairCost = 3;

// Result-ring slot of the stream kernel (floats): o[G][D] | m[G] | l[G] |
// s, kv, kind, n (as ints, padded to 16 bytes).
__host__ __device__ constexpr int stream_slot_floats(int g, int d) { return ((g * d + 2 * g + 4) + 3) & ~3; }

// Kinds of a segment's result.
enum : int { kSegDirect = 0, kSegTail = 1, kSegHead = 2 };

// LDS ints of the stream schedule: lens[S] | cs[S + 1] | wave_tot[kWaves]
__host__ __device__ constexpr size_t stream_sched_ints(int num_seqs) {
    return static_cast<size_t>((num_seqs + 3) & ~3) + static_cast<size_t>((num_seqs + 4) & ~3) + kWaves;
}

// Tiles of a sequence of L tokens in the stream (an empty one counts one).
__device__ __forceinline__ int stream_ntiles(int L) { return L > 0 ? (L + 15) >> 4 : 1; }

// lens[s] = clamped context length, cs[s] = cost of the pairs of sequences
// before s (cs[S] = C). Every thread of the workgroup takes part.
__device__ void build_stream_schedule(const DecodeParams& p, int* lens, int* cs, int* wave_tot) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int S = p.num_seqs;
    if (tid == 0) cs[0] = 0;
    int carry = 0;
    for (int base = 0; base < S; base += kThreads) {
        const int i = base + tid;
        int x = 0;
        if (i < S) {
            const int L = clamp_ctx(p.context_lens[i], p);
            lens[i] = L;
            x = p.num_kv_heads * (kStreamTileCost * stream_ntiles(L) + kStreamPairCost);
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (lane == 63) wave_tot[wave] = x;
        __syncthreads();
        int add = carry;
        for (int w = 0; w < wave; ++w) add += wave_tot[w];
        if (i < S) cs[i + 1] = x + add;
        carry += wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
        __syncthreads();
    }
}

// A run's position: pair (s, kv), tile t of the pair; s == num_seqs: none.
struct StreamCursor {
    int s, kv, t;
};

// One piece: a maximal stretch of a wave's run inside one partition of one
// pair, tokens [t0, t1). seg_start: the piece opens the run's segment of its
// pair (the run's first piece, or the pair's first tile); pair_start: that
// segment begins at the pair's first tile; seg_end: the piece closes the
// segment (the pair's last tile, or the end of the run); wspan: for a piece
// at the pair's first tile, the number of later waves the pair reaches.
struct Piece {
    int s, kv, t0, t1, b0, nblk;
    int seg_start, pair_start, seg_end, wspan;
};

struct StreamRun {
    long long lo, hi;  // cost positions [lo, hi) of this wave's run
    long long total;   // C
    int w, weff;       // this wave, waves with a run
};

__device__ __forceinline__ long long stream_pos(const DecodeParams& p, const int* lens, const int* cs,
                                                const StreamCursor& c) {
    const int pc = kStreamTileCost * stream_ntiles(lens[c.s]) + kStreamPairCost;
    return static_cast<long long>(cs[c.s]) + static_cast<long long>(c.kv) * pc + kStreamPairCost +
           static_cast<long long>(kStreamTileCost) * c.t;
}

// The first tile whose position is at least x (x < C).
__device__ __forceinline__ StreamCursor stream_seek(const DecodeParams& p, const int* lens, const int* cs,
                                                    long long x) {
    int lo = 0, hi = p.num_seqs;  // cs[lo] <= x < cs[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cs[mid] <= x) lo = mid; else hi = mid;
    }
    StreamCursor c;
    c.s = lo;
    const int n = stream_ntiles(lens[lo]);
    const int pc = kStreamTileCost * n + kStreamPairCost;
    const long long r = x - cs[lo];
    c.kv = static_cast<int>(r / pc);
    const int o = static_cast<int>(r - static_cast<long long>(c.kv) * pc);
    c.t = o <= kStreamPairCost ? 0 : (o - kStreamPairCost + kStreamTileCost - 1) / kStreamTileCost;
    if (c.t >= n) {
        c.t = 0;
        if (++c.kv == p.num_kv_heads) {
            c.kv = 0;
            ++c.s;
        }
    }
    return c;
}

// The piece at cursor c (which this wave owns; `first`: the run's first
// piece), and the cursor of the next one (s = num_seqs when the run ends).
__device__ __forceinline__ Piece stream_piece(const DecodeParams& p, const int* lens, const int* cs,
                                              const StreamRun& run, const StreamCursor& c, bool first,
                                              StreamCursor& next) {
    const int L = lens[c.s];
    const int n = stream_ntiles(L);
    const int pc = kStreamTileCost * n + kStreamPairCost;
    const long long base = static_cast<long long>(cs[c.s]) + static_cast<long long>(c.kv) * pc;
    const int ptiles = p.part >> 4;
    const int pidx = c.t / ptiles;
    const int last_owned = static_cast<int>((run.hi - 1 - base - kStreamPairCost) / kStreamTileCost);
    const int te = min(min(n, (pidx + 1) * ptiles), last_owned + 1);
    Piece x;
    x.s = c.s;
    x.kv = c.kv;
    x.t0 = c.t * 16;
    x.t1 = min(L, te * 16);
    x.b0 = x.t0 >> p.log2_bs;
    x.nblk = x.t1 > x.t0 ? ((x.t1 - 1) >> p.log2_bs) - x.b0 + 1 : 0;
    x.seg_start = first || c.t == 0;
    x.seg_end = te >= n || te > last_owned;
    x.pair_start = c.t == 0;  // (meaningful on the segment's first piece)
    x.wspan = 0;
    if (c.t == 0) {
        const long long last = base + kStreamPairCost + static_cast<long long>(kStreamTileCost) * (n - 1);
        x.wspan = static_cast<int>(last * run.weff / run.total) - run.w;
    }
    next = c;
    next.t = te;
    if (next.t >= n) {
        next.t = 0;
        if (++next.kv == p.num_kv_heads) {
            next.kv = 0;
            ++next.s;
        }
    }
    if (next.s < p.num_seqs && stream_pos(p, lens, cs, next) >= run.hi) next.s = p.num_seqs;
    return x;
}

// Store one ring slot: a head or tail record of wave `w`, or a pair's rows of
// `out`; a segment that began at its pair's first tile also stores the pair's
// (first wave, later waves). Every lane first reads its 16-byte chunks of the
// rows from LDS, then stores them.
template <int DT, int D, int G>
__device__ __forceinline__ void stream_write_slot(const DecodeParams& p, const float* sl, int w, int lane) {
    using EL = Elem<DT>;
    constexpr int E = 2;
    constexpr int OC = G * D / 4;          // 16-byte chunks of the rows
    constexpr int OCL = (OC + 63) / 64;    // per lane
    const int* meta = reinterpret_cast<const int*>(sl + G * D + 2 * G);
    const int s = meta[0], kv = meta[1], kind = meta[2], span = meta[3];
    f32x4_t ch[OCL];
#pragma unroll
    for (int c = 0; c < OCL; ++c) ch[c] = *reinterpret_cast<const f32x4_t*>(sl + 4 * min(lane + 64 * c, OC - 1));
    const float mv = sl[G * D + (lane < G ? lane : 0)];
    const float lv = sl[G * D + G + (lane < G ? lane : 0)];
    if (kind == kSegDirect) {
        const size_t row0 = static_cast<size_t>(s) * p.num_heads + kv * G;  // first query head row
#pragma unroll
        for (int c = 0; c < OCL; ++c) {
            if (lane + 64 * c < OC) {
                u32x2 v;
                v.x = static_cast<uint32_t>(EL::round(ch[c][0])) | (static_cast<uint32_t>(EL::round(ch[c][1])) << 16);
                v.y = static_cast<uint32_t>(EL::round(ch[c][2])) | (static_cast<uint32_t>(EL::round(ch[c][3])) << 16);
                *reinterpret_cast<u32x2*>(static_cast<char*>(p.out) + (row0 * D + 4 * (lane + 64 * c)) * E) = v;
            }
        }
    } else {
        const size_t x0 = (static_cast<size_t>(kind == kSegTail ? 0 : kMaxStreamWaves) + w) * G;
#pragma unroll
        for (int c = 0; c < OCL; ++c)
            if (lane + 64 * c < OC) *reinterpret_cast<f32x4_t*>(p.ws_xo + x0 * D + 4 * (lane + 64 * c)) = ch[c];
        if (lane < G) {
            p.ws_xm[x0 + lane] = mv;
            p.ws_xl[x0 + lane] = lv;
        }
    }
    if (kind == kSegTail && lane == 0)
        *reinterpret_cast<int4*>(p.ws_meta + 4 * static_cast<size_t>(w)) = make_int4(s, kv, span, 0);
}

// The merge's list has kMaxStreamWaves entries: wave w of a grid of W waves
// clears entries w + W, w + 2W, ... (no wave of this launch has them) and,
// unless it holds a tail record (which writes entry w), entry w too.
__device__ __forceinline__ void stream_list_end(const DecodeParams& p, int w, bool own, int lane) {
    const int W = gridDim.x * kWaves;
    for (int x = w + W * (lane + (own ? 0 : 1)); x < kMaxStreamWaves; x += W * 64)
        *reinterpret_cast<int4*>(p.ws_meta + 4 * static_cast<size_t>(x)) = make_int4(0, 0, 0, 0);
}

// KEEP: K/V tiles are read with ordinary loads instead of nontemporal ones,
// so that the L2 keeps them for the other sequences that list the same
// blocks (a caller's hint that the batch shares blocks; blocks of 16 or more
// tokens). Streaming loads are faster when nothing is shared.
template <int DT, int D, int G, bool BIGB, bool KEEP = false>
__global__ __launch_bounds__(kThreads) void pa_decode_stream(DecodeParams p) {
    static_assert(DT == PA_BF16 || DT == PA_F16, "MFMA path is for 16-bit elements");
    static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "group size");
    constexpr int E = 2;
    constexpr int NK = D / 32;
    constexpr int NV = D / 16;
    constexpr int QW = G * D / 2;
    constexpr int QWP = wave_q_words(G, D);
    constexpr int QPL = (QW + 63) / 64;
    constexpr int TPL = kWaveSlice / 64;
    constexpr float kLazy = 8.f;
    constexpr int SL = stream_slot_floats(G, D);

    // LDS: schedule | tbl[kWaves][kWaveSlice] | qs[kWaves][QWP] | ring[kWaves][wring]
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int* lens = reinterpret_cast<int*>(smem);
    int* cs = lens + ((p.num_seqs + 3) & ~3);
    int* wave_tot = cs + ((p.num_seqs + 4) & ~3);
    int* tbl_all = reinterpret_cast<int*>(smem) + stream_sched_ints(p.num_seqs);
    uint32_t* qs_all = reinterpret_cast<uint32_t*>(tbl_all + kWaves * kWaveSlice);
    float* ring_all = reinterpret_cast<float*>(qs_all + kWaves * QWP);
    const int wring = p.ring_slots / kWaves;
    int* tbl = tbl_all + wave * kWaveSlice;
    uint32_t* qs = qs_all + wave * QWP;
    float* ring = ring_all + wave * wring * SL;
    int nring = 0;

    const int r16 = lane & 15;
    const int j = lane >> 4;
    const int bs = 1 << p.log2_bs;
    const int hkv = p.num_kv_heads;
    const size_t blk_el = static_cast<size_t>(bs) * D;
    const char* kbase = static_cast<const char*>(p.k_cache);
    const char* vbase = static_cast<const char*>(p.v_cache);
    const uint32_t* qwords = static_cast<const uint32_t*>(p.q);

    if (p.num_seqs == 0) return;
    build_stream_schedule(p, lens, cs, wave_tot);  // the last barrier of the kernel
    StreamRun run;
    run.total = cs[p.num_seqs];
    // every run spans at least 8 cost units, so that each owns a tile
    const long long wmax = static_cast<long long>(gridDim.x) * kWaves;
    run.weff = static_cast<int>(min(wmax, max(1ll, run.total / 8)));
    run.w = xcd_run_id<kWaves>(run.weff, wave);  // (a bijection onto 0 .. gridDim.x * kWaves - 1)
    if (run.w >= run.weff) {
        stream_list_end(p, run.w, true, lane);
        return;
    }
    run.lo = (static_cast<long long>(run.w) * run.total + run.weff - 1) / run.weff;
    run.hi = (static_cast<long long>(run.w + 1) * run.total + run.weff - 1) / run.weff;

    struct Buf {
        u32x4 k[NK];
        u32x2 v[NV];
    };
    auto ntiles_of = [](const Piece& x) { return x.t1 > x.t0 ? (x.t1 - x.t0 + 15) >> 4 : 0; };
    auto last4_of = [](const Piece& x) { return x.t1 > x.t0 ? ((x.t1 - 1) >> 2) << 2 : 0; };
    auto q_word0 = [&](const Piece& x) {
        return (static_cast<size_t>(x.s) * p.num_heads + x.kv * G) * (D / 2);
    };
    auto clamp_pid = [&](int pid) { return pid < 0 ? 0 : (pid >= p.num_blocks ? p.num_blocks - 1 : pid); };

    // K/V loads of one 16-token tile. Blocks of 16 tokens or more: the tile
    // lies in one block and one 16-token V tile, so the bases are scalar.
    // Smaller blocks: a lane's K row (key tt0 + r16) and its four V keys
    // (tt0 + 4j ..) each lie in one block, whose ids pk and pv it holds.
    auto load_with = [&](const Piece& x, int tile, int pk, int pv, Buf& b) {
        const int tt0 = x.t0 + 16 * tile;
        const int krow = min(tt0 + r16, x.t1 - 1);
        const int vtok = min(tt0 + 4 * j, last4_of(x));
        if constexpr (BIGB) {
            const int pid = __builtin_amdgcn_readfirstlane(pk);
            const size_t tile_el = (static_cast<size_t>(pid) * hkv + x.kv) * blk_el;
            const char* kt = kbase + tile_el * E;
            const char* vtp = vbase + (tile_el + static_cast<size_t>((tt0 & (bs - 1)) >> 4) * D * 16) * E;
            const uint32_t ko = static_cast<uint32_t>(((krow & (bs - 1)) * D + 8 * j) * E);
            const uint32_t vo = static_cast<uint32_t>(((vtok & 15) + 16 * r16) * E);
            if constexpr (KEEP) {
#pragma unroll
                for (int c = 0; c < NK; ++c) b.k[c] = *reinterpret_cast<const u32x4*>(kt + ko + 64 * c);
#pragma unroll
                for (int v = 0; v < NV; ++v) b.v[v] = *reinterpret_cast<const u32x2*>(vtp + vo + 512 * v);
            } else {
#pragma unroll
                for (int c = 0; c < NK; ++c) b.k[c] = nt_load<u32x4>(kt, ko + 64 * c);
#pragma unroll
                for (int v = 0; v < NV; ++v) b.v[v] = nt_load<u32x2>(vtp, vo + 512 * v);
            }
        } else {
            const int vt = 1 << p.log2_vt;
            const size_t kel = (static_cast<size_t>(pk) * hkv + x.kv) * blk_el +
                               static_cast<size_t>(krow & (bs - 1)) * D + 8 * j;
#pragma unroll
            for (int c = 0; c < NK; ++c) b.k[c] = nt_load<u32x4>(kbase, (kel + 32 * c) * E);
            const int voff = vtok & (bs - 1);
            const size_t vel = (static_cast<size_t>(pv) * hkv + x.kv) * blk_el +
                               static_cast<size_t>(voff >> p.log2_vt) * D * vt + (voff & (vt - 1)) +
                               static_cast<size_t>(r16) * vt;
#pragma unroll
            for (int v = 0; v < NV; ++v)
                b.v[v] = nt_load<u32x2>(vbase, (vel + static_cast<size_t>(16 * v) * vt) * E);
        }
    };
    auto tile_blocks = [&](const Piece& x, const int* tb, int tile, int& pk, int& pv) {
        const int tt0 = x.t0 + 16 * tile;
        if constexpr (BIGB) {
            pk = pv = tb[(min(tt0, x.t1 - 1) >> p.log2_bs) - x.b0];
        } else {
            pk = tb[(min(tt0 + r16, x.t1 - 1) >> p.log2_bs) - x.b0];
            pv = tb[(min(tt0 + 4 * j, last4_of(x)) >> p.log2_bs) - x.b0];
        }
    };
    auto stage_slice = [&](const Piece& x, int* tb) {
        const int* trow = p.block_tables + static_cast<size_t>(x.s) * p.max_blocks + x.b0;
#pragma unroll
        for (int i = 0; i < TPL; ++i)
            if (lane + 64 * i < x.nblk) tb[lane + 64 * i] = clamp_pid(trow[lane + 64 * i]);
    };

    // prologue: the first piece's table slice and query block, its first tile
    const StreamCursor at = stream_seek(p, lens, cs, run.lo);
    if (at.s >= p.num_seqs) {  // (a run of 8 or more units always holds a tile)
        stream_list_end(p, run.w, true, lane);
        return;
    }
    StreamCursor after;
    Piece cur = stream_piece(p, lens, cs, run, at, true, after);
    bool has_next = after.s < p.num_seqs;
    Piece nxt = cur;
    if (has_next) {
        const StreamCursor c2 = after;
        nxt = stream_piece(p, lens, cs, run, c2, false, after);
    }
    stage_slice(cur, tbl);
    for (int w = lane; w < QW; w += 64) qs[w] = qwords[q_word0(cur) + w];
    Buf A, B;
    {
        int pk = 0, pv = 0;
        if (ntiles_of(cur) > 0) tile_blocks(cur, tbl, 0, pk, pv);
        load_with(cur, 0, pk, pv, A);
    }

    // the segment's running result: the merged partitions so far (max in
    // log2 units, this lane's share of the sum, unnormalised V rows)
    f32x4_t seg_o[NV];
    float seg_m = -INFINITY, seg_l = 0.f;
    int seg_kind = kSegDirect, seg_span = 0;

    while (true) {
        const bool next_tile = has_next && ntiles_of(nxt) > 0;
        // raw loads of the next piece's metadata, consumed at the end
        const int* trow = p.block_tables + static_cast<size_t>(nxt.s) * p.max_blocks + nxt.b0;
        const int* safe = p.context_lens;
        int pk_raw, pv_raw;
        if constexpr (BIGB) {
            pk_raw = *(next_tile ? trow : safe);
            pv_raw = pk_raw;
        } else {
            pk_raw = *(next_tile ? trow + ((min(nxt.t0 + r16, nxt.t1 - 1) >> p.log2_bs) - nxt.b0) : safe);
            pv_raw = *(next_tile ? trow + ((min(nxt.t0 + 4 * j, last4_of(nxt)) >> p.log2_bs) - nxt.b0) : safe);
        }
        int tbl_raw[TPL];
#pragma unroll
        for (int i = 0; i < TPL; ++i)
            tbl_raw[i] = *(has_next && lane + 64 * i < nxt.nblk ? trow + lane + 64 * i : safe);
        uint32_t q_raw[QPL];
#pragma unroll
        for (int i = 0; i < QPL; ++i) q_raw[i] = qwords[q_word0(nxt) + min(lane + 64 * i, QW - 1)];

        if (cur.seg_start) {
#pragma unroll
            for (int v = 0; v < NV; ++v) seg_o[v] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            seg_m = -INFINITY;
            seg_l = 0.f;
            seg_kind = !cur.pair_start ? kSegHead : kSegDirect;
            seg_span = cur.wspan;
        }
        u32x4 qf[NK];
        {
            const uint32_t* qrow = qs + (r16 % G) * (D / 2);
#pragma unroll
            for (int c = 0; c < NK; ++c) qf[c] = *reinterpret_cast<const u32x4*>(qrow + 16 * c + 4 * j);
        }
        f32x4_t acc[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[v] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        float m_run = -INFINITY, lsum = 0.f;
        const int t1 = cur.t1;
        const int ntiles = ntiles_of(cur);

        auto compute_tile = [&](int tile, const Buf& b) {
            const int tt0 = cur.t0 + 16 * tile;
            f32x4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NK; ++c) st = mfma_qk<DT>(b.k[c], qf[c], st);
            float x[4];
            bool valid[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                valid[r] = tt0 + 4 * j + r < t1;
                x[r] = valid[r] ? st[r] * p.scale_log2 : -INFINITY;
            }
            float tmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
            const bool need = tmax > m_run + kLazy;
            if (__any(need)) {
                const float mn = need ? tmax : m_run;
                const float alpha = fast_exp2(m_run - mn);
#pragma unroll
                for (int v = 0; v < NV; ++v) acc[v] *= alpha;
                lsum *= alpha;
                m_run = mn;
            }
            float pr[4];
            u32x2 pb;
            pb.x = pack2<DT>(fast_exp2(x[0] - m_run), fast_exp2(x[1] - m_run), pr[0], pr[1]);
            pb.y = pack2<DT>(fast_exp2(x[2] - m_run), fast_exp2(x[3] - m_run), pr[2], pr[3]);
            lsum += (pr[0] + pr[1]) + (pr[2] + pr[3]);
            const uint32_t mask0 = (valid[0] ? 0xffffu : 0u) | (valid[1] ? 0xffff0000u : 0u);
            const uint32_t mask1 = (valid[2] ? 0xffffu : 0u) | (valid[3] ? 0xffff0000u : 0u);
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                u32x2 a = b.v[v];
                a.x &= mask0;
                a.y &= mask1;
                acc[v] = mfma_pv<DT>(a, pb, acc[v]);
            }
        };
        auto load_tile = [&](int tile, Buf& b) {
            int pk, pv;
            tile_blocks(cur, tbl, tile, pk, pv);
            load_with(cur, tile, pk, pv, b);
        };
        auto load_next = [&](Buf& b) {
            int pk = pk_raw, pv = pv_raw;
            asm volatile("" : "+v"(pk), "+v"(pv));
            if (next_tile) load_with(nxt, 0, clamp_pid(pk), clamp_pid(pv), b);
            else load_with(cur, 0, 0, 0, b);
        };
        // the piece's tiles, two deep
        int t = 0;
        if (ntiles > 0) {
            for (int i = 0; i < ((ntiles - 1) >> 1); ++i) {
                load_tile(t + 1, B);
                __builtin_amdgcn_sched_barrier(0);
                compute_tile(t, A);
                __builtin_amdgcn_sched_barrier(0);
                load_tile(t + 2, A);
                __builtin_amdgcn_sched_barrier(0);
                compute_tile(t + 1, B);
                t += 2;
            }
            if (ntiles & 1) {
                compute_tile(t, A);
            } else {
                load_tile(t + 1, B);
                __builtin_amdgcn_sched_barrier(0);
                compute_tile(t, A);
                compute_tile(t + 1, B);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        load_next(A);
        asm volatile("" ::"v"(pk_raw), "v"(pv_raw));

        // the partition (piece) joins the segment by the log-sum-exp rule:
        // both sides are rescaled to the larger max (m_run is the same on
        // the four lanes of a column, and sums stay per lane)
        {
            const float mn = fmaxf(seg_m, m_run);
            const float mu = mn == -INFINITY ? 0.f : mn;
            const float a = fast_exp2(seg_m - mu), b = fast_exp2(m_run - mu);
#pragma unroll
            for (int v = 0; v < NV; ++v) seg_o[v] = seg_o[v] * a + acc[v] * b;
            seg_l = seg_l * a + lsum * b;
            seg_m = mn;
        }

        if (cur.seg_end) {
            // seg_o[v][r] = O^T[d = 16v + 4j + r][head column r16]; the sum
            // over the column's four lanes
            float l = seg_l;
            l += __shfl_xor(l, 16);
            l += __shfl_xor(l, 32);
            // a segment that began at the pair's first tile and stops short of
            // its last is the pair's tail record
            const bool pair_done = cur.t1 >= lens[cur.s];
            const int kind = seg_kind == kSegHead ? kSegHead : (pair_done ? kSegDirect : kSegTail);
            if (!has_next) stream_list_end(p, run.w, kind != kSegTail, lane);
            float* slot = ring + nring * SL;
            if (r16 < G) {
                const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
                for (int v = 0; v < NV; ++v)
                    *reinterpret_cast<f32x4_t*>(slot + r16 * D + 16 * v + 4 * j) = seg_o[v] * inv;
                if (j == 0) {
                    slot[G * D + r16] = seg_m;
                    slot[G * D + G + r16] = l;
                }
            }
            if (lane == 0) {
                int* meta = reinterpret_cast<int*>(slot + G * D + 2 * G);
                meta[0] = cur.s;
                meta[1] = cur.kv;
                meta[2] = kind;
                meta[3] = seg_span;
            }
            ++nring;
        }
        // the next piece's table slice and query block (unconditional stores:
        // every path consumes the raw loads)
#pragma unroll
        for (int i = 0; i < TPL; ++i) tbl[lane + 64 * i] = clamp_pid(tbl_raw[i]);
#pragma unroll
        for (int i = 0; i < QPL; ++i) qs[min(lane + 64 * i, QW - 1)] = q_raw[i];
        if (nring == wring || !has_next) {
            for (int i = 0; i < nring; ++i) stream_write_slot<DT, D, G>(p, ring + i * SL, run.w, lane);
            nring = 0;
        }
        if (!has_next) break;
        cur = nxt;
        has_next = after.s < p.num_seqs;
        if (has_next) {
            const StreamCursor c2 = after;
            nxt = stream_piece(p, lens, cs, run, c2, false, after);
        }
    }
}

// Merge of the stream kernel's split pairs: one wave per (w, h) takes query
// head h of the pair whose tail record wave w holds, if any,
// and combines that record with the head records of the n waves that
// continue the pair by the log-sum-exp rule. All loads of a chunk of CH
// records (CH the smallest of 2, 4, 8, 16, 32 that holds them, chunks of 32
// beyond) are issued together: lane i reads record i's max and sum, every
// lane its head_dim elements of each record; the records are then added in
// record order. Pairs one wave held whole were written directly.
template <int DT, int D, int CH>
__device__ __forceinline__ void merge_stream_pair(const DecodeParams& p, int w0, int h, int n, size_t row,
                                                  int lane) {
    using EL = Elem<DT>;
    constexpr int PER = D / 64;
    const int G = p.group;
    // record i: i = 0 the tail of w0, i >= 1 the head of w0 + i
    auto rec = [&](int i) -> size_t {
        return (static_cast<size_t>(i == 0 ? 0 : kMaxStreamWaves) + w0 + i) * G + h;
    };
    float M = -INFINITY;
    for (int i = lane; i <= n; i += 64) M = fmaxf(M, p.ws_xm[rec(i)]);
    M = wave_max(M);
    const float Mu = M == -INFINITY ? 0.f : M;
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    float wsum = 0.f;  // this lane's records' weights
    for (int base = 0; base <= n; base += CH) {
        const int cnt = min(CH, n + 1 - base);
        float o[CH][PER];
#pragma unroll
        for (int k2 = 0; k2 < CH; ++k2) {
            const float* src = p.ws_xo + rec(base + min(k2, cnt - 1)) * D;
#pragma unroll
            for (int e = 0; e < PER; ++e) o[k2][e] = src[lane + 64 * e];
        }
        float wi = 0.f;
        if (lane < cnt) {
            const size_t r = rec(base + lane);
            wi = p.ws_xl[r] * fast_exp2(p.ws_xm[r] - Mu);
        }
        wsum += wi;
#pragma unroll
        for (int k2 = 0; k2 < CH; ++k2) {
            const float wk = k2 < cnt ? __shfl(wi, k2) : 0.f;
#pragma unroll
            for (int e = 0; e < PER; ++e) acc[e] = fmaf(wk, o[k2][e], acc[e]);
        }
    }
    const float W = group_sum<64>(wsum);
    const float inv = W > 0.f ? 1.f / W : 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) EL::store(p.out, row * D + lane + 64 * e, acc[e] * inv);
}

template <int DT, int D>
__global__ __launch_bounds__(256) void pa_merge_stream(DecodeParams p) {
    // four (wave, head) tasks per workgroup: task i is head i % G of the
    // tail record of wave i / G (most have none: few workgroups to dispatch)
    const int G = p.group;
    const int task = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int w0 = task / G;
    const int h = task - w0 * G;
    const int lane = threadIdx.x & 63;
    const int4 t = *reinterpret_cast<const int4*>(p.ws_meta + 4 * static_cast<size_t>(w0));
    const int s = t.x, kv = t.y, n = t.z;
    if (n <= 0) return;
    const size_t row = static_cast<size_t>(s) * p.num_heads + kv * G + h;
    if (n < 2) merge_stream_pair<DT, D, 2>(p, w0, h, n, row, lane);
    else if (n < 4) merge_stream_pair<DT, D, 4>(p, w0, h, n, row, lane);
    else if (n < 8) merge_stream_pair<DT, D, 8>(p, w0, h, n, row, lane);
    else if (n < 16) merge_stream_pair<DT, D, 16>(p, w0, h, n, row, lane);
    else merge_stream_pair<DT, D, 32>(p, w0, h, n, row, lane);
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

// The same merge for batches with many partitions per sequence: one wave
// reading one partition record after another keeps too few loads in flight
// (on the 131k-token batch at 512-token partitions, 256 records per
// sequence, it moved 1.8 TB/s). Here four waves share a (sequence, query
// head): each takes every fourth record, eight at a time, and the four
// partial sums are added in a fixed order through LDS.
constexpr int kMergeWideWaves = 4;
constexpr int kMergeWideMinParts = 9;  // the single-wave merge up to 8 records per sequence

template <int DT, int D>
__global__ __launch_bounds__(64 * kMergeWideWaves) void pa_merge_wide(DecodeParams p) {
    using EL = Elem<DT>;
    constexpr int PER = D / 64;
    constexpr int NW = kMergeWideWaves;
    static_assert(NW == 4, "the combines below add four partial sums");
    __shared__ float red_m[NW];
    __shared__ float red_w[NW];
    __shared__ float red_o[NW][D];
    const int hq = blockIdx.x;
    const int s = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int L = clamp_ctx(p.context_lens[s], p);
    const int P = L > 0 ? ceil_div(L, p.part) : 1;
    if (P == 1) return;
    const size_t rec0 = (static_cast<size_t>(s) * p.num_heads + hq) * p.pmax;
    const float* mrow = p.ws_m + rec0;
    const float* lrow = p.ws_l + rec0;
    float M = -INFINITY;
    for (int i = tid; i < P; i += 64 * NW) M = fmaxf(M, mrow[i]);
    M = wave_max(M);
    if (lane == 0) red_m[wave] = M;
    __syncthreads();
    M = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
    const float Mu = M == -INFINITY ? 0.f : M;
    float acc[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = 0.f;
    float W = 0.f;
    const float* o = p.ws_o + rec0 * D;
#pragma unroll 8
    for (int i = wave; i < P; i += NW) {
        const float w = lrow[i] * fast_exp2(mrow[i] - Mu);
        W += w;
#pragma unroll
        for (int k = 0; k < PER; ++k) acc[k] = fmaf(w, o[static_cast<size_t>(i) * D + lane + 64 * k], acc[k]);
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) red_o[wave][lane + 64 * k] = acc[k];
    if (lane == 0) red_w[wave] = W;
    __syncthreads();
    if (wave != 0) return;
    const float Wt = (red_w[0] + red_w[1]) + (red_w[2] + red_w[3]);
    const float inv = Wt > 0.f ? 1.f / Wt : 0.f;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int d = lane + 64 * k;
        const float a = (red_o[0][d] + red_o[1][d]) + (red_o[2][d] + red_o[3][d]);
        EL::store(p.out, (static_cast<size_t>(s) * p.num_heads + hq) * D + d, a * inv);
    }
}

// ---------------------------------------------------------------------------
// Host-side launch plan and dispatch
// ---------------------------------------------------------------------------

namespace {

// A workgroup's LDS is allocated in whole granules, so every fit below is
// computed on rounded sizes (1 KB is at least the hardware's unit).
constexpr size_t kLdsGranule = 1024;
constexpr int kMaxRingSlots = 32;

// Workgroups per compute unit of the MFMA kernels. Their scattered 4 KB tile
// reads run faster from fewer, deeper streams: measured on MI355X, one
// workgroup per CU is as fast as two or three on the batch-256 grouped-query
// decode and 10 % faster on the long-context one.
constexpr int kMfmaWgPerCu = 1;

constexpr size_t lds_alloc(size_t bytes) { return (bytes + kLdsGranule - 1) / kLdsGranule * kLdsGranule; }

size_t ring_slot_bytes(int d, int g, bool stream) {
    return static_cast<size_t>(stream ? stream_slot_floats(g, d) : ring_slot_floats(g, d)) * sizeof(float);
}

// Ring slots that fit next to `used` bytes of LDS when `resident` workgroups
// share a compute unit of `lds_per_cu` bytes; at least one if a single
// workgroup of used + one slot fits in `lds_per_wg`, else 0.
int ring_slots_for(size_t used, size_t slot, int resident, size_t lds_per_cu, size_t lds_per_wg) {
    if (lds_alloc(used + slot) > lds_per_wg) return 0;
    const size_t share = std::min(lds_per_wg, lds_per_cu / static_cast<size_t>(resident < 1 ? 1 : resident));
    int n = 1;
    while (n < kMaxRingSlots && lds_alloc(used + static_cast<size_t>(n + 1) * slot) <= share) ++n;
    return n;
}

// Dynamic LDS of each kernel besides its result ring.
size_t decode_smem_valu(int num_seqs, int d, int g) {
    // schedule | table slice | wave partials
    return (sched_ints(num_seqs) + kMaxTableSlice) * sizeof(int) +
           static_cast<size_t>(kWaves) * g * red_stride(d) * sizeof(float);
}

size_t decode_smem_mfma(int num_seqs, int d, int g) {
    // schedule | two table slices | two query blocks | one or two sets of wave partials
    const size_t qw = ((static_cast<size_t>(g) * d / 2 + 3) & ~static_cast<size_t>(3));
    return (sched_ints(num_seqs) + 2 * kMaxTableSlice) * sizeof(int) +
           2 * qw * sizeof(uint32_t) +
           (mfma_red_double(g, d) ? 2 : 1) * static_cast<size_t>(kWaves) * g * red_stride(d) * sizeof(float);
}

size_t decode_smem_stream(int num_seqs, int d, int g) {
    // schedule | per wave: a table slice and a query block
    return (stream_sched_ints(num_seqs) + static_cast<size_t>(kWaves) * kWaveSlice) * sizeof(int) +
           static_cast<size_t>(kWaves) * wave_q_words(g, d) * sizeof(uint32_t);
}

size_t decode_smem_mfma_wave(int num_seqs, int d, int g) {
    // schedule | per wave: a table slice and a query block
    return (sched_ints(num_seqs) + static_cast<size_t>(kWaves) * kWaveSlice) * sizeof(int) +
           static_cast<size_t>(kWaves) * wave_q_words(g, d) * sizeof(uint32_t);
}

// Workgroups of kThreads threads that one compute unit can hold for `kern`
// with `smem` bytes of dynamic LDS, from the runtime's occupancy query, made
// once per (device, kernel, smem) and then served from a cache.
hipError_t residency(const void* kern, int dev, size_t smem, int threads, int* out) {
    static std::mutex mu;
    static std::map<std::tuple<int, const void*, size_t, int>, int> cache;
    const auto key = std::make_tuple(dev, kern, smem, threads);
    {
        std::lock_guard<std::mutex> lock(mu);
        const auto it = cache.find(key);
        if (it != cache.end()) {
            *out = it->second;
            return hipSuccess;
        }
    }
    int n = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, threads, smem);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    cache[key] = n;
    *out = n;
    return hipSuccess;
}

// Launch a persistent kernel as planned: as many workgroups as the plan and
// the runtime's occupancy for the planned LDS allow on every compute unit.
hipError_t run_planned(void (*kern)(DecodeParams), DecodeParams p, const DecodePlan& pl, const DeviceInfo& dv,
                       hipStream_t stream) {
    const int threads = kThreads;
    int occ = 0;
    const hipError_t e = residency(reinterpret_cast<const void*>(kern), dv.id, pl.smem, threads, &occ);
    if (e != hipSuccess) return e;
    const int resident = std::min(pl.resident, occ);
    if (resident < 1) return hipErrorInvalidConfiguration;
    p.ring_slots = pl.ring_slots;
    const long long upper = pl.kernel == PA_DECODE_MFMA_STREAM
                                ? kMaxStreamWaves / kWaves
                                : static_cast<long long>(p.num_seqs) * p.num_kv_heads * p.pmax;
    long long grid = static_cast<long long>(dv.cus) * resident;
    if (grid > upper) grid = upper;
    if (grid < 1) grid = 1;
    return launch_kernel(kern, dim3(static_cast<unsigned>(grid)), dim3(threads), pl.smem, stream, p);
}

template <int DT, int D, int G>
hipError_t launch_valu(const DecodeParams& p, const DeviceInfo& dv, hipStream_t stream) {
    constexpr int step = ValuGeom<Elem<DT>::E, D>::STEP;
    void (*kern)(DecodeParams) =
        (1 << p.log2_bs) >= step ? pa_decode_valu<DT, D, G, true> : pa_decode_valu<DT, D, G, false>;
    int occ = 0;  // as many as the registers allow
    hipError_t e = residency(reinterpret_cast<const void*>(kern), dv.id, 0, kThreads, &occ);
    if (e != hipSuccess) return e;
    DecodePlan pl;
    if (plan_decode(static_cast<pa_dtype_t>(DT), D, G, p.num_seqs, p.part >> p.log2_bs, false, dv.lds_per_cu,
                    dv.lds_per_wg, occ, &pl) != PA_OK)
        return hipErrorInvalidConfiguration;
    return run_planned(kern, p, pl, dv, stream);
}

template <int DT, int D, int G>
hipError_t launch_mfma(const DecodeParams& p, const DeviceInfo& dv, hipStream_t stream) {
    DecodePlan pl;
    if (plan_decode(static_cast<pa_dtype_t>(DT), D, G, p.num_seqs, p.part >> p.log2_bs, p.stream != 0,
                    dv.lds_per_cu, dv.lds_per_wg, kMfmaWgPerCu, &pl) != PA_OK)
        return hipErrorInvalidConfiguration;
    const bool big = (1 << p.log2_bs) >= 16;
    void (*kern)(DecodeParams);
    if (pl.kernel == PA_DECODE_MFMA_STREAM)
        kern = !big ? pa_decode_stream<DT, D, G, false>
                    : (p.keep_tiles ? pa_decode_stream<DT, D, G, true, true> : pa_decode_stream<DT, D, G, true>);
    else if (pl.kernel == PA_DECODE_MFMA_WAVE)
        kern = big ? pa_decode_mfma_wave<DT, D, G, true> : pa_decode_mfma_wave<DT, D, G, false>;
    else
        kern = big ? pa_decode_mfma<DT, D, G, true> : pa_decode_mfma<DT, D, G, false>;
    return run_planned(kern, p, pl, dv, stream);
}

// One query head per KV head on the stream split (16-bit elements): the MFMA
// tiles then carry one distinct column, but the kernel is bound by the K/V
// stream, not by its products.
template <int DT, int D, int G>
hipError_t launch_stream_only(const DecodeParams& p, const DeviceInfo& dv, hipStream_t stream) {
    DecodePlan pl;
    if (plan_decode(static_cast<pa_dtype_t>(DT), D, G, p.num_seqs, p.part >> p.log2_bs, true, dv.lds_per_cu,
                    dv.lds_per_wg, kMfmaWgPerCu, &pl) != PA_OK || pl.kernel != PA_DECODE_MFMA_STREAM)
        return hipErrorInvalidConfiguration;
    const bool big = (1 << p.log2_bs) >= 16;
    void (*kern)(DecodeParams) = !big ? pa_decode_stream<DT, D, G, false>
                                      : (p.keep_tiles ? pa_decode_stream<DT, D, G, true, true>
                                                      : pa_decode_stream<DT, D, G, true>);
    return run_planned(kern, p, pl, dv, stream);
}

template <int DT, int D>
hipError_t launch_d(const DecodeParams& p, const DeviceInfo& dv, hipStream_t stream) {
    if constexpr (DT == PA_F32) {
        switch (p.group) {
            case 1: return launch_valu<DT, D, 1>(p, dv, stream);
            case 2: return launch_valu<DT, D, 2>(p, dv, stream);
            case 4: return launch_valu<DT, D, 4>(p, dv, stream);
            case 8: return launch_valu<DT, D, 8>(p, dv, stream);
        }
    } else {
        switch (p.group) {
            case 1: return p.stream ? launch_stream_only<DT, D, 1>(p, dv, stream) : launch_valu<DT, D, 1>(p, dv, stream);
            case 2: return launch_mfma<DT, D, 2>(p, dv, stream);
            case 4: return launch_mfma<DT, D, 4>(p, dv, stream);
            case 8: return launch_mfma<DT, D, 8>(p, dv, stream);
            case 16: return launch_mfma<DT, D, 16>(p, dv, stream);
        }
    }
    return hipErrorInvalidValue;
}

template <int DT>
hipError_t launch_dt(const DecodeParams& p, int head_dim, const DeviceInfo& dv, hipStream_t stream) {
    switch (head_dim) {
        case 64: return launch_d<DT, 64>(p, dv, stream);
        case 128: return launch_d<DT, 128>(p, dv, stream);
        case 256: return launch_d<DT, 256>(p, dv, stream);
    }
    return hipErrorInvalidValue;
}

template <int DT, int D>
hipError_t launch_merge_dd(const DecodeParams& p, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(p.num_heads), static_cast<unsigned>(p.num_seqs));
    if (p.stream)  // (kMaxStreamWaves is a multiple of 4)
        return launch_kernel(pa_merge_stream<DT, D>, dim3(kMaxStreamWaves / 4 * static_cast<unsigned>(p.group)),
                             dim3(256), 0, stream, p);
    if (p.pmax >= kMergeWideMinParts)
        return launch_kernel(pa_merge_wide<DT, D>, grid, dim3(64 * kMergeWideWaves), 0, stream, p);
    return launch_kernel(pa_merge<DT, D>, grid, dim3(64), 0, stream, p);
}

template <int DT>
hipError_t launch_merge_d(const DecodeParams& p, int head_dim, hipStream_t stream) {
    switch (head_dim) {
        case 64: return launch_merge_dd<DT, 64>(p, stream);
        case 128: return launch_merge_dd<DT, 128>(p, stream);
        case 256: return launch_merge_dd<DT, 256>(p, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

pa_status_t plan_decode(pa_dtype_t dt, int head_dim, int group, int num_seqs, int part_blocks, bool stream,
                        size_t lds_per_cu, size_t lds_per_wg, int max_per_cu, DecodePlan* out) {
    struct Candidate {
        pa_decode_kernel_t kernel;
        size_t fixed;
        int cap;       // most resident workgroups per CU
        int multiple;  // ring slots come in multiples of this (one share per wave)
    };
    Candidate c[2];
    int n = 0;
    const int regs = max_per_cu < 1 ? 1 : max_per_cu;
    if (stream) {
        // the stream split's records differ: no other kernel can stand in
        c[n++] = {PA_DECODE_MFMA_STREAM, decode_smem_stream(num_seqs, head_dim, group),
                  std::min(kMfmaWgPerCu, regs), kWaves};
    } else if (decode_uses_mfma(dt, group)) {
        const int cap = std::min(kMfmaWgPerCu, regs);
        if (part_blocks <= kWaveSlice)
            c[n++] = {PA_DECODE_MFMA_WAVE, decode_smem_mfma_wave(num_seqs, head_dim, group), cap, kWaves};
        c[n++] = {PA_DECODE_MFMA, decode_smem_mfma(num_seqs, head_dim, group), cap, 1};
    } else {
        c[n++] = {PA_DECODE_VALU, decode_smem_valu(num_seqs, head_dim, group), regs, 1};
    }
    for (int i = 0; i < n; ++i) {
        const size_t slot = ring_slot_bytes(head_dim, group, c[i].kernel == PA_DECODE_MFMA_STREAM);
        const int ring = ring_slots_for(c[i].fixed, slot, c[i].cap, lds_per_cu, lds_per_wg) /
                         c[i].multiple * c[i].multiple;
        if (ring < 1) continue;  // (for the wave kernel: the one-item-per-workgroup kernel needs less)
        const size_t smem = c[i].fixed + static_cast<size_t>(ring) * slot;
        const size_t alloc = lds_alloc(smem);
        if (alloc > lds_per_wg || alloc > lds_per_cu) continue;
        const int resident = std::min(c[i].cap, static_cast<int>(lds_per_cu / alloc));
        if (resident < 1) continue;
        out->kernel = c[i].kernel;
        out->smem = smem;
        out->ring_slots = ring;
        out->resident = resident;
        return PA_OK;
    }
    return PA_ERR_UNSUPPORTED;
}

bool decode_uses_mfma(pa_dtype_t dt, int group) { return dt != PA_F32 && group >= 2; }

bool decode_wave_items(pa_dtype_t dt, int group, int part_blocks) {
    return decode_uses_mfma(dt, group) && part_blocks <= kWaveSlice;
}

bool decode_stream_shape(pa_dtype_t dt, int block_size) { return dt != PA_F32 && block_size >= 4; }

bool decode_stream(pa_dtype_t dt, int group, int block_size, int part, int num_seqs, int num_kv_heads, int max_ctx) {
    if (group < 1 || !decode_stream_shape(dt, block_size) || part / block_size > kWaveSlice) return false;
    // cost positions are int32 in the kernel
    const long long tiles = max_ctx > 0 ? (static_cast<long long>(max_ctx) + 15) / 16 : 1;
    const long long cost = static_cast<long long>(num_seqs) * num_kv_heads * (kStreamTileCost * tiles + kStreamPairCost);
    return cost < (1ll << 31) - 1;
}

int decode_min_block_size(pa_dtype_t dt, int head_dim, int group) {
    if (decode_uses_mfma(dt, group)) return 4;
    const int e = dt == PA_F32 ? 4 : 2;
    const int lpr = head_dim / (16 / e);
    const int rpi = 64 / lpr;
    const int u = rpi >= 4 ? 4 : 16 / rpi;
    return rpi > u ? rpi : u;
}

bool decode_supported(pa_dtype_t dt, int head_dim, int group) {
    if (!(head_dim == 64 || head_dim == 128 || head_dim == 256)) return false;
    if (dt == PA_F32) return group == 1 || group == 2 || group == 4 || group == 8;
    if (dt == PA_BF16 || dt == PA_F16) return group == 1 || group == 2 || group == 4 || group == 8 || group == 16;
    return false;
}

hipError_t launch_decode_partitions(const DecodeParams& p, pa_dtype_t dt, int head_dim, const DeviceInfo& dv,
                                    hipStream_t stream) {
    switch (dt) {
        case PA_F32: return launch_dt<PA_F32>(p, head_dim, dv, stream);
        case PA_BF16: return launch_dt<PA_BF16>(p, head_dim, dv, stream);
        case PA_F16: return launch_dt<PA_F16>(p, head_dim, dv, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_decode_merge(const DecodeParams& p, pa_dtype_t dt, int head_dim,
                               hipStream_t stream) {
    // without the stream split, single-partition batches were written directly
    if (p.pmax <= 1 && !p.stream) return hipSuccess;
    switch (dt) {
        case PA_F32: return launch_merge_d<PA_F32>(p, head_dim, stream);
        case PA_BF16: return launch_merge_d<PA_BF16>(p, head_dim, stream);
        case PA_F16: return launch_merge_d<PA_F16>(p, head_dim, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace pa
