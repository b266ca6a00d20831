// Paged prefill attention for gfx950 (MI355X): several new tokens per
// sequence, each attending to the sequence's cached tokens up to and
// including its own position, read through the block table.
//
// Operation. Sequence s holds L tokens in its blocks, the last M of them new
// (already written by the cache write). New token i sits at position
// p = L - M + i and attends to positions 0..p (lihaoran.work note, section
// 块表把逻辑顺序映射到物理位置: causal attention covers the whole visible
// history; the paging only changes where the rows live). Token t is read at
// block_table[t / B], offset t % B (aiqz.cc tutorial, section 块表映射机制).
// With M = 1 this is the decode of the same sequence.
//
// Work decomposition. A workgroup takes (query tile, sequence, KV head): up to
// QT new tokens of one sequence times the G query heads that share the KV
// head. Each of its four waves owns 16 * NC query columns, a column being a
// (token, head) pair with the head fastest, so a wave holds TPW = 16 * NC / G
// consecutive tokens. Query tiles are counted back from the last new token,
// and the workgroup ids cover the last tile of every sequence first: the
// tiles with the most keys start first.
//
// Keys go through LDS in tiles of KT tokens, double buffered: every thread
// fetches its share of the next tile (block ids one tile further ahead) into
// registers while the current tile is reduced, then writes it to the other
// buffer. K rows are padded by 16 bytes so that the MFMA operand reads are
// free of bank conflicts. V is kept as the cache keeps it, head_dim-major, in
// groups of 32 keys whose order is permuted to the operand layout below.
//
// Per 32 keys and 16-column block, S^T = K Q^T is two 16x16 tiles of D/32
// v_mfma_f32_16x16x32 (K rows as A from LDS, the query columns as B, held in
// registers for the whole item). Lane (r16, j) of a tile holds keys 4j..4j+3
// of column r16. After exp2 and rounding, the lane's eight probabilities --
// keys 4j..4j+3 of the first tile and 16+4j..16+4j+3 of the second -- are
// exactly the B operand of one v_mfma_f32_16x16x32 over those 32 keys, taken
// as its k index 8j..8j+7; the A operand, V^T rows with the same key order, is
// one 16-byte LDS read because the staging wrote V in that order. P never
// leaves registers, and both products run at the double-rate 16x16x32 form.
// The running max is rescaled lazily, only when a block's max exceeds it by
// more than 2^8, as in the decode kernel.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Tile geometry for one head_dim.
template <int D>
struct PrefillShape {
    static constexpr int NC = D >= 256 ? 2 : 4;   // 16-column blocks per wave
    static constexpr int KT = D >= 256 ? 32 : 64;  // keys per LDS tile
    static constexpr int KROW = D + 8;             // LDS K row stride (elements)
    static constexpr int VROW = 32 + 8;            // LDS V row stride of a 32-key group (elements)
    static constexpr int K_EL = KT * KROW;
    static constexpr int V_EL = (KT / 32) * D * VROW;
    static constexpr int BUF_EL = K_EL + V_EL;     // one buffer, in 16-bit elements
    static constexpr int U = KT * D / 8 / kThreads;  // 16-byte K units (and V units) per thread
    static_assert(U * kThreads * 8 == KT * D, "tile must split evenly over the threads");
};

template <int D>
constexpr int prefill_query_tile(int g) { return kWaves * 16 * PrefillShape<D>::NC / g; }

template <int D>
constexpr size_t prefill_smem() { return 2 * static_cast<size_t>(PrefillShape<D>::BUF_EL) * 2; }

template <int DT>
__device__ __forceinline__ f32x4_t mfma32(const u32x4& a, const u32x4& b, f32x4_t c) {
    if constexpr (DT == PA_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Two probabilities as the element type (round to nearest even); ra / rb are
// the rounded values, so the denominator sums what the numerator multiplies.
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

// Four floats rounded to the element type, packed for one 8-byte store.
template <int DT>
__device__ __forceinline__ u32x2 pack4(float a, float b, float c, float d) {
    float ra, rb;
    return u32x2{pack2<DT>(a, b, ra, rb), pack2<DT>(c, d, ra, rb)};
}

template <int DT, int D, int G>
__global__ __launch_bounds__(kThreads) void pa_prefill_mfma(PrefillParams p) {
    static_assert(DT == PA_BF16 || DT == PA_F16, "MFMA path is for 16-bit elements");
    static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "group size");
    using SH = PrefillShape<D>;
    constexpr int NC = SH::NC, KT = SH::KT, KROW = SH::KROW, VROW = SH::VROW, U = SH::U;
    constexpr int NK = D / 32;          // 16x16x32 products per S^T tile
    constexpr int NV = D / 16;          // 16-row blocks of O^T
    constexpr int TPW = 16 * NC / G;    // query tokens per wave
    constexpr int QT = kWaves * TPW;    // query tokens per workgroup
    constexpr int E = 2;
    constexpr float kLazy = 8.f;
    constexpr float kFloor = -1e30f;    // running-max start: exp2(x - kFloor) never meets -inf - -inf

    extern __shared__ __align__(16) uint16_t lds[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, j = lane >> 4;

    // ---- the item: query tile kq (counted from the end), sequence, KV head
    const int per_tile = p.num_seqs * p.num_kv_heads;
    const int kq = blockIdx.x / per_tile;
    const int rest = blockIdx.x - kq * per_tile;
    const int s = rest / p.num_kv_heads;
    const int kv = rest - s * p.num_kv_heads;

    int L = p.context_lens[s];
    L = L < 0 ? 0 : (L > p.max_ctx ? p.max_ctx : L);
    int q0 = p.query_start[s], q1 = p.query_start[s + 1];
    q0 = q0 < 0 ? 0 : (q0 > p.num_tokens ? p.num_tokens : q0);
    q1 = q1 < q0 ? q0 : (q1 > p.num_tokens ? p.num_tokens : q1);
    const int M = min(q1 - q0, p.max_q);
    const int e_lo = kq * QT;  // new tokens after this tile
    if (e_lo >= M) return;
    const int nrow = min(M - e_lo, QT);
    const int pos0 = L - e_lo - nrow;  // position of the tile's first token (negative if M > L)
    const int row0 = q1 - e_lo - nrow; // its row of q / out
    const int nkeys = max(0, L - e_lo);
    const int nkt = (nkeys + KT - 1) / KT;

    // this wave's tokens [uw0, uw1) of the tile; positions pw_min..pw_max
    const int uw0 = wave * TPW;
    const int uw1 = min(uw0 + TPW, nrow);
    const int pw_min = pos0 + uw0;
    const int pw_max = uw1 > uw0 ? pos0 + uw1 - 1 : -1;

    // ---- query fragments and positions of this lane's columns
    const int hq = p.num_heads;
    u32x4 qf[NC][NK];
    int pcol[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const int c = 16 * n + r16;
        const int u = min(uw0 + c / G, nrow - 1);
        const int h = kv * G + c % G;
        pcol[n] = pos0 + u;
        const char* qrow = static_cast<const char*>(p.q) +
                           ((static_cast<size_t>(row0 + u) * hq + h) * D + 8 * j) * E;
#pragma unroll
        for (int c2 = 0; c2 < NK; ++c2) qf[n][c2] = *reinterpret_cast<const u32x4*>(qrow + 64 * c2);
    }

    f32x4_t acc[NC][NV];
#pragma unroll
    for (int n = 0; n < NC; ++n)
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[n][v] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run[NC], lsum[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        m_run[n] = kFloor;
        lsum[n] = 0.f;
    }

    if (nkt > 0) {
        // ---- staging geometry: this thread's K units (key, 8-element chunk)
        // and V units (d, 8 keys) of a tile
        const int bs = 1 << p.log2_bs;
        const int vt = 1 << p.log2_vt;
        const int hkv = p.num_kv_heads;
        const size_t blk_el = static_cast<size_t>(bs) * D;
        const char* kbase = static_cast<const char*>(p.k_cache);
        const char* vbase = static_cast<const char*>(p.v_cache);
        const int* trow = p.block_tables + static_cast<size_t>(s) * p.max_blocks;
        const int lastk = L - 1;
        const bool v16 = vt >= 8;  // 8 consecutive keys are one 16-byte run
        int k_key[U], k_ch[U], v_key[U], v_d[U], v_lds[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int uk = tid + i * kThreads;
            k_key[i] = uk / (D / 8);
            k_ch[i] = uk % (D / 8);
            const int grp = uk / (4 * D);  // 32-key group of the tile
            const int w = uk % (4 * D);
            const int h = w / (2 * D);     // which 16 keys of the group
            const int d = (w % (2 * D)) >> 1;
            const int half = w & 1;        // which 8 of those 16
            v_key[i] = 32 * grp + 16 * h + 8 * half;
            v_d[i] = d;
            // key 16h + 4j' + r of a group sits at position 8j' + 4h + r of its row
            v_lds[i] = SH::K_EL + (grp * D + d) * VROW + 16 * half + 4 * h;
        }
        auto clamp_pid = [&](int pid) { return pid < 0 ? 0 : (pid >= p.num_blocks ? p.num_blocks - 1 : pid); };
        // keys past the last one are read at a clamped, in-bounds position
        // (their values are masked or zeroed)
        auto kkey = [&](int t) { return min(t, lastk); };
        auto vkey0 = [&](int t) { return min(t, v16 ? (lastk & ~7) : (lastk & ~3)); };
        auto vkey1 = [&](int t) { return min(t + 4, lastk & ~3); };

        int tk[U], tv0[U], tv1[U];
        auto fetch_table = [&](int kt) {
            const int t0 = kt * KT;
#pragma unroll
            for (int i = 0; i < U; ++i) {
                tk[i] = trow[kkey(t0 + k_key[i]) >> p.log2_bs];
                tv0[i] = trow[vkey0(t0 + v_key[i]) >> p.log2_bs];
                if (!v16) tv1[i] = trow[vkey1(t0 + v_key[i]) >> p.log2_bs];
                else tv1[i] = 0;
            }
        };
        auto v_elem = [&](int pid, int t, int d) {
            const int off = t & (bs - 1);
            return (static_cast<size_t>(pid) * hkv + kv) * blk_el +
                   static_cast<size_t>(off >> p.log2_vt) * D * vt + static_cast<size_t>(d) * vt + (off & (vt - 1));
        };
        u32x4 rk[U], rv[U];
        auto fetch_kv = [&](int kt) {
            const int t0 = kt * KT;
#pragma unroll
            for (int i = 0; i < U; ++i) {
                const int t = kkey(t0 + k_key[i]);
                const size_t kel = (static_cast<size_t>(clamp_pid(tk[i])) * hkv + kv) * blk_el +
                                   static_cast<size_t>(t & (bs - 1)) * D + 8 * k_ch[i];
                rk[i] = *reinterpret_cast<const u32x4*>(kbase + kel * E);
                const int tv = t0 + v_key[i];
                if (v16) {
                    rv[i] = *reinterpret_cast<const u32x4*>(vbase + v_elem(clamp_pid(tv0[i]), vkey0(tv), v_d[i]) * E);
                } else {
                    const u32x2 a = *reinterpret_cast<const u32x2*>(vbase + v_elem(clamp_pid(tv0[i]), vkey0(tv), v_d[i]) * E);
                    const u32x2 b = *reinterpret_cast<const u32x2*>(vbase + v_elem(clamp_pid(tv1[i]), vkey1(tv), v_d[i]) * E);
                    rv[i] = u32x4{a.x, a.y, b.x, b.y};
                }
                // keys at or past nkeys are zeroed: their probability is 0,
                // and a stale slot may hold a non-finite value
                const int nv = nkeys - tv;
                if (nv < 8) {
                    const uint32_t lo = 0x0000ffffu, hi = 0xffff0000u;
                    rv[i].x &= (nv > 0 ? lo : 0u) | (nv > 1 ? hi : 0u);
                    rv[i].y &= (nv > 2 ? lo : 0u) | (nv > 3 ? hi : 0u);
                    rv[i].z &= (nv > 4 ? lo : 0u) | (nv > 5 ? hi : 0u);
                    rv[i].w &= (nv > 6 ? lo : 0u) | (nv > 7 ? hi : 0u);
                }
            }
        };
        auto store_tile = [&](int buf) {
            uint16_t* b = lds + buf * SH::BUF_EL;
#pragma unroll
            for (int i = 0; i < U; ++i) {
                *reinterpret_cast<u32x4*>(b + k_key[i] * KROW + 8 * k_ch[i]) = rk[i];
                *reinterpret_cast<u32x2*>(b + v_lds[i]) = u32x2{rv[i].x, rv[i].y};
                *reinterpret_cast<u32x2*>(b + v_lds[i] + 8) = u32x2{rv[i].z, rv[i].w};
            }
        };

        // ---- reduce one LDS tile
        auto compute = [&](int kt, int buf) {
            const uint16_t* bk = lds + buf * SH::BUF_EL;
            const uint16_t* bv = bk + SH::K_EL;
#pragma unroll
            for (int g32 = 0; g32 < KT / 32; ++g32) {
                const int tok0 = kt * KT + 32 * g32;
                if (tok0 > pw_max) break;  // uniform: past this wave's last position
                f32x4_t st[2][NC];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    u32x4 kf[NK];
                    const uint16_t* krow = bk + (32 * g32 + 16 * tt + r16) * KROW + 8 * j;
#pragma unroll
                    for (int c = 0; c < NK; ++c) kf[c] = *reinterpret_cast<const u32x4*>(krow + 32 * c);
#pragma unroll
                    for (int n = 0; n < NC; ++n) {
                        f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int c = 0; c < NK; ++c) a = mfma32<DT>(kf[c], qf[n][c], a);
                        st[tt][n] = a;
                    }
                }
                // keys at positions past a column's own are masked (only the
                // diagonal groups have any)
                const bool diag = tok0 + 31 > pw_min;
                u32x4 pb[NC];
#pragma unroll
                for (int n = 0; n < NC; ++n) {
                    float x[8];
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int key = tok0 + 16 * tt + 4 * j + r;
                            const bool ok = !diag || key <= pcol[n];
                            x[4 * tt + r] = ok ? st[tt][n][r] * p.scale_log2 : -INFINITY;
                        }
                    float tmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                                       fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
                    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
                    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
                    const bool need = tmax > m_run[n] + kLazy;
                    if (__any(need)) {
                        const float mn = need ? tmax : m_run[n];
                        const float alpha = fast_exp2(m_run[n] - mn);
#pragma unroll
                        for (int v = 0; v < NV; ++v) acc[n][v] *= alpha;
                        lsum[n] *= alpha;
                        m_run[n] = mn;
                    }
                    float pr[8];
                    const float m = m_run[n];
                    pb[n].x = pack2<DT>(fast_exp2(x[0] - m), fast_exp2(x[1] - m), pr[0], pr[1]);
                    pb[n].y = pack2<DT>(fast_exp2(x[2] - m), fast_exp2(x[3] - m), pr[2], pr[3]);
                    pb[n].z = pack2<DT>(fast_exp2(x[4] - m), fast_exp2(x[5] - m), pr[4], pr[5]);
                    pb[n].w = pack2<DT>(fast_exp2(x[6] - m), fast_exp2(x[7] - m), pr[6], pr[7]);
                    lsum[n] += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
                }
                const uint16_t* vrow = bv + (g32 * D + r16) * VROW + 8 * j;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const u32x4 vf = *reinterpret_cast<const u32x4*>(vrow + 16 * v * VROW);
#pragma unroll
                    for (int n = 0; n < NC; ++n) acc[n][v] = mfma32<DT>(vf, pb[n], acc[n][v]);
                }
            }
        };

        // ---- pipeline: tile kt is reduced while tile kt+1 is fetched and the
        // block ids of tile kt+2 are read; fetches past the last tile repeat it
        fetch_table(0);
        fetch_kv(0);
        fetch_table(min(1, nkt - 1));
        store_tile(0);
        __syncthreads();
        for (int kt = 0; kt < nkt; ++kt) {
            fetch_kv(min(kt + 1, nkt - 1));
            fetch_table(min(kt + 2, nkt - 1));
            compute(kt, kt & 1);
            store_tile((kt + 1) & 1);  // the buffer nobody reads during this tile
            __syncthreads();
        }
    }

    // ---- normalise and store: acc[n][v][r] = O^T[d = 16v + 4j + r][column r16 of block n]
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        float l = lsum[n];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const int c = 16 * n + r16;
        const int u = uw0 + c / G;
        if (u < nrow) {
            const int h = kv * G + c % G;
            char* orow = static_cast<char*>(p.out) + ((static_cast<size_t>(row0 + u) * hq + h) * D + 4 * j) * E;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const f32x4_t o = acc[n][v] * inv;
                *reinterpret_cast<u32x2*>(orow + 32 * v) = pack4<DT>(o[0], o[1], o[2], o[3]);
            }
        }
    }
}

template <int DT, int D, int G>
hipError_t launch_prefill_g(const PrefillParams& p, hipStream_t stream) {
    constexpr int QT = prefill_query_tile<D>(G);
    const long long qtiles = (static_cast<long long>(p.max_q) + QT - 1) / QT;
    const long long grid = qtiles * p.num_seqs * p.num_kv_heads;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((pa_prefill_mfma<DT, D, G>), dim3(static_cast<unsigned>(grid)), dim3(kThreads),
                       prefill_smem<D>(), stream, p);
    return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_prefill_d(const PrefillParams& p, int group, hipStream_t stream) {
    switch (group) {
        case 1: return launch_prefill_g<DT, D, 1>(p, stream);
        case 2: return launch_prefill_g<DT, D, 2>(p, stream);
        case 4: return launch_prefill_g<DT, D, 4>(p, stream);
        case 8: return launch_prefill_g<DT, D, 8>(p, stream);
        case 16: return launch_prefill_g<DT, D, 16>(p, stream);
    }
    return hipErrorInvalidValue;
}

template <int DT>
hipError_t launch_prefill_dt(const PrefillParams& p, int head_dim, int group, hipStream_t stream) {
    switch (head_dim) {
        case 64: return launch_prefill_d<DT, 64>(p, group, stream);
        case 128: return launch_prefill_d<DT, 128>(p, group, stream);
        case 256: return launch_prefill_d<DT, 256>(p, group, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool prefill_supported(pa_dtype_t dt, int head_dim, int group) {
    if (dt != PA_BF16 && dt != PA_F16) return false;
    if (!(head_dim == 64 || head_dim == 128 || head_dim == 256)) return false;
    return group == 1 || group == 2 || group == 4 || group == 8 || group == 16;
}

hipError_t launch_prefill(const PrefillParams& p, pa_dtype_t dt, int head_dim, int group, hipStream_t stream) {
    switch (dt) {
        case PA_BF16: return launch_prefill_dt<PA_BF16>(p, head_dim, group, stream);
        case PA_F16: return launch_prefill_dt<PA_F16>(p, head_dim, group, stream);
        default: break;
    }
    return hipErrorInvalidValue;
}

}  // namespace pa
