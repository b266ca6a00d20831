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
// tiles with the most keys start first. Two workgroups fit per CU.
//
// Keys go through LDS in tiles of KT tokens, double buffered, loaded by
// global_load_lds (no register holds staged data): the next tile's loads fly
// while the current tile is reduced. Each load instruction covers keys of one
// aligned 16-key group, so with blocks of 16 or more tokens its block id is
// wave-uniform (read from the wave's own lanes of the table entries, loaded a
// tile ahead). K rows are stored in a permuted order (below) with their
// 16-byte chunks XOR-swizzled; V keeps the cache's own 16-key tiles [D][16],
// the two halves of a row swizzled; both keep the MFMA operand reads on
// distinct banks.
//
// Per 32 keys and 16-column block, S^T = K Q^T is two 16x16 tiles of D/32
// v_mfma_f32_16x16x32 (K rows as A from LDS, the query columns as B, held in
// registers for the whole item). The K rows of a 32-key group are stored so
// that lane (r16, j) of the two tiles holds keys 8j..8j+3 and 8j+4..8j+7:
// eight consecutive keys, which after exp2 and rounding are exactly the B
// operand of one v_mfma_f32_16x16x32 over the 32 keys (k index 8j..8j+7),
// whose A operand, V^T, is then a plain 16-byte read of the cache's V layout.
// P never leaves registers, and both products run at the double-rate 16x16x32
// form. The softmax keeps its running max over unscaled logits (a negative
// scale is folded into q), reduces a column's four lanes with lane swaps,
// rescales lazily (only when the max grows by more than 2^8, as in the decode
// kernel), and takes its denominator from one more MFMA against a row of
// ones.
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
    static constexpr int NC = D >= 256 ? 1 : 2;    // 16-column blocks per wave
    static constexpr int KT = D >= 256 ? 32 : 64;   // keys per LDS tile
    static constexpr int ROWB = D * 2;              // bytes of one K row
    static constexpr int K_BYTES = KT * ROWB;       // K of a tile
    static constexpr int V_BYTES = KT * ROWB;       // V of a tile
    static constexpr int BUF_BYTES = K_BYTES + V_BYTES;
    static constexpr int UK = K_BYTES / 1024 / kWaves;  // 16-byte DMA loads of K per lane and tile
    static constexpr int UV = V_BYTES / 1024 / kWaves;  // of V (blocks of 8 or more tokens)
    static constexpr int UV4 = V_BYTES / 256 / kWaves;  // 4-byte DMA loads of V (blocks of 4 tokens)
    static constexpr int TBL = 16;                  // block ids of one tile: KT / 4 at most
    static_assert(UK * kWaves * 1024 == K_BYTES && UV * kWaves * 1024 == V_BYTES, "whole loads");
    static_assert(KT / 4 <= TBL, "table slice");
};

template <int D>
constexpr int prefill_query_tile(int g) { return kWaves * 16 * PrefillShape<D>::NC / g; }

constexpr int kXcds = 8;  // XCDs of MI355X, which take consecutive workgroup ids in turn

// Key (within the tile) that LDS row r of K holds: the rows of a 32-key
// group are permuted so that each lane's eight S^T scores are eight
// consecutive keys.
__host__ __device__ constexpr int k_key_of_row(int r) {
    return 32 * (r >> 5) + 8 * ((r & 15) >> 2) + 4 * ((r >> 4) & 1) + (r & 3);
}

// First LDS row of K load instruction i of wave w when every block holds
// whole 16-key groups: wave w fills exactly the rows of keys KT/4 * w ..
// KT/4 * (w + 1) - 1 (16 keys, 8 at D = 256), so all its K loads (and its
// V loads, the 16-key tile holding those keys) read one block.
template <int D>
__host__ __device__ constexpr int k_row0(int w, int i) {
    if constexpr (D == 64) return 32 * (w >> 1) + 16 * i + 8 * (w & 1);
    else if constexpr (D == 128) return 32 * (w >> 1) + 16 * (i >> 1) + 8 * (w & 1) + 4 * (i & 1);
    else return 16 * (i >> 1) + 4 * w + 2 * (i & 1);
}

template <int D>
constexpr size_t prefill_smem() {
    return 2 * static_cast<size_t>(PrefillShape<D>::BUF_BYTES) + 2 * PrefillShape<D>::TBL * sizeof(int);
}

// Swizzle of the 16-byte chunks of K row r in LDS: any 8 (and any 16)
// consecutive rows of one MFMA operand read land on distinct banks.
template <int D>
__device__ __forceinline__ int k_swz(int r) {
    if constexpr (D == 64) return (r & 7) ^ ((r >> 3) & 1);
    else return r & 15;
}

// Which stored 16-byte half of V row d holds key half `h` (same rule).
__device__ __forceinline__ int v_swz(int d) { return ((d >> 2) ^ (d >> 3)) & 1; }

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

// max(a, b, c) in one instruction. The operands are finite or -inf here, so
// the IEEE-mode quieting the compiler would add around fmaxf is not needed.
__device__ __forceinline__ float max3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Max and sum over the four lanes r16, r16 + 16, r16 + 32, r16 + 48 (one
// column of a 16x16 MFMA result), every one of them receiving the result:
// v_permlane16_swap exchanges rows 1 and 3 of its first operand with rows 0
// and 2 of its second, v_permlane32_swap the upper half of the first with the
// lower half of the second, so with both operands equal to v each pair of
// results holds the two values to combine.
__device__ __forceinline__ float column_max(float v) {
    const uint32_t a = f32_as_u32(v);
    const auto r = __builtin_amdgcn_permlane16_swap(a, a, false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    const float a0 = u32_as_f32(r0), a1 = u32_as_f32(r1);
    const uint32_t b = f32_as_u32(a0 > a1 ? a0 : a1);
    const auto t = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    const uint32_t t0 = t[0], t1 = t[1];
    const float b0 = u32_as_f32(t0), b1 = u32_as_f32(t1);
    return b0 > b1 ? b0 : b1;
}

__device__ __forceinline__ float column_sum(float v) {
    const uint32_t a = f32_as_u32(v);
    const auto r = __builtin_amdgcn_permlane16_swap(a, a, false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    const uint32_t b = f32_as_u32(u32_as_f32(r0) + u32_as_f32(r1));
    const auto t = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    const uint32_t t0 = t[0], t1 = t[1];
    return u32_as_f32(t0) + u32_as_f32(t1);
}

typedef __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// Global -> LDS load: every lane's `bytes` land at lds_base + lane * bytes
// (lds_base is the same for the whole wave).
template <int BYTES>
__device__ __forceinline__ void dma(const void* src, void* lds_base) {
    static_assert(BYTES == 4 || BYTES == 16, "load size");
    if constexpr (BYTES == 16)
        __builtin_amdgcn_global_load_lds((gptr_t)(const_cast<void*>(src)), (lptr_t)(lds_base), 16, 0, 0);
    else
        __builtin_amdgcn_global_load_lds((gptr_t)(const_cast<void*>(src)), (lptr_t)(lds_base), 4, 0, 0);
}

// Two waves per SIMD (two workgroups per CU): the register budget is held to
// 256 per lane.
template <int DT, int D, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void pa_prefill_mfma(
    PrefillParams p) {
    static_assert(DT == PA_BF16 || DT == PA_F16, "MFMA path is for 16-bit elements");
    static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "group size");
    using SH = PrefillShape<D>;
    constexpr int NC = SH::NC, KT = SH::KT, ROWB = SH::ROWB;
    constexpr int NK = D / 32;          // 16x16x32 products per S^T tile
    constexpr int NV = D / 16;          // 16-row blocks of O^T
    constexpr int TPW = 16 * NC / G;    // query tokens per wave
    constexpr int QT = kWaves * TPW;    // query tokens per workgroup
    constexpr int E = 2;
    constexpr float kLazy = 8.f;
    constexpr float kFloor = -1e30f;    // running-max start: exp2(x - kFloor) never meets -inf - -inf

    // LDS: two tile buffers [K | V], then two table slices of block ids
    // (used with blocks of fewer than 16 tokens)
    extern __shared__ __align__(16) unsigned char lds[];
    int* tbl = reinterpret_cast<int*>(lds + 2 * SH::BUF_BYTES);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, j = lane >> 4;

    // ---- the item: query tile kq (counted from the end), sequence, KV head.
    // Tile-major by default: the last tile of every pair (the most keys)
    // first. Workgroup ids go to the XCDs in turn; with pair_major set and
    // the (sequence, KV head) pairs splitting evenly over the XCDs, each XCD
    // takes whole pairs instead, one after the other with all query tiles of
    // a pair in a row (its last tile first): the tiles of a pair run side by
    // side on one XCD and read the pair's K/V rows through that XCD's L2
    // instead of each from memory.
    const int per_tile = p.num_seqs * p.num_kv_heads;
    int kq, pair;
    if (p.pair_major && per_tile % kXcds == 0) {
        const int tiles = gridDim.x / per_tile;
        const int x = blockIdx.x % kXcds;  // this XCD
        const int k = blockIdx.x / kXcds;  // index on this XCD
        int pl = k / tiles;
        kq = k - pl * tiles;
        // Longest first: the XCD's pairs x + 8 i are taken in the order of
        // their sequences' context lengths, longest first (ties by i), so
        // that the last items to start are short ones. Every wave ranks the
        // (at most 64) pairs in its lanes itself.
        const int nx = per_tile / kXcds;
        if (nx <= 64) {
            const int li = lane < nx ? p.context_lens[(x + kXcds * lane) / p.num_kv_heads] : -1;
            int r = 0;
            for (int i2 = 0; i2 < nx; ++i2) {
                const int l2 = __builtin_amdgcn_readlane(li, i2);
                r += (l2 > li) || (l2 == li && i2 < lane);
            }
            const unsigned long long hit = __ballot(lane < nx && r == pl);
            if (hit != 0) pl = __builtin_ctzll(hit);
        }
        pair = x + kXcds * pl;
    } else {
        kq = blockIdx.x / per_tile;
        pair = blockIdx.x - kq * per_tile;
    }
    const int s = pair / p.num_kv_heads;
    const int kv = pair - s * p.num_kv_heads;

    // Block ids of the first two key tiles, loaded before the sequence's
    // length is known: entries past its last block are loaded but never used
    // (every load of a tile reads the block of a key at most the last one).
    int traw0 = 0, traw1 = 0;
    {
        const int ntb = KT >= (1 << p.log2_bs) ? KT >> p.log2_bs : 1;
        const int* trow = p.block_tables + static_cast<size_t>(s) * p.max_blocks;
        const int hi = p.max_blocks - 1;
        if (lane < ntb && hi >= 0) {
            traw0 = trow[min(lane, hi)];
            traw1 = trow[min((KT >> p.log2_bs) + lane, hi)];
        }
    }

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

    // this wave's first token of the tile and its position
    const int uw0 = wave * TPW;
    const int pw_min = pos0 + uw0;

    // ---- query fragments and positions of this lane's columns. A negative
    // scale is folded into q (a sign flip is exact), so that the running
    // maximum can be taken over the unscaled products.
    const int hq = p.num_heads;
    const uint32_t qsign = p.scale_log2 < 0.f ? 0x80008000u : 0u;
    // (a zero scale is taken as 1e-30: masked keys then stay at -inf, and
    // exp2 of any finite logit times 1e-30 rounds to exactly 1)
    const float sc = fmaxf(fabsf(p.scale_log2), 1e-30f);
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
        for (int c2 = 0; c2 < NK; ++c2) qf[n][c2] = *reinterpret_cast<const u32x4*>(qrow + 64 * c2) ^ qsign;
    }

    // O^T accumulators, and per block one more 16x16 tile whose row 0 sums
    // the probabilities: its A operand is 1 in row 0 and 0 elsewhere, so the
    // softmax denominator comes out of the same MFMA pipe as the numerator
    // and sums exactly the rounded weights the numerator multiplies.
    f32x4_t acc[NC][NV], accl[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        accl[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[n][v] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    constexpr uint32_t kOne2 = DT == PA_BF16 ? 0x3f803f80u : 0x3c003c00u;  // two 1.0 elements
    const u32x4 ones = r16 == 0 ? u32x4{kOne2, kOne2, kOne2, kOne2} : u32x4{0u, 0u, 0u, 0u};
    float m_run[NC];  // running max of the scaled logits, log2 units
    float thr[NC];    // (m_run + 8) / scale: unscaled logits above it trigger a rescale
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        m_run[n] = kFloor;
        thr[n] = (kFloor + kLazy) / sc;
    }

    if (nkt > 0) {
        const int lb = p.log2_bs;
        const int bs = 1 << lb;
        const int lvt = p.log2_vt;
        const int vt = 1 << lvt;
        const int hkv = p.num_kv_heads;
        const size_t blk_el = static_cast<size_t>(bs) * D;
        const char* kbase = static_cast<const char*>(p.k_cache);
        const char* vbase = static_cast<const char*>(p.v_cache);
        const int* trow = p.block_tables + static_cast<size_t>(s) * p.max_blocks;
        const int lastk = L - 1;
        const int last_blk = lastk >> lb;
        const int ntb = KT >= bs ? KT >> lb : 1;  // block ids one tile spans
        const bool big = bs >= 16;                 // every aligned 16 keys share a block
        auto clamp_pid = [&](int pid) { return pid < 0 ? 0 : (pid >= p.num_blocks ? p.num_blocks - 1 : pid); };
        // raw block id of table entry (kt * KT >> lb) + lane, in lanes < ntb of
        // every wave (clamped where it is used); entries past the context's
        // last block are never read
        auto lookup = [&](int kt) {
            const int e = min(((kt * KT) >> lb) + lane, last_blk);
            return trow[lane < ntb ? e : 0];
        };
        auto head_el = [&](int pid) { return (static_cast<size_t>(pid) * hkv + kv) * blk_el; };
        // byte address of (block pid, this KV head) for a wave-uniform pid:
        // one 32 x 32 -> 64-bit product on the scalar unit (a block's heads
        // span hkv * B * D * E < 2^32 bytes)
        const uint32_t blk_bytes = static_cast<uint32_t>(hkv * blk_el * E);
        const char* kbase_kv = kbase + kv * blk_el * E;
        const char* vbase_kv = vbase + kv * blk_el * E;
        auto head_bytes = [&](int pid) {
            return static_cast<uint64_t>(static_cast<uint32_t>(pid)) * blk_bytes;
        };

        // Static part of this lane's loads. LDS row r of K holds key
        // 32 (r / 32) + 8 ((r % 16) / 4) + 4 ((r / 16) % 2) + r % 4 of the tile,
        // so that the two 16-row S^T tiles of a 32-key group give every lane
        // eight consecutive keys; chunk ch of row r sits at ch ^ k_swz(r). One
        // K load instruction covers rows of one aligned 16-key group. V keeps
        // the cache's layout of 16-key tiles [D][16], its two 16-byte halves
        // stored in the order v_swz(d); one 16-byte V load instruction covers
        // rows of one 16-key tile.
        // (recomputed at every tile: a few instructions, no registers held)
        auto k_key = [&](int i) {
            const int r = ((wave * SH::UK + i) * 1024 + lane * 16) / ROWB;
            const int m = r & 15;
            return 32 * (r >> 5) + 8 * (m >> 2) + 4 * ((r >> 4) & 1) + (m & 3);
        };
        auto k_chb = [&](int i) {
            const int P = (wave * SH::UK + i) * 1024 + lane * 16;
            return (((P % ROWB) >> 4) ^ k_swz<D>(P / ROWB)) << 4;
        };
        auto v_d = [&](int i) { return (((wave * SH::UV + i) * 1024 + lane * 16) % (D * 32)) >> 5; };
        auto v_half = [&](int i) { return (lane & 1) ^ v_swz(v_d(i)); };  // bit 4 of the LDS byte position

        // Issue the loads of tile kt into buffer `buf`; keys past the context
        // are read at the last key's position (their values are masked).
        auto issue = [&](int kt, int buf, int traw) __attribute__((always_inline)) {
            unsigned char* bk = lds + buf * SH::BUF_BYTES;
            unsigned char* bv = bk + SH::K_BYTES;
            const int* tb = tbl + (kt & 1) * SH::TBL;
            const int t0 = kt * KT;
            const int blk0 = t0 >> lb;
            if (big) {
                // This wave's keys (one aligned 16-key group, 8 keys at
                // D = 256) and their V tile lie in one block: one id, read
                // from LDS once, and wave-uniform bases. Keys past the
                // context are read from the block that holds the last key
                // (in bounds; masked: scores to -inf, V to zero).
                constexpr int KPW = KT / kWaves;
                const int g0 = t0 + KPW * wave;
                const int pid = clamp_pid(__builtin_amdgcn_readlane(traw, (min(g0, lastk) >> lb) - blk0));
                const char* blk = kbase_kv + head_bytes(pid);
                const uint32_t k0 = static_cast<uint32_t>((g0 & (bs - 1)) * (D * E));
#pragma unroll
                for (int i = 0; i < SH::UK; ++i) {
                    const int r0 = k_row0<D>(wave, i);
                    const int r = r0 + lane * 16 / ROWB;
                    const int ch = ((lane * 16) % ROWB >> 4) ^ k_swz<D>(r);
                    const uint32_t off = k0 + static_cast<uint32_t>((k_key_of_row(r) - KPW * wave) * (D * E) + ch * 16);
                    dma<16>(blk + off, bk + r0 * ROWB);
                }
                const char* vblk = vbase_kv + head_bytes(pid);
#pragma unroll
                for (int i = 0; i < SH::UV; ++i) {
                    const int sub = (wave * SH::UV + i) * 1024 / (D * 32);
                    const uint32_t off = static_cast<uint32_t>((((t0 + 16 * sub) & (bs - 1)) >> 4) * (D * 16 * E) +
                                                               v_d(i) * 32 + v_half(i) * 16);
                    dma<16>(vblk + off, bv + (wave * SH::UV + i) * 1024);
                }
            } else {
#pragma unroll
                for (int i = 0; i < SH::UK; ++i) {
                    const int key = min(t0 + k_key(i), lastk);
                    const int pid = tb[(key >> lb) - blk0];
                    const char* src = kbase + (head_el(pid) + static_cast<size_t>(key & (bs - 1)) * D) * E + k_chb(i);
                    dma<16>(src, bk + (wave * SH::UK + i) * 1024);
                }
                if (lvt == 3) {
#pragma unroll
                    for (int i = 0; i < SH::UV; ++i) {
                        const int P = (wave * SH::UV + i) * 1024 + lane * 16;
                        const int key = min(t0 + 16 * (P / (D * 32)) + 8 * v_half(i), lastk & ~7);
                        const int pid = tb[(key >> lb) - blk0];
                        const size_t el = head_el(pid) + static_cast<size_t>(v_d(i)) * 8;
                        dma<16>(vbase + el * E, bv + (wave * SH::UV + i) * 1024);
                    }
                } else {
#pragma unroll 4
                    for (int i = 0; i < SH::UV4; ++i) {
                        const int P = (wave * SH::UV4 + i) * 256 + lane * 4;
                        const int d = (P % (D * 32)) >> 5;
                        const int half = ((P >> 4) & 1) ^ v_swz(d);
                        const int key = min(t0 + 16 * (P / (D * 32)) + 8 * half + 2 * ((P >> 2) & 3), lastk & ~1);
                        const int pid = tb[(key >> lb) - blk0];
                        const size_t el = head_el(pid) + static_cast<size_t>(d) * vt + (key & (bs - 1));
                        dma<4>(vbase + el * E, bv + (wave * SH::UV4 + i) * 256);
                    }
                }
            }
        };

        // ---- one 32-key step g (keys 32g .. 32g + 31) in four parts. Step g
        // lies in tile g / SPT, held by buffer (g / SPT) & 1.
        constexpr int SPT = KT / 32;  // steps per tile
        auto step_base = [&](int g) {
            return lds + ((g / SPT) & 1) * SH::BUF_BYTES;
        };
        // K rows of the step's two S^T tiles
        auto read_k = [&](int g, u32x4 (&kf)[2][NK]) {
            const unsigned char* bk = step_base(g);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const int r = 32 * (g % SPT) + 16 * tt + r16;
                const unsigned char* krow = bk + r * ROWB;
#pragma unroll
                for (int c = 0; c < NK; ++c)
                    kf[tt][c] = *reinterpret_cast<const u32x4*>(krow + (((4 * c + j) ^ k_swz<D>(r)) << 4));
            }
        };
        // V^T rows d = 16v + r16 of keys 32g + 8j .. + 7 (16-key tile
        // 2 (g % SPT) + j / 2 of the buffer, half j % 2)
        auto read_v = [&](int g, u32x4 (&vf)[NV]) {
            const unsigned char* bv = step_base(g) + SH::K_BYTES;
            const int vsub = 2 * (g % SPT) + (j >> 1);
            const unsigned char* vrow = bv + (vsub * D + r16) * 32 + (((j & 1) ^ v_swz(r16)) << 4);
#pragma unroll
            for (int v = 0; v < NV; ++v) vf[v] = *reinterpret_cast<const u32x4*>(vrow + 16 * v * 32);
        };
        // S^T = K Q^T: st[tt][n][r] is the unscaled logit of key 32g + 8j + 4tt + r
        // and column r16 of block n
        auto qk = [&](const u32x4 (&kf)[2][NK], f32x4_t (&st)[2][NC]) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int n = 0; n < NC; ++n) {
                    f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int c = 0; c < NK; ++c) a = mfma32<DT>(kf[tt][c], qf[n][c], a);
                    st[tt][n] = a;
                }
        };
        // keys past a column's own position are masked (only the diagonal
        // steps have any; keys past the context are among them)
        auto mask = [&](int g, f32x4_t (&st)[2][NC]) {
            const int tok0 = 32 * g;
            if (tok0 + 31 > pw_min) {
#pragma unroll
                for (int n = 0; n < NC; ++n)
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (tok0 + 8 * j + 4 * tt + r > pcol[n]) st[tt][n][r] = -INFINITY;
            }
        };
        // probabilities of the step against the running max m_run as the PV
        // operand (element type, rounded)
        auto exps = [&](const f32x4_t (&st)[2][NC], u32x4 (&pb)[NC]) {
#pragma unroll
            for (int n = 0; n < NC; ++n) {
                const float m = -m_run[n];
                float pr[8];
                float e[8];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) e[4 * tt + r] = fast_exp2(fmaf(st[tt][n][r], sc, m));
                pb[n].x = pack2<DT>(e[0], e[1], pr[0], pr[1]);
                pb[n].y = pack2<DT>(e[2], e[3], pr[2], pr[3]);
                pb[n].z = pack2<DT>(e[4], e[5], pr[4], pr[5]);
                pb[n].w = pack2<DT>(e[6], e[7], pr[6], pr[7]);
            }
        };
        // online softmax: the probabilities are computed against the current
        // running max first (valid whenever it does not grow by more than
        // 2^8, which is the lazy-rescale rule) and only recomputed, after the
        // accumulators are rescaled, in the rare step where it does. Whether
        // it does is decided on each lane's own eight logits against
        // thr = (m_run + 8) / scale: a column's max passes the threshold iff
        // one of its four lanes does, so the cross-lane max is only needed
        // in that rare step.
        auto softmax = [&](const f32x4_t (&st)[2][NC], u32x4 (&pb)[NC], float (&tl)[NC], bool& need_any) {
            need_any = false;
#pragma unroll
            for (int n = 0; n < NC; ++n) {
                const f32x4_t a = st[0][n], b = st[1][n];
                tl[n] = max3(max3(a[0], a[1], a[2]), max3(a[3], b[0], b[1]), max3(b[2], b[3], -INFINITY));
                need_any |= tl[n] > thr[n];
            }
            exps(st, pb);
        };
        auto rescale = [&](const f32x4_t (&st)[2][NC], u32x4 (&pb)[NC], const float (&tl)[NC]) {
#pragma unroll
            for (int n = 0; n < NC; ++n) {
                const float tmax = column_max(tl[n]) * sc;
                const float mn = tmax > m_run[n] + kLazy ? tmax : m_run[n];
                const float alpha = fast_exp2(m_run[n] - mn);
#pragma unroll
                for (int v = 0; v < NV; ++v) acc[n][v] *= alpha;
                accl[n] *= alpha;
                m_run[n] = mn;
                thr[n] = (mn + kLazy) / sc;
            }
            exps(st, pb);
        };
        // O^T += V^T P^T and the denominator
        auto pv = [&](int g, u32x4 (&vf)[NV], const u32x4 (&pb)[NC]) {
            const int tok0 = 32 * g;
            // keys past the context may hold anything: zero their V
            if (tok0 + 32 > L) {
                const int nv = L - (tok0 + 8 * j);
                const uint32_t lo = 0x0000ffffu, hi = 0xffff0000u;
                const u32x4 vm = {(nv > 0 ? lo : 0u) | (nv > 1 ? hi : 0u), (nv > 2 ? lo : 0u) | (nv > 3 ? hi : 0u),
                                  (nv > 4 ? lo : 0u) | (nv > 5 ? hi : 0u), (nv > 6 ? lo : 0u) | (nv > 7 ? hi : 0u)};
#pragma unroll
                for (int v = 0; v < NV; ++v) vf[v] &= vm;
            }
#pragma unroll
            for (int n = 0; n < NC; ++n) accl[n] = mfma32<DT>(ones, pb[n], accl[n]);
#pragma unroll
            for (int v = 0; v < NV; ++v)
#pragma unroll
                for (int n = 0; n < NC; ++n) acc[n][v] = mfma32<DT>(vf[v], pb[n], acc[n][v]);
        };

        // ---- pipeline. Tiles: the loads of tile t + 1 fly while tile t is
        // reduced; block ids run one tile further ahead through tbl[tile & 1].
        // Steps: the products S of step g + 1 are issued before the softmax
        // of step g, so that the matrix pipe works on them while the vector
        // ALU computes the exponentials; the operands of step g + 1 are read
        // from LDS one step ahead.
        const int nsteps = (nkeys + 31) / 32;
        // With blocks of 16 or more tokens each wave reads its block id from
        // its own lanes of the raw entries (no LDS round trip after the
        // barrier); smaller blocks go through the table slice in LDS.
        if (!big) {
            if (tid < SH::TBL) tbl[tid] = clamp_pid(traw0);
            __syncthreads();
        }
        issue(0, 0, traw0);
        int treg = traw1;
        if (!big && tid < SH::TBL) tbl[SH::TBL + tid] = clamp_pid(treg);
        __syncthreads();
        if (1 < nkt) issue(1, 1, treg);
        treg = lookup(min(2, nkt - 1));

        f32x4_t st_a[2][NC], st_b[2][NC];
        u32x4 vf[NV];
        {
            u32x4 kf[2][NK];
            read_k(0, kf);
            qk(kf, st_a);
            read_v(0, vf);
        }
        // Every wave runs every step (a step past a wave's own positions is
        // fully masked and adds nothing), so that a step is one straight run
        // in which the products of step g + 1 (the last step repeats its own)
        // are in flight during the softmax of step g. The loop is unrolled
        // by two so that the two score buffers trade roles instead of being
        // copied.
        auto step = [&](int g, f32x4_t (&st_cur)[2][NC], f32x4_t (&st_nxt)[2][NC]) __attribute__((always_inline)) {
            const int g1 = g + 1;
            if (g1 < nsteps && g1 % SPT == 0) {
                // step g + 1 starts tile t1: wait for it, then reuse the
                // buffer of tile t1 - 1 (its last operands are in registers)
                // for tile t1 + 1
                const int t1 = g1 / SPT;
                if (!big && tid < SH::TBL) tbl[((t1 + 1) & 1) * SH::TBL + tid] = clamp_pid(treg);
                __syncthreads();
                if (t1 + 1 < nkt) issue(t1 + 1, (t1 + 1) & 1, treg);
                treg = lookup(min(t1 + 2, nkt - 1));
            }
            const int gn = g1 < nsteps ? g1 : g;
            mask(g, st_cur);
            u32x4 kf[2][NK];
            read_k(gn, kf);
            qk(kf, st_nxt);
            u32x4 pb[NC];
            float tl[NC];
            bool need_any;
            softmax(st_cur, pb, tl, need_any);
            if (__any(need_any)) rescale(st_cur, pb, tl);
            pv(g, vf, pb);
            read_v(gn, vf);
        };
        for (int g = 0; g < nsteps; g += 2) {
            step(g, st_a, st_b);
            if (g + 1 < nsteps) step(g + 1, st_b, st_a);
        }
    }

    // ---- normalise and store: acc[n][v][r] = O^T[d = 16v + 4j + r][column r16
    // of block n]; the denominator of column r16 is row 0 of accl[n], held by
    // lane (r16, j = 0)
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const float l = column_sum(j == 0 ? accl[n][0] : 0.f);
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

// ---------------------------------------------------------------------------
// float32 prefill
// ---------------------------------------------------------------------------
//
// The same work decomposition, tile loads and online softmax as the 16-bit
// kernel, on v_mfma_f32_16x16x4_f32. A lane reads 16-byte operand chunks (4
// floats) and spends them on four products whose k index j stands for the
// chunk's component: S^T = K Q^T over d = 16c + 4j + comp takes D/4 products
// per 16x16 tile, and after the softmax the lane's four scores -- keys 4j+r,
// r = 0..3, of column r16 -- are, one per product, the B operand of
// O^T += V^T P^T over those keys, whose A operand component r is a plain
// 16-byte read of the cache's V tile [D][16]. Probabilities stay in float32,
// so the denominator is a plain sum. Steps are 16 keys; tiles 32 keys (16 at
// head_dim 256).

template <int D>
struct PrefillShapeF32 {
    static constexpr int NC = D >= 256 ? 1 : 2;    // 16-column blocks per wave
    static constexpr int KT = D >= 256 ? 16 : 32;   // keys per LDS tile
    static constexpr int ROWB = D * 4;              // bytes of one K row
    static constexpr int K_BYTES = KT * ROWB;
    static constexpr int V_BYTES = KT * ROWB;
    static constexpr int BUF_BYTES = K_BYTES + V_BYTES;
    static constexpr int UK = K_BYTES / 1024 / kWaves;  // 16-byte loads per lane and tile
    static constexpr int UV = V_BYTES / 1024 / kWaves;
    static constexpr int TBL = 16;
    static_assert(UK * kWaves * 1024 == K_BYTES && UV * kWaves * 1024 == V_BYTES, "whole loads");
};

template <int D>
constexpr int prefill_query_tile_f32(int g) { return kWaves * 16 * PrefillShapeF32<D>::NC / g; }

template <int D>
constexpr size_t prefill_smem_f32() {
    return 2 * static_cast<size_t>(PrefillShapeF32<D>::BUF_BYTES) + 2 * PrefillShapeF32<D>::TBL * sizeof(int);
}

__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int D, int G>
__global__ __launch_bounds__(kThreads) void pa_prefill_f32(PrefillParams p) {
    static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "group size");
    using SH = PrefillShapeF32<D>;
    constexpr int NC = SH::NC, KT = SH::KT, ROWB = SH::ROWB;
    constexpr int NQ = D / 16;          // 16-byte chunks of a row per lane (d = 16c + 4j + comp)
    constexpr int NV = D / 16;          // 16-row blocks of O^T
    constexpr int TPW = 16 * NC / G;
    constexpr int QT = kWaves * TPW;
    constexpr float kLazy = 8.f;
    constexpr float kFloor = -1e30f;

    extern __shared__ __align__(16) unsigned char lds[];
    int* tbl = reinterpret_cast<int*>(lds + 2 * SH::BUF_BYTES);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, j = lane >> 4;

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
    const int e_lo = kq * QT;
    if (e_lo >= M) return;
    const int nrow = min(M - e_lo, QT);
    const int pos0 = L - e_lo - nrow;
    const int row0 = q1 - e_lo - nrow;
    const int nkeys = max(0, L - e_lo);
    const int nkt = (nkeys + KT - 1) / KT;
    const int uw0 = wave * TPW;
    const int uw1 = min(uw0 + TPW, nrow);
    const int pw_min = pos0 + uw0;
    const int pw_max = uw1 > uw0 ? pos0 + uw1 - 1 : -1;

    const int hq = p.num_heads;
    const uint32_t qsign = p.scale_log2 < 0.f ? 0x80000000u : 0u;
    const float sc = fmaxf(fabsf(p.scale_log2), 1e-30f);
    f32x4_t qf[NC][NQ];
    int pcol[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const int c = 16 * n + r16;
        const int u = min(uw0 + c / G, nrow - 1);
        const int h = kv * G + c % G;
        pcol[n] = pos0 + u;
        const float* qrow = static_cast<const float*>(p.q) + (static_cast<size_t>(row0 + u) * hq + h) * D + 4 * j;
#pragma unroll
        for (int c2 = 0; c2 < NQ; ++c2)
            qf[n][c2] = __builtin_bit_cast(f32x4_t, *reinterpret_cast<const u32x4*>(qrow + 16 * c2) ^ qsign);
    }
    f32x4_t acc[NC][NV];
    float m_run[NC], lsum[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        m_run[n] = kFloor;
        lsum[n] = 0.f;
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[n][v] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    if (nkt > 0) {
        const int lb = p.log2_bs;
        const int bs = 1 << lb;
        const int lvt = p.log2_vt;
        const int vt = 1 << lvt;
        const int hkv = p.num_kv_heads;
        const size_t blk_el = static_cast<size_t>(bs) * D;
        const char* kbase = static_cast<const char*>(p.k_cache);
        const char* vbase = static_cast<const char*>(p.v_cache);
        const int* trow = p.block_tables + static_cast<size_t>(s) * p.max_blocks;
        const int lastk = L - 1;
        const int last_blk = lastk >> lb;
        const int ntb = KT >= bs ? KT >> lb : 1;
        auto clamp_pid = [&](int pid) { return pid < 0 ? 0 : (pid >= p.num_blocks ? p.num_blocks - 1 : pid); };
        auto lookup = [&](int kt) {
            const int e = min(((kt * KT) >> lb) + tid, last_blk);
            return trow[tid < ntb ? e : 0];
        };
        auto head_el = [&](int pid) { return (static_cast<size_t>(pid) * hkv + kv) * blk_el; };

        // LDS: K rows in key order, 16-byte chunk ch of row r at ch ^ (r & 15);
        // V as the cache's 16-key tiles [D][16], chunk c4 (keys 4 c4 .. + 3)
        // of row d at c4 ^ ((d >> 2) & 3). Keys past the context are read at
        // the last key (masked).
        auto issue = [&](int kt, int buf) {
            unsigned char* bk = lds + buf * SH::BUF_BYTES;
            unsigned char* bv = bk + SH::K_BYTES;
            const int* tb = tbl + (kt & 1) * SH::TBL;
            const int t0 = kt * KT;
            const int blk0 = t0 >> lb;
#pragma unroll
            for (int i = 0; i < SH::UK; ++i) {
                const int P = (wave * SH::UK + i) * 1024 + lane * 16;
                const int r = P / ROWB;
                const int ch = ((P % ROWB) >> 4) ^ (r & 15);
                const int key = min(t0 + r, lastk);
                const int pid = tb[(key >> lb) - blk0];
                const char* src = kbase + (head_el(pid) + static_cast<size_t>(key & (bs - 1)) * D) * 4 + ch * 16;
                dma<16>(src, bk + (wave * SH::UK + i) * 1024);
            }
#pragma unroll
            for (int i = 0; i < SH::UV; ++i) {
                const int P = (wave * SH::UV + i) * 1024 + lane * 16;
                const int sub = P / (D * 64);
                const int d = (P % (D * 64)) >> 6;
                const int c4 = ((P >> 4) & 3) ^ ((d >> 2) & 3);
                const int key = min(t0 + 16 * sub + 4 * c4, lastk & ~3);
                const int pid = tb[(key >> lb) - blk0];
                const int off = key & (bs - 1);
                const size_t el = head_el(pid) + static_cast<size_t>(off >> lvt) * D * vt + static_cast<size_t>(d) * vt +
                                  (off & (vt - 1));
                dma<16>(vbase + el * 4, bv + (wave * SH::UV + i) * 1024);
            }
        };

        auto compute = [&](int kt, int buf) {
            const unsigned char* bk = lds + buf * SH::BUF_BYTES;
            const unsigned char* bv = bk + SH::K_BYTES;
#pragma unroll
            for (int st16 = 0; st16 < KT / 16; ++st16) {
                const int tok0 = kt * KT + 16 * st16;
                if (tok0 > pw_max) break;  // uniform
                const int r = 16 * st16 + r16;
                const unsigned char* krow = bk + r * ROWB;
                f32x4_t st[NC];
#pragma unroll
                for (int n = 0; n < NC; ++n) st[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < NQ; ++c) {
                    const f32x4_t kf = *reinterpret_cast<const f32x4_t*>(krow + (((4 * c + j) ^ (r & 15)) << 4));
#pragma unroll
                    for (int n = 0; n < NC; ++n)
#pragma unroll
                        for (int comp = 0; comp < 4; ++comp) st[n] = mfma_f32(kf[comp], qf[n][c][comp], st[n]);
                }
                // st[n][rr] is the unscaled logit of key tok0 + 4j + rr, column r16
                if (tok0 + 15 > pw_min) {
#pragma unroll
                    for (int n = 0; n < NC; ++n)
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr)
                            if (tok0 + 4 * j + rr > pcol[n]) st[n][rr] = -INFINITY;
                }
                float tmax[NC];
                bool need_any = false;
#pragma unroll
                for (int n = 0; n < NC; ++n) {
                    tmax[n] = column_max(max3(max3(st[n][0], st[n][1], st[n][2]), st[n][3], -INFINITY)) * sc;
                    need_any |= tmax[n] > m_run[n] + kLazy;
                }
                if (__any(need_any)) {
#pragma unroll
                    for (int n = 0; n < NC; ++n) {
                        const float mn = tmax[n] > m_run[n] + kLazy ? tmax[n] : m_run[n];
                        const float alpha = fast_exp2(m_run[n] - mn);
#pragma unroll
                        for (int v = 0; v < NV; ++v) acc[n][v] *= alpha;
                        lsum[n] *= alpha;
                        m_run[n] = mn;
                    }
                }
                f32x4_t pr[NC];
#pragma unroll
                for (int n = 0; n < NC; ++n) {
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) pr[n][rr] = fast_exp2(fmaf(st[n][rr], sc, -m_run[n]));
                    lsum[n] += (pr[n][0] + pr[n][1]) + (pr[n][2] + pr[n][3]);
                }
                // V^T rows d = 16v + r16, keys tok0 + 4j .. + 3 (chunk j of row d
                // of 16-key tile st16); keys past the context are zeroed
                const unsigned char* vrow = bv + (st16 * D + r16) * 64 + ((j ^ ((r16 >> 2) & 3)) << 4);
                const int nv = L - (tok0 + 4 * j);
                const bool vmask = tok0 + 16 > L;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    f32x4_t vf = *reinterpret_cast<const f32x4_t*>(vrow + 16 * v * 64);
                    if (vmask) {
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) vf[rr] = nv > rr ? vf[rr] : 0.f;
                    }
#pragma unroll
                    for (int n = 0; n < NC; ++n)
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) acc[n][v] = mfma_f32(vf[rr], pr[n][rr], acc[n][v]);
                }
            }
        };

        if (tid < SH::TBL) tbl[tid] = clamp_pid(lookup(0));
        __syncthreads();
        issue(0, 0);
        {
            const int t1 = lookup(min(1, nkt - 1));
            if (tid < SH::TBL) tbl[SH::TBL + tid] = clamp_pid(t1);
        }
        __syncthreads();
        for (int kt = 0; kt < nkt; ++kt) {
            if (kt + 1 < nkt) issue(kt + 1, (kt + 1) & 1);
            const int tnext = lookup(min(kt + 2, nkt - 1));
            compute(kt, kt & 1);
            if (tid < SH::TBL) tbl[(kt & 1) * SH::TBL + tid] = clamp_pid(tnext);
            __syncthreads();
        }
    }

#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const float l = column_sum(lsum[n]);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const int c = 16 * n + r16;
        const int u = uw0 + c / G;
        if (u < nrow) {
            const int h = kv * G + c % G;
            float* orow = static_cast<float*>(p.out) + (static_cast<size_t>(row0 + u) * hq + h) * D + 4 * j;
#pragma unroll
            for (int v = 0; v < NV; ++v) *reinterpret_cast<f32x4_t*>(orow + 16 * v) = acc[n][v] * inv;
        }
    }
}

template <int D, int G>
hipError_t launch_prefill_f32_g(const PrefillParams& p, hipStream_t stream) {
    constexpr int QT = prefill_query_tile_f32<D>(G);
    const long long qtiles = (static_cast<long long>(p.max_q) + QT - 1) / QT;
    const long long grid = qtiles * p.num_seqs * p.num_kv_heads;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    return launch_kernel(pa_prefill_f32<D, G>, dim3(static_cast<unsigned>(grid)), dim3(kThreads),
                         prefill_smem_f32<D>(), stream, p);
}

template <int D>
hipError_t launch_prefill_f32_d(const PrefillParams& p, int group, hipStream_t stream) {
    switch (group) {
        case 1: return launch_prefill_f32_g<D, 1>(p, stream);
        case 2: return launch_prefill_f32_g<D, 2>(p, stream);
        case 4: return launch_prefill_f32_g<D, 4>(p, stream);
        case 8: return launch_prefill_f32_g<D, 8>(p, stream);
        case 16: return launch_prefill_f32_g<D, 16>(p, stream);
    }
    return hipErrorInvalidValue;
}

template <int DT, int D, int G>
hipError_t launch_prefill_g(const PrefillParams& p, hipStream_t stream) {
    constexpr int QT = prefill_query_tile<D>(G);
    const long long qtiles = (static_cast<long long>(p.max_q) + QT - 1) / QT;
    const long long grid = qtiles * p.num_seqs * p.num_kv_heads;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    return launch_kernel(pa_prefill_mfma<DT, D, G>, dim3(static_cast<unsigned>(grid)), dim3(kThreads),
                         prefill_smem<D>(), stream, p);
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
    if (dt != PA_BF16 && dt != PA_F16 && dt != PA_F32) return false;
    if (!(head_dim == 64 || head_dim == 128 || head_dim == 256)) return false;
    return group == 1 || group == 2 || group == 4 || group == 8 || group == 16;
}

hipError_t launch_prefill(const PrefillParams& p, pa_dtype_t dt, int head_dim, int group, hipStream_t stream) {
    switch (dt) {
        case PA_BF16: return launch_prefill_dt<PA_BF16>(p, head_dim, group, stream);
        case PA_F16: return launch_prefill_dt<PA_F16>(p, head_dim, group, stream);
        case PA_F32:
            switch (head_dim) {
                case 64: return launch_prefill_f32_d<64>(p, group, stream);
                case 128: return launch_prefill_f32_d<128>(p, group, stream);
                case 256: return launch_prefill_f32_d<256>(p, group, stream);
            }
            break;
        default: break;
    }
    return hipErrorInvalidValue;
}

}  // namespace pa
