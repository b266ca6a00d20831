// Host-side block manager (include/pa_blocks.h): block tables, reference
// counts, the free list, slot reservation and copy-on-write pairs. Host code
// only; the device path receives what it produces as plain int32 arrays.
//
// Allocation on demand (aiqz.cc tutorial, section 分页核心思想), prefix
// sharing by reference count and copy-on-write on the first write into a
// shared block (section 前缀共享机制; cf-1.com blog 4.2), release at count
// zero (cf-1.com 3.2) and the consistency check (cf-1.com 4.3).

#include <algorithm>
#include <deque>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pa.h"
#include "pa_blocks.h"
#include "pa_internal.h"

struct pa_block_manager {
    struct Seq {
        std::vector<int32_t> blocks;
        int64_t tokens = 0;
    };
    int num_blocks = 0;
    int block_size = 0;
    std::vector<int32_t> refs;
    std::deque<int32_t> free;
    std::unordered_map<int64_t, Seq> seqs;

    int32_t take() {  // caller has checked that a block is free
        const int32_t pid = free.front();
        free.pop_front();
        refs[pid] += 1;
        return pid;
    }
    void drop(int32_t pid) {
        refs[pid] -= 1;
        if (refs[pid] == 0) free.push_back(pid);
    }
    int64_t blocks_for(int64_t tokens) const { return (tokens + block_size - 1) / block_size; }
};

using pa::fail;

namespace {

pa_status_t null_manager() { return fail(PA_ERR_INVALID_ARG, "null block manager"); }

}  // namespace

extern "C" {

pa_status_t pa_bm_create(int num_blocks, int block_size, const int32_t* free_order,
                         pa_block_manager_t** out) {
    if (!out) return fail(PA_ERR_INVALID_ARG, "null output pointer");
    *out = nullptr;
    if (num_blocks <= 0 || block_size <= 0)
        return fail(PA_ERR_INVALID_ARG, "invalid size (num_blocks=%d block_size=%d)", num_blocks, block_size);
    if (static_cast<int64_t>(num_blocks) * block_size > INT32_MAX)
        return fail(PA_ERR_INVALID_ARG, "num_blocks * block_size = %lld slots do not fit the int32 slot mapping",
                    static_cast<long long>(num_blocks) * block_size);
    pa_block_manager* bm = new (std::nothrow) pa_block_manager;
    if (!bm) return fail(PA_ERR_INVALID_ARG, "out of host memory");
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->refs.assign(num_blocks, 0);
    if (free_order) {
        std::vector<char> seen(num_blocks, 0);
        for (int i = 0; i < num_blocks; ++i) {
            const int32_t b = free_order[i];
            if (b < 0 || b >= num_blocks || seen[b]) {
                delete bm;
                return fail(PA_ERR_INVALID_ARG, "free_order is not a permutation of [0, %d)", num_blocks);
            }
            seen[b] = 1;
            bm->free.push_back(b);
        }
    } else {
        for (int i = 0; i < num_blocks; ++i) bm->free.push_back(i);
    }
    *out = bm;
    return PA_OK;
}

void pa_bm_destroy(pa_block_manager_t* bm) { delete bm; }

pa_status_t pa_bm_prefill(pa_block_manager_t* bm, int64_t seq, int num_tokens) {
    if (!bm) return null_manager();
    if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "negative token count %d", num_tokens);
    if (bm->seqs.count(seq)) return fail(PA_ERR_INVALID_ARG, "sequence %lld exists", static_cast<long long>(seq));
    const int64_t need = bm->blocks_for(num_tokens);
    if (need > static_cast<int64_t>(bm->free.size()))
        return fail(PA_ERR_NO_BLOCKS, "prefill of %d tokens needs %lld blocks, %zu free", num_tokens,
                    static_cast<long long>(need), bm->free.size());
    pa_block_manager::Seq s;
    s.tokens = num_tokens;
    s.blocks.reserve(need);
    for (int64_t i = 0; i < need; ++i) s.blocks.push_back(bm->take());
    bm->seqs.emplace(seq, std::move(s));
    return PA_OK;
}

pa_status_t pa_bm_share(pa_block_manager_t* bm, int64_t seq, int64_t src, int num_tokens) {
    if (!bm) return null_manager();
    if (bm->seqs.count(seq)) return fail(PA_ERR_INVALID_ARG, "sequence %lld exists", static_cast<long long>(seq));
    auto it = bm->seqs.find(src);
    if (it == bm->seqs.end()) return fail(PA_ERR_INVALID_ARG, "unknown sequence %lld", static_cast<long long>(src));
    if (num_tokens < 0 || num_tokens > it->second.tokens)
        return fail(PA_ERR_INVALID_ARG, "cannot share %d tokens of a sequence holding %lld", num_tokens,
                    static_cast<long long>(it->second.tokens));
    pa_block_manager::Seq s;
    s.tokens = num_tokens;
    s.blocks.assign(it->second.blocks.begin(), it->second.blocks.begin() + bm->blocks_for(num_tokens));
    for (int32_t pid : s.blocks) bm->refs[pid] += 1;
    bm->seqs.emplace(seq, std::move(s));
    return PA_OK;
}

pa_status_t pa_bm_append(pa_block_manager_t* bm, const int64_t* seqs, int n, int32_t* slots, int32_t* pairs,
                         int* num_pairs) {
    if (!bm) return null_manager();
    if (n < 0) return fail(PA_ERR_INVALID_ARG, "negative batch size %d", n);
    if (num_pairs) *num_pairs = 0;
    if (n == 0) return PA_OK;
    if (!seqs || !slots || !pairs || !num_pairs) return fail(PA_ERR_INVALID_ARG, "null pointer argument");
    // validate and count the blocks the batch takes, without changing anything
    std::unordered_set<int64_t> seen;
    std::unordered_map<int32_t, int32_t> refs_after;  // reference counts the batch has changed so far
    int64_t need = 0;
    for (int i = 0; i < n; ++i) {
        auto it = bm->seqs.find(seqs[i]);
        if (it == bm->seqs.end())
            return fail(PA_ERR_INVALID_ARG, "unknown sequence %lld", static_cast<long long>(seqs[i]));
        if (!seen.insert(seqs[i]).second)
            return fail(PA_ERR_INVALID_ARG, "sequence %lld appears twice in one batch", static_cast<long long>(seqs[i]));
        const auto& s = it->second;
        if (s.tokens % bm->block_size == 0) {
            ++need;
        } else {
            const int32_t last = s.blocks.back();
            auto r = refs_after.find(last);
            const int32_t ref = r == refs_after.end() ? bm->refs[last] : r->second;
            if (ref > 1) {
                ++need;
                refs_after[last] = ref - 1;
            }
        }
    }
    if (need > static_cast<int64_t>(bm->free.size()))
        return fail(PA_ERR_NO_BLOCKS, "the batch needs %lld new blocks, %zu free", static_cast<long long>(need),
                    bm->free.size());
    int np = 0;
    for (int i = 0; i < n; ++i) {
        auto& s = bm->seqs[seqs[i]];
        const int pos = static_cast<int>(s.tokens % bm->block_size);
        if (pos == 0) {
            s.blocks.push_back(bm->take());
        } else {
            const int32_t last = s.blocks.back();
            if (bm->refs[last] > 1) {
                const int32_t fresh = bm->take();
                s.blocks.back() = fresh;
                bm->drop(last);
                pairs[2 * np] = last;
                pairs[2 * np + 1] = fresh;
                ++np;
            }
        }
        s.tokens += 1;
        slots[i] = s.blocks.back() * bm->block_size + pos;
    }
    *num_pairs = np;
    return PA_OK;
}

pa_status_t pa_bm_free(pa_block_manager_t* bm, int64_t seq) {
    if (!bm) return null_manager();
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end()) return fail(PA_ERR_INVALID_ARG, "unknown sequence %lld", static_cast<long long>(seq));
    const std::vector<int32_t> blocks = std::move(it->second.blocks);
    bm->seqs.erase(it);  // the mapping goes first, then the references
    for (int32_t pid : blocks) bm->drop(pid);
    return PA_OK;
}

pa_status_t pa_bm_block_tables(const pa_block_manager_t* bm, const int64_t* seqs, int n, int32_t* tables,
                               int max_blocks, int32_t pad, int32_t* context_lens) {
    if (!bm) return null_manager();
    if (n < 0 || max_blocks < 0) return fail(PA_ERR_INVALID_ARG, "negative size");
    if (n > 0 && (!seqs || !context_lens || (max_blocks > 0 && !tables)))
        return fail(PA_ERR_INVALID_ARG, "null pointer argument");
    for (int i = 0; i < n; ++i) {
        auto it = bm->seqs.find(seqs[i]);
        if (it == bm->seqs.end())
            return fail(PA_ERR_INVALID_ARG, "unknown sequence %lld", static_cast<long long>(seqs[i]));
        if (static_cast<int64_t>(it->second.blocks.size()) > max_blocks)
            return fail(PA_ERR_INVALID_ARG, "sequence %lld holds %zu blocks, more than max_blocks %d",
                        static_cast<long long>(seqs[i]), it->second.blocks.size(), max_blocks);
        if (it->second.tokens > INT32_MAX)
            return fail(PA_ERR_INVALID_ARG, "sequence %lld is longer than int32", static_cast<long long>(seqs[i]));
    }
    for (int i = 0; i < n; ++i) {
        const auto& s = bm->seqs.at(seqs[i]);
        int32_t* row = tables + static_cast<size_t>(i) * max_blocks;
        std::copy(s.blocks.begin(), s.blocks.end(), row);
        std::fill(row + s.blocks.size(), row + max_blocks, pad);
        context_lens[i] = static_cast<int32_t>(s.tokens);
    }
    return PA_OK;
}

int pa_bm_num_free(const pa_block_manager_t* bm) { return bm ? static_cast<int>(bm->free.size()) : -1; }

int pa_bm_blocks_in_use(const pa_block_manager_t* bm) {
    return bm ? bm->num_blocks - static_cast<int>(bm->free.size()) : -1;
}

int pa_bm_refcount(const pa_block_manager_t* bm, int block) {
    if (!bm || block < 0 || block >= bm->num_blocks) return -1;
    return bm->refs[block];
}

int64_t pa_bm_seq_tokens(const pa_block_manager_t* bm, int64_t seq) {
    if (!bm) return -1;
    auto it = bm->seqs.find(seq);
    return it == bm->seqs.end() ? -1 : it->second.tokens;
}

int64_t pa_bm_blocks_without_sharing(const pa_block_manager_t* bm) {
    if (!bm) return -1;
    int64_t total = 0;
    for (const auto& kv : bm->seqs) total += bm->blocks_for(kv.second.tokens);
    return total;
}

pa_status_t pa_bm_check(const pa_block_manager_t* bm) {
    if (!bm) return null_manager();
    std::vector<int32_t> counts(bm->num_blocks, 0);
    for (const auto& kv : bm->seqs) {
        if (static_cast<int64_t>(kv.second.blocks.size()) != bm->blocks_for(kv.second.tokens))
            return fail(PA_ERR_INVALID_ARG, "sequence %lld: %zu blocks for %lld tokens",
                        static_cast<long long>(kv.first), kv.second.blocks.size(),
                        static_cast<long long>(kv.second.tokens));
        for (int32_t pid : kv.second.blocks) counts[pid] += 1;
    }
    std::vector<char> on_free(bm->num_blocks, 0);
    for (int32_t pid : bm->free) {
        if (on_free[pid]) return fail(PA_ERR_INVALID_ARG, "block %d is on the free list twice", pid);
        on_free[pid] = 1;
    }
    for (int b = 0; b < bm->num_blocks; ++b) {
        if (counts[b] != bm->refs[b])
            return fail(PA_ERR_INVALID_ARG, "block %d: reference count %d, named by %d table entries", b,
                        bm->refs[b], counts[b]);
        if ((bm->refs[b] == 0) != (on_free[b] != 0))
            return fail(PA_ERR_INVALID_ARG, "block %d: reference count %d but %s the free list", b, bm->refs[b],
                        on_free[b] ? "on" : "not on");
    }
    return PA_OK;
}

}  // extern "C"
