"""Host-side input generation: the block pool against the Python demo of the
aiqz.cc tutorial, and the structure of every synthetic workload. No GPU."""

import json
import math
import os

import numpy as np
import pytest

import workloads as W
from workloads import HostBlockPool, PoolExhausted

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_pool_reproduces_tutorial_demo():
    with open(os.path.join(GOLDEN, "demo_block_manager.json")) as f:
        g = json.load(f)
    pool = HostBlockPool(g["total_blocks"], g["block_size"])
    cows = []
    for step in g["script"]:
        if step[0] == "prefill":
            pool.prefill(step[1], step[2])
        elif step[0] == "share":
            pool.share(step[1], step[2], step[3])
        elif step[0] == "append":
            for _ in range(step[2]):
                _, cow = pool.append_token(step[1])
                if cow:
                    cows.append(list(cow))
    e = g["expected"]
    assert pool.refs == e["refs"]
    assert {k: v for k, v in pool.tables.items()} == e["tables"]
    assert pool.used == e["used_tokens"]
    assert cows == e["cow_pairs"]
    assert pool.blocks_without_sharing() == e["blocks_without_sharing"]
    assert pool.blocks_in_use() == e["blocks_with_sharing"]
    pool.check_consistency()


def test_pool_release_and_exhaustion():
    pool = HostBlockPool(3, 4)
    pool.prefill("a", 9)  # 3 blocks
    with pytest.raises(PoolExhausted):
        pool.prefill("b", 1)
    pool.share("c", "a", 5)
    pool.free_seq("a")
    assert pool.refs == [1, 1, 0]
    pool.check_consistency()
    pool.free_seq("c")
    assert pool.blocks_in_use() == 0
    pool.check_consistency()


def test_consistency_check_catches_leak():
    pool = HostBlockPool(4, 2)
    pool.prefill("a", 3)
    pool._holders[0] += 1  # a lost decrement
    with pytest.raises(AssertionError):
        pool.check_consistency()


def test_pool_batch_is_all_or_nothing_and_copies_for_all_but_the_last_sharer():
    pool = HostBlockPool(6, 4)
    pool.prefill("p", 6)            # blocks 0, 1 (block 1 half full)
    pool.share("a", "p", 6)
    pool.share("b", "p", 6)
    pool.free_seq("p")              # the two samples keep the blocks
    slots, pairs = pool.append_batch(["a", "b"])
    assert pairs == [(1, 2)]                  # the first sharer copies block 1 into block 2
    assert slots == [2 * 4 + 2, 1 * 4 + 2]    # the last one writes in place
    pool.prefill("c", 12)           # 3 of the 3 free blocks left
    before = (pool.refs, pool.tables, pool.used, pool.free)
    pool.append_batch(["a"])        # still room in block 2
    with pytest.raises(PoolExhausted):
        pool.append_batch(["b", "c"])   # c needs a new block: none left
    assert (pool.refs, pool.used["b"], pool.used["c"]) == (before[0], before[2]["b"], before[2]["c"])
    with pytest.raises(ValueError):
        pool.append_batch(["a", "a"])
    pool.check_consistency()


def test_layout_example_workload():
    w = W.build("layout")
    assert w.block_tables.tolist() == [[5, 1, 7]]
    assert w.context_lens.tolist() == [10]
    assert w.writes[0].slots.tolist() == [29]
    assert sorted(w.prefill_slots.tolist()) == [4, 5, 6, 7, 20, 21, 22, 23, 28]


def _check_tables(w):
    b = w.block_size
    for s in range(w.num_seqs):
        L = int(w.context_lens[s])
        n = -(-L // b)
        row = w.block_tables[s]
        assert np.all(row[:n] >= 0) and np.all(row[:n] < w.num_blocks)
        assert np.all(row[n:] == w.trap_block)
        assert w.trap_block not in set(row[:n].tolist())
    live = w.prefill_slots
    assert len(np.unique(live)) == len(live)
    for op in w.writes:
        assert len(np.unique(op.slots)) == len(op.slots)
        assert not np.isin(op.slots, live).any()


@pytest.mark.parametrize("name", ["tiny", "mha7b", "gqa8b", "long"])
def test_private_workloads(name):
    w = W.build(name)
    _check_tables(w)
    b = w.block_size
    used = np.concatenate([w.block_tables[s, : -(-int(L) // b)] for s, L in enumerate(w.context_lens)])
    assert len(np.unique(used)) == len(used)  # no sharing
    # the write step fills each sequence's last position
    for s, slot in enumerate(w.writes[0].slots):
        L = int(w.context_lens[s])
        assert slot == w.block_tables[s, (L - 1) // b] * b + (L - 1) % b
    # blocks are scattered: not laid out in order
    assert np.mean(np.diff(used) == 1) < 0.05


def test_workload_recipes():
    t = W.build("tiny")
    assert t.context_lens.tolist() == [1, 17, 100, 256] and t.num_blocks == 64 and t.dtype == "f32"
    m = W.build("mha7b")
    assert m.num_blocks == 20000 and m.context_lens.min() >= 128 and m.context_lens.max() <= 4096
    g = W.build("gqa8b")
    assert g.context_lens.min() >= 1 and g.context_lens.max() <= 8192
    assert 700 < np.median(g.context_lens) < 1400
    need = sum(-(-int(L) // 16) for L in g.context_lens)
    assert g.num_blocks == math.ceil(1.1 * need)
    lo = W.build("long")
    assert lo.block_size == 32 and lo.context_lens.min() >= 32768 and lo.context_lens.max() <= 131072


def test_prefix_sharing_workload():
    w = W.build("prefix")
    _check_tables(w)
    assert w.num_seqs == 256 and len(w.cow_pairs) == 192
    b = w.block_size
    src, dst = w.cow_pairs[:, 0], w.cow_pairs[:, 1]
    assert len(np.unique(dst)) == 192 and not np.isin(dst, src).any()
    counts = {}
    for s, L in enumerate(w.context_lens):
        for pid in w.block_tables[s, : -(-int(L) // b)]:
            counts[int(pid)] = counts.get(int(pid), 0) + 1
    for p in range(64):
        rows = w.block_tables[4 * p: 4 * p + 4]
        # the 64 full prefix blocks are shared by all four samples
        assert np.all(rows[:, :64] == rows[0, :64])
        assert all(counts[int(x)] == 4 for x in rows[0, :64])
        # block 64 (the partly filled one): three samples hold copies, one the original
        lasts = rows[:, 64].tolist()
        assert len(set(lasts)) == 4
        assert sum(1 for x in lasts if x in set(src.tolist())) == 1
    assert w.refcount_max == 4
    fork = w.writes[0].slots
    assert len(fork) == 256
    for s in range(256):
        L = int(w.context_lens[s])
        assert 1024 + 1 + 1 <= L <= 1024 + 15 + 1 + 512


def test_prefix_sharing_savings_follow_the_tutorial_formula():
    """aiqz.cc tutorial, section 前缀共享机制: M_saved = N_p x B_block x bytes x (R - 1).
    The prefix batch shares each prompt's 64 full blocks among its 4 samples
    (the partly filled 65th is copied by three of them), so N_p = 64 x 64,
    R = 4, and a block of 16 tokens of 8 KV heads x 128 bf16 values is 32 KB
    of K plus 32 KB of V."""
    w = W.build("prefix")
    m = w.sharing_savings()
    assert m["shared_blocks_by_refcount"] == {"4": 64 * 64}
    assert m["block_bytes"] == 2 * 16 * 8 * 128 * 2
    assert m["m_saved_bytes"] == 64 * 64 * 65536 * 3 == m["m_saved_direct_bytes"]
    assert W.build("gqa8b").sharing_savings()["m_saved_bytes"] == 0
