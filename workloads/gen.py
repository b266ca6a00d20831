"""Seeded synthetic workloads for paged decode attention.

This module only generates inputs: context lengths, block tables, slot
mappings, copy-on-write pairs (through ``HostBlockPool``) and N(0, 1) values.
It holds none of the attention arithmetic and is the one module that both the
oracle-side tests and the GPU-side tests/bench draw their inputs from.

Recipes (the shapes are those of the five decode workloads this library is
measured on; numbers in brackets are the seeds):
  tiny      [1651] 4 seqs, ctx {1, 17, 100, 256}, 4 q heads = 4 KV heads, D 64,
            B 16, fp32, scale 1/8, 64-block pool handed out in a seeded random
            order.
  layout    the worked example of the lihaoran.work note: 1 seq, ctx 10, B 4,
            table [5, 1, 7], 8-block pool (fp32, D 64, 4 heads, scale 1/8).
  mha7b     [1652] batch 64, 32/32 heads, D 128, bf16, B 16, ctx uniform in
            [128, 4096], 20000-block pool.
  gqa8b     [1653] batch 256, 32/8 heads, D 128, bf16, B 16, ctx lognormal
            with median 1024 and sigma 1, rounded and clipped to [1, 8192],
            pool 1.1x the blocks needed.
  prefix    [1654] 64 prompts x 4 samples, GQA 32/8, D 128, bf16, B 16. Prompt
            p has 1024 + r_p tokens, r_p uniform in [1, 15], so its last block
            is partly filled; its 4 samples share all of its blocks. Each sample
            then appends one fork token (the first three copy the shared last
            block first, the fourth writes in place) and a tail of U[0, 512]
            tokens in private blocks.
  long      [1655] batch 8, ctx uniform in [32768, 131072], 64/8 heads, D 128,
            bf16, B 32, partitions of 512 tokens, pool 1.1x the blocks needed.
Every sequence except in ``prefix`` holds ctx - 1 prefilled tokens and appends
its last token through the cache-write step. Physical block ids come from a
seeded random permutation of the pool, so blocks are scattered. One unused
block is reserved as a trap: the padding entries of every block table point at
it, and in correctness mode it, every other unused block and every unwritten
slot hold NaN.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from .pool import HostBlockPool

F32 = "f32"
BF16 = "bf16"


@dataclass
class WriteOp:
    slots: np.ndarray          # int32 [n]
    name: str


@dataclass
class Workload:
    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str
    scale: float
    seed: int
    num_blocks: int
    trap_block: int
    block_tables: np.ndarray   # int32 [S, max_blocks]
    context_lens: np.ndarray   # int32 [S]
    prefill_slots: np.ndarray  # int64 [n] slots holding prefilled data
    cow_pairs: np.ndarray      # int32 [n, 2]
    writes: list = field(default_factory=list)
    partition_size: int = 0          # 0 = the library's default
    ctx_recipe: str = ""
    refcount_max: int = 1

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes one decode reads: 2 * ctx * Hkv * D * e per seq."""
        e = 4 if self.dtype == F32 else 2
        return int(2 * int(self.context_lens.astype(np.int64).sum()) * self.num_kv_heads * self.head_dim * e)

    def unique_kv_bytes(self) -> int:
        """K+V bytes of distinct (physical block, slot) pairs one decode reads."""
        e = 4 if self.dtype == F32 else 2
        b = self.block_size
        per_block = {}
        for s in range(self.num_seqs):
            L = int(self.context_lens[s])
            for t in range(0, L, b):
                pid = int(self.block_tables[s, t // b])
                per_block[pid] = max(per_block.get(pid, 0), min(b, L - t))
        return int(2 * sum(per_block.values()) * self.num_kv_heads * self.head_dim * e)

    def sharing_savings(self) -> dict:
        """K+V memory that prefix sharing saves on this batch (one layer).
        The aiqz.cc tutorial (section 前缀共享机制) gives M_saved = N_p x B_block
        x bytes x (R - 1) for N_p blocks shared by R sequences; here it is
        summed over the reference counts the tables show, and checked against
        the direct count: blocks the tables would take without sharing minus
        the distinct blocks they list."""
        e = 4 if self.dtype == F32 else 2
        b = self.block_size
        block_bytes = 2 * b * self.num_kv_heads * self.head_dim * e  # K and V of one block
        counts = {}
        listed = 0
        for s in range(self.num_seqs):
            n = -(-int(self.context_lens[s]) // b)
            listed += n
            for pid in self.block_tables[s, :n]:
                counts[int(pid)] = counts.get(int(pid), 0) + 1
        by_r = {}
        for r in counts.values():
            if r > 1:
                by_r[r] = by_r.get(r, 0) + 1
        formula = sum(n_p * block_bytes * (r - 1) for r, n_p in by_r.items())
        direct = (listed - len(counts)) * block_bytes
        return {"shared_blocks_by_refcount": {str(r): n for r, n in sorted(by_r.items())},
                "block_bytes": block_bytes, "m_saved_bytes": formula, "m_saved_direct_bytes": direct,
                "blocks_listed": listed, "blocks_distinct": len(counts),
                "what": "M_saved = N_p x B_block x bytes x (R - 1) summed over the refcounts R of the shared blocks "
                        "(aiqz.cc tutorial, 前缀共享机制), one layer of K and V; direct = (listed - distinct) blocks"}

    def summary(self) -> dict:
        c = self.context_lens.astype(np.int64)
        return {
            "workload": self.name, "num_seqs": self.num_seqs, "num_heads": self.num_heads,
            "num_kv_heads": self.num_kv_heads, "head_dim": self.head_dim,
            "block_size": self.block_size, "dtype": self.dtype, "seed": self.seed,
            "num_blocks": self.num_blocks, "partition_size": self.partition_size,
            "ctx_recipe": self.ctx_recipe, "ctx_min": int(c.min()), "ctx_median": float(np.median(c)),
            "ctx_mean": float(c.mean()), "ctx_max": int(c.max()), "tokens": int(c.sum()),
            "cow_pairs": int(len(self.cow_pairs)),
            "write_tokens": int(sum(len(w.slots) for w in self.writes)),
        }


# ---------------------------------------------------------------------------
# Builders
# ---------------------------------------------------------------------------

def _finish(name, pool: HostBlockPool, seqs, prefill_slots, cow_pairs, writes, *, num_heads,
            num_kv_heads, head_dim, dtype, scale, seed, trap, partition_size=0, ctx_recipe=""):
    pool.check_consistency()
    lens = np.array([pool.tokens(s) for s in seqs], dtype=np.int32)
    bs = pool.block_size
    width = max(1, max(-(-int(L) // bs) for L in lens))
    tables = np.full((len(seqs), width), trap, dtype=np.int32)
    for i, s in enumerate(seqs):
        t = pool.blocks_of(s)
        assert len(t) == -(-int(lens[i]) // bs)
        tables[i, :len(t)] = t
    if trap in set(np.asarray(tables[tables != trap]).tolist()):
        raise AssertionError("trap block is in use")
    return Workload(
        name=name, num_seqs=len(seqs), num_heads=num_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, block_size=bs, dtype=dtype, scale=scale, seed=seed,
        num_blocks=pool.num_blocks, trap_block=trap, block_tables=tables, context_lens=lens,
        prefill_slots=np.array(sorted(prefill_slots), dtype=np.int64),
        cow_pairs=np.array(cow_pairs, dtype=np.int32).reshape(-1, 2),
        writes=writes, partition_size=partition_size, ctx_recipe=ctx_recipe,
        refcount_max=max(pool.refs) if pool.num_blocks else 0,
    )


def _prefill_then_append(name, lens, *, block_size, num_blocks, seed, rng, **kw):
    """Each sequence prefills ctx - 1 tokens and appends its last token."""
    lens = [int(x) for x in lens]
    if num_blocks is None:
        need = sum(-(-L // block_size) for L in lens)
        num_blocks = int(math.ceil(1.1 * need))
        if num_blocks == need:
            num_blocks += 1
    order = rng.permutation(num_blocks)
    pool = HostBlockPool(num_blocks, block_size, free_order=order)
    prefill_slots = []
    slots = []
    for i, L in enumerate(lens):
        if L <= 0:
            raise ValueError("every sequence of these workloads has at least one token")
        blocks = pool.prefill(i, L - 1)
        for t in range(L - 1):
            prefill_slots.append(blocks[t // block_size] * block_size + t % block_size)
        slot, cow = pool.append_token(i)
        assert cow is None
        slots.append(slot)
    trap = pool.free[-1]
    return _finish(name, pool, list(range(len(lens))), prefill_slots, [],
                   [WriteOp(np.array(slots, dtype=np.int32), "last_token")], seed=seed, trap=trap, **kw)


def tiny() -> Workload:
    seed = 1651
    rng = np.random.default_rng(seed)
    return _prefill_then_append("tiny", [1, 17, 100, 256], block_size=16, num_blocks=64, seed=seed,
                                rng=rng, num_heads=4, num_kv_heads=4, head_dim=64, dtype=F32,
                                scale=1.0 / 8.0, ctx_recipe="fixed {1,17,100,256}")


def layout_example() -> Workload:
    """The [5, 1, 7] example: 10 cached positions, B = 4, 8-block pool."""
    bs = 4
    table = [5, 1, 7]
    prefill = [table[t // bs] * bs + t % bs for t in range(9)]
    slot = table[9 // bs] * bs + 9 % bs  # position 9 -> block 7, offset 1 -> slot 29
    return Workload(
        name="layout", num_seqs=1, num_heads=4, num_kv_heads=4, head_dim=64, block_size=bs,
        dtype=F32, scale=1.0 / 8.0, seed=1650, num_blocks=8, trap_block=0,
        block_tables=np.array([table], dtype=np.int32), context_lens=np.array([10], dtype=np.int32),
        prefill_slots=np.array(prefill, dtype=np.int64), cow_pairs=np.zeros((0, 2), np.int32),
        writes=[WriteOp(np.array([slot], dtype=np.int32), "last_token")], ctx_recipe="fixed 10",
    )


def mha7b() -> Workload:
    seed = 1652
    rng = np.random.default_rng(seed)
    lens = rng.integers(128, 4096, size=64, endpoint=True)
    return _prefill_then_append("mha7b", lens, block_size=16, num_blocks=20000, seed=seed, rng=rng,
                                num_heads=32, num_kv_heads=32, head_dim=128, dtype=BF16,
                                scale=1.0 / math.sqrt(128), ctx_recipe="uniform [128, 4096]")


def gqa8b_lengths(rng, n=256, median=1024, sigma=1.0, cap=8192):
    x = np.exp(rng.normal(math.log(median), sigma, size=n))
    return np.clip(np.rint(x), 1, cap).astype(np.int64)


def gqa8b(block_size: int = 16) -> Workload:
    """The batch-256 GQA workload; ``block_size`` other than 16 gives the
    same sequences paged with another block size (block-size sweep)."""
    seed = 1653
    rng = np.random.default_rng(seed)
    lens = gqa8b_lengths(rng)
    return _prefill_then_append("gqa8b", lens, block_size=block_size, num_blocks=None, seed=seed, rng=rng,
                                num_heads=32, num_kv_heads=8, head_dim=128, dtype=BF16,
                                scale=1.0 / math.sqrt(128),
                                ctx_recipe="lognormal median 1024 sigma 1, clipped to [1, 8192]")


def long_context() -> Workload:
    seed = 1655
    rng = np.random.default_rng(seed)
    lens = rng.integers(32768, 131072, size=8, endpoint=True)
    return _prefill_then_append("long", lens, block_size=32, num_blocks=None, seed=seed, rng=rng,
                                num_heads=64, num_kv_heads=8, head_dim=128, dtype=BF16,
                                scale=1.0 / math.sqrt(128), partition_size=512,
                                ctx_recipe="uniform [32768, 131072]")


def _prefix_script(pool: HostBlockPool, prompts, tails, samples):
    """Run the prefix-sharing script on ``pool``; returns bookkeeping."""
    bs = pool.block_size
    prefill_slots, cow_pairs, fork_slots, tail_slots, seqs = [], [], [], [], []
    for p, plen in enumerate(prompts):
        root = ("prompt", p)
        blocks = pool.prefill(root, plen)
        for t in range(plen):
            prefill_slots.append(blocks[t // bs] * bs + t % bs)
        for j in range(samples):
            pool.share((p, j), root, plen)
        pool.free_seq(root)  # the prompt itself does not decode; its samples hold the blocks
    for p in range(len(prompts)):
        for j in range(samples):
            slot, cow = pool.append_token((p, j))
            fork_slots.append(slot)
            if cow is not None:
                cow_pairs.append(cow)
    for p in range(len(prompts)):
        for j in range(samples):
            s = (p, j)
            for _ in range(int(tails[p * samples + j])):
                slot, cow = pool.append_token(s)
                assert cow is None
                tail_slots.append(slot)
            seqs.append(s)
    return prefill_slots, cow_pairs, fork_slots, tail_slots, seqs


def prefix_sharing() -> Workload:
    seed = 1654
    rng = np.random.default_rng(seed)
    n_prompts, samples, bs = 64, 4, 16
    prompts = (1024 + rng.integers(1, 15, size=n_prompts, endpoint=True)).tolist()
    tails = rng.integers(0, 512, size=n_prompts * samples, endpoint=True).tolist()
    # dry run on an unbounded pool to size the real one
    dry = HostBlockPool(10 ** 7, bs)
    _prefix_script(dry, prompts, tails, samples)
    need = dry.allocations
    num_blocks = int(math.ceil(1.1 * need))
    pool = HostBlockPool(num_blocks, bs, free_order=rng.permutation(num_blocks))
    prefill_slots, cow_pairs, fork_slots, tail_slots, seqs = _prefix_script(pool, prompts, tails, samples)
    trap = pool.free[-1]
    w = _finish("prefix", pool, seqs, prefill_slots, cow_pairs,
                [WriteOp(np.array(fork_slots, dtype=np.int32), "fork_token"),
                 WriteOp(np.array(tail_slots, dtype=np.int32), "tails")],
                num_heads=32, num_kv_heads=8, head_dim=128, dtype=BF16,
                scale=1.0 / math.sqrt(128), seed=seed, trap=trap,
                ctx_recipe="1024 + U[1,15] prompt, 1 fork token, tail U[0,512]")
    # reference count of the shared full prefix blocks at decode time
    counts = {}
    for row, L in zip(w.block_tables, w.context_lens):
        for pid in row[: -(-int(L) // bs)]:
            counts[int(pid)] = counts.get(int(pid), 0) + 1
    w.refcount_max = max(counts.values())
    return w


BUILDERS = {
    "tiny": tiny,
    "layout": layout_example,
    "mha7b": mha7b,
    "gqa8b": gqa8b,
    "prefix": prefix_sharing,
    "long": long_context,
}


def build(name: str, **kw) -> Workload:
    return BUILDERS[name](**kw)


def tail_waste(w: Workload) -> float:
    """Fraction of allocated slots past the context ends: the empty tail of
    each sequence's last block, over all allocated slots."""
    b = w.block_size
    alloc = (-(-w.context_lens.astype(np.int64) // b)) * b
    return float((alloc - w.context_lens).sum() / alloc.sum()) if alloc.sum() else 0.0


# ---------------------------------------------------------------------------
# Values
# ---------------------------------------------------------------------------

def v_tile(block_size: int) -> int:
    """Tokens per transposed V tile of the cache layout: min(block_size, 16)."""
    return min(block_size, 16)


def make_values(w: Workload, device="cpu", poison=True):
    """Seeded N(0, 1) values as torch tensors on ``device``.

    Returns a dict with q [S, Hq, D], k_cache [NB, Hkv, B, D], v_cache in the
    transposed tile layout [NB, Hkv, B // T, D, T] (T = min(B, 16)) and, per
    write op, k / v rows [n, Hkv, D]. Values are drawn in float32 and rounded
    to the storage type (round to nearest even for bfloat16). With ``poison``
    every slot that holds no prefilled token is NaN.
    """
    import torch

    tdt = {F32: torch.float32, BF16: torch.bfloat16}[w.dtype]
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32).to(tdt)

    nb, hkv, bs, d = w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim
    t = v_tile(bs)
    q = randn(w.num_seqs, w.num_heads, d)
    k_cache = randn(nb, hkv, bs, d)
    v_cache = randn(nb, hkv, bs // t, d, t)
    if poison:
        m = torch.zeros(nb * bs, dtype=torch.bool)
        m[torch.from_numpy(w.prefill_slots)] = True
        nan = torch.full((), float("nan"), dtype=tdt, device=dev)
        k_cache = torch.where(m.view(nb, 1, bs, 1).to(dev), k_cache, nan)
        v_cache = torch.where(m.view(nb, 1, bs // t, 1, t).to(dev), v_cache, nan)
    writes = []
    for op in w.writes:
        n = len(op.slots)
        writes.append((randn(n, hkv, d), randn(n, hkv, d)))
    return {"q": q, "k_cache": k_cache, "v_cache": v_cache, "writes": writes}
