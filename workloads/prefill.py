"""Seeded synthetic inputs for paged prefill attention (several new tokens per
sequence). Like ``gen``, this module only generates inputs -- lengths, block
tables, query starts and N(0, 1) values -- and holds none of the attention
arithmetic.

A sequence holds L cached tokens whose last M are new; new token i sits at
position L - M + i. The cache is filled as after the cache write of those
tokens: every one of the L slots holds a value, every other slot (the tail of
the last block, unused blocks) holds NaN, and padding table entries point at a
NaN trap block, so any read past what attention may see shows up in the
output.

Recipes (seeds in brackets):
  prompts   [1661] 8 whole prompts of 2048 tokens (M = L = 2048), GQA 32/8,
            D 128, bf16, B 16.
  chunked   [1662] 32 sequences continuing a prompt in chunks: a cached
            history of U[0, 3072] tokens plus a chunk of 512 new tokens,
            GQA 32/8, D 128, bf16, B 16.
Physical block ids come from a seeded random permutation of a pool of 1.1x
the blocks needed plus the trap block.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

BF16 = "bf16"
F16 = "f16"
F32 = "f32"


@dataclass
class PrefillWorkload:
    name: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str
    seed: int
    scale: float
    context_lens: np.ndarray   # int32 [S]
    query_lens: np.ndarray     # int32 [S]
    block_tables: np.ndarray   # int32 [S, max_blocks]
    num_blocks: int
    trap_block: int
    filled_slots: np.ndarray   # int64 slots holding a token

    @property
    def num_seqs(self) -> int:
        return len(self.context_lens)

    @property
    def query_start(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.query_lens)]).astype(np.int32)

    @property
    def num_tokens(self) -> int:
        return int(self.query_lens.sum())

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.num_seqs else 0

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    def positions(self) -> np.ndarray:
        """Position of every query row (L - M + i), int64 [num_tokens]."""
        return np.concatenate([np.arange(L - m, L, dtype=np.int64)
                               for L, m in zip(self.context_lens, self.query_lens)] or [np.zeros(0, np.int64)])

    def attended_pairs(self) -> int:
        """(query row, key) pairs attention covers, summed over rows: sum of p + 1."""
        p = self.positions()
        return int(np.maximum(p + 1, 0).sum())

    def flops(self) -> int:
        """Multiply-adds of S = QK^T and O = PV, counted as 2 flops each, over
        the visible (row, key) pairs of every query head: 4 * D * Hq * pairs."""
        return 4 * self.head_dim * self.num_heads * self.attended_pairs()

    def summary(self) -> dict:
        return {"workload": self.name, "num_seqs": self.num_seqs, "num_tokens": self.num_tokens,
                "num_heads": self.num_heads, "num_kv_heads": self.num_kv_heads, "head_dim": self.head_dim,
                "block_size": self.block_size, "max_query_len": self.max_query_len,
                "max_context_len": self.max_context_len}


def make(name, context_lens, query_lens, *, num_heads, num_kv_heads, head_dim, block_size, dtype=BF16,
         seed=0, scale=None, pool_factor=1.1, extra_table_cols=1) -> PrefillWorkload:
    lens = np.asarray(context_lens, dtype=np.int32)
    news = np.asarray(query_lens, dtype=np.int32)
    if lens.shape != news.shape:
        raise ValueError("one query length per sequence")
    rng = np.random.default_rng(seed)
    need = [-(-int(L) // block_size) for L in lens]
    total = sum(need)
    nb = max(int(math.ceil(total * pool_factor)), total + 1) + 1
    perm = rng.permutation(nb)
    trap = int(perm[-1])
    maxb = max(need + [1]) + extra_table_cols
    tables = np.full((len(lens), maxb), trap, dtype=np.int32)
    slots = []
    k = 0
    for s, n in enumerate(need):
        tables[s, :n] = perm[k:k + n]
        k += n
        t = np.arange(int(lens[s]), dtype=np.int64)
        slots.append(tables[s, t // block_size].astype(np.int64) * block_size + t % block_size)
    filled = np.concatenate(slots) if slots else np.zeros(0, np.int64)
    return PrefillWorkload(name, num_heads, num_kv_heads, head_dim, block_size, dtype, seed,
                           scale if scale is not None else 1.0 / math.sqrt(head_dim), lens, news, tables, nb,
                           trap, filled)


def prompts() -> PrefillWorkload:
    lens = [2048] * 8
    return make("prefill_prompts", lens, lens, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                seed=1661)


def chunked() -> PrefillWorkload:
    rng = np.random.default_rng(1662)
    hist = rng.integers(0, 3073, size=32)
    return make("prefill_chunked", hist + 512, [512] * 32, num_heads=32, num_kv_heads=8, head_dim=128,
                block_size=16, seed=1662)


BUILDERS = {"prompts": prompts, "chunked": chunked}


def v_tile(block_size: int) -> int:
    return min(block_size, 16)


def make_values(w: PrefillWorkload, device="cpu", poison=True):
    """Seeded N(0, 1) values rounded to the storage type: q [num_tokens, Hq, D],
    k_cache [NB, Hkv, B, D] and v_cache [NB, Hkv, B // T, D, T] with every
    slot that holds no token set to NaN when ``poison``."""
    import torch

    tdt = {BF16: torch.bfloat16, F16: torch.float16, F32: torch.float32}[w.dtype]
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32).to(tdt)

    nb, hkv, bs, d = w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim
    t = v_tile(bs)
    q = randn(w.num_tokens, w.num_heads, d)
    k_cache = randn(nb, hkv, bs, d)
    v_cache = randn(nb, hkv, bs // t, d, t)
    if poison:
        m = torch.zeros(nb * bs, dtype=torch.bool)
        m[torch.from_numpy(w.filled_slots)] = True
        nan = torch.full((), float("nan"), dtype=tdt, device=dev)
        k_cache = torch.where(m.view(nb, 1, bs, 1).to(dev), k_cache, nan)
        v_cache = torch.where(m.view(nb, 1, bs // t, 1, t).to(dev), v_cache, nan)
    return {"q": q, "k_cache": k_cache, "v_cache": v_cache}
