"""Plain float64 CPU oracle for paged KV-cache decode attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path. It
imports nothing from ``paged_kv_cache_165_amd`` and shares no code with it.

Pages cited (the four web pages this method is taken from):
  [aiqz]     aiqz.cc/article/paged-attention-mechanism.html -- PagedAttention
             tutorial (library metaphor, formulas, BlockManager demo, quiz).
  [lihaoran] lihaoran.work/auto-20261007-1900 -- PagedAttention mechanism note
             (the [5, 1, 7] worked example and ``block_layout``).
  [cf-1]     cf-1.com/news/5879632 -- engineering blog on block mapping,
             on-demand allocation and copy-on-write (numbered sections).
  [ipipp]    ipipp.com/html/20260817/41684.html -- "PagedAttention原理是什么？
             vLLM如何用它解决大模型推理显存碎片问题".

Storage layout (the pages fix none; this is the reading used everywhere):
  k_cache          : [num_blocks, num_kv_heads, block_size, head_dim]
  v_cache          : [num_blocks, num_kv_heads, block_size // T, head_dim, T],
                     T = min(block_size, 16): each block's V rows are stored as
                     tiles of T tokens, transposed (head_dim-major, token-minor).
                     V row of (block pid, offset off) = v_cache[pid, :, off // T, :, off % T].
  q, out           : [num_seqs, num_heads, head_dim]
  k, v (new tokens): [num_tokens, num_kv_heads, head_dim]
  block_tables     : int [num_seqs, max_blocks_per_seq]
  context_lens     : int [num_seqs]
  slot_mapping     : int [num_tokens], slot = physical_block * B + offset, -1 = skip
  src_dst_pairs    : int [num_pairs, 2]

Element types: ``F32`` arrays are numpy float32; ``F16`` arrays are numpy
float16; ``BF16`` arrays are numpy uint16 holding bfloat16 bit patterns (numpy
has no bfloat16). Attention converts every element it reads to float64
exactly; the cache writes and copies move raw elements and never convert.

Pins (all in ``tests/test_oracle.py``, run with ``-m "not gpu"``):
  block_layout            printed results and asserts of [lihaoran]; quiz Q10 of [aiqz]
  translate               [5, 1, 7] example of [lihaoran]; BlockTable example of [ipipp]
  gather_rows/paged_decode slot-id probe (closed form 16.5), ctx = 1, K == 0,
                          GQA head-mapping probe, two-token scale probe, float64
                          scaled_dot_product_attention, pure-Python brute force,
                          permutation invariance, shared-vs-copied blocks, NaN poison
  partition_stats/lse_merge equality with the unsplit softmax, single partition,
                          empty partition
  paged_prefill           one new token per sequence equals paged_decode; a whole
                          prompt equals float64 causal scaled_dot_product_attention;
                          pure-Python brute force; the last new token equals the
                          decode of the full context; a planted off-by-one in the
                          causal bound is caught
  write_cache             write probe (position 9 -> slot 29 -> block 7 offset 1),
                          skip slot -1, raw-bit copies of NaN payloads
  copy_blocks             whole-block copy, source untouched, precondition errors
  write_cache_layers /    (tests/test_oracle_layers.py) the write probe and a copy
  copy_blocks_layers      probe in every layer with layer-specific values, one
                          layer equal to the single-layer call, planted mistakes
                          (layer 0's rows everywhere, copying layer 0 only) caught
No function here is "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

F32 = "f32"
BF16 = "bf16"
F16 = "f16"

_STORAGE = {F32: np.float32, F16: np.float16, BF16: np.uint16}


def _check_storage(x: np.ndarray, dtype: str, name: str) -> None:
    want = _STORAGE[dtype]
    if x.dtype != want:
        raise TypeError(f"{name}: expected numpy {np.dtype(want).name} storage for {dtype}, got {x.dtype}")


def v_tile(block_size: int) -> int:
    """Tokens per transposed V tile: min(block_size, 16)."""
    return min(block_size, 16)


def v_cache_shape(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int) -> tuple:
    t = v_tile(block_size)
    return (num_blocks, num_kv_heads, block_size // t, head_dim, t)


def k_rows_at(cache: np.ndarray, pid, off) -> np.ndarray:
    """K rows [..., num_kv_heads, head_dim] of (block, offset) pairs."""
    return cache[pid, :, off, :]


def v_rows_at(cache: np.ndarray, pid, off, block_size: int) -> np.ndarray:
    """V rows [..., num_kv_heads, head_dim] of (block, offset) pairs, read from
    the transposed tile layout."""
    t = v_tile(block_size)
    return cache[pid, :, off // t, :, off % t]


def to_float64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of every stored element.

    A bfloat16 value is, by definition, the float32 whose upper 16 bits are the
    stored pattern and whose lower 16 bits are zero; float32 and float16 widen
    exactly to float64.
    """
    _check_storage(x, dtype, "array")
    if dtype == BF16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


# --------------------------------------------------------------------------
# Block arithmetic
# --------------------------------------------------------------------------

def block_layout(tokens: int, block_size: int) -> tuple[int, int]:
    """Blocks needed for ``tokens`` cached positions and the empty slots left
    in the last block.

    [lihaoran] section "末块会浪费多少空间？": the block count is the ceiling of
    T / b and the empty slots are that count times b minus T; a negative token
    count or a non-positive block size is an error. The block count is also the
    ceiling formula N = ceil(S_used / B_block) of [aiqz] section "分页核心思想".
    """
    if tokens < 0 or block_size <= 0:
        raise ValueError("invalid size")
    blocks = -(-tokens // block_size)
    return blocks, blocks * block_size - tokens


def translate(block_table_row, position: int, block_size: int) -> tuple[int, int]:
    """Logical token position -> (physical block id, offset inside the block).

    [aiqz] section "块表映射机制", equation pid = block_table[i], off = j mod B,
    with the logical block index i = j // B made explicit by [lihaoran] section
    "块表把逻辑顺序映射到物理位置" (position t: logical block t // b, offset t % b).
    """
    if position < 0 or block_size <= 0:
        raise ValueError("invalid position or block size")
    logical, offset = divmod(position, block_size)
    return int(block_table_row[logical]), offset


def gather_rows(cache: np.ndarray, block_table_row, context_len: int, block_size: int,
                dtype: str, kind: str = "k") -> np.ndarray:
    """Contiguous float64 view [context_len, num_kv_heads, head_dim] of one
    sequence's cached K rows (kind "k") or V rows (kind "v"), read through its
    block table.

    Each logical position t in [0, context_len) is translated with
    ``translate`` and the row at (pid, off) is taken. Only the first
    ceil(context_len / B) table entries are read and no slot at or beyond
    context_len is read ([lihaoran] "末块会浪费多少空间？": the tail slots of the
    last block are empty; [ipipp] "分页式KV缓存的底层设计": the kernel presents a
    contiguous sequence view assembled from the physical blocks).
    """
    _check_storage(cache, dtype, "cache")
    nb, hkv = cache.shape[0], cache.shape[1]
    if kind == "k":
        if cache.ndim != 4 or cache.shape[2] != block_size:
            raise ValueError("k_cache must be [num_blocks, num_kv_heads, block_size, head_dim]")
        d = cache.shape[3]
    elif kind == "v":
        if cache.ndim != 5 or cache.shape != v_cache_shape(nb, hkv, block_size, cache.shape[3]):
            raise ValueError("v_cache must be [num_blocks, num_kv_heads, block_size // T, head_dim, T]")
        d = cache.shape[3]
    else:
        raise ValueError("kind must be 'k' or 'v'")
    if context_len == 0:
        return np.zeros((0, hkv, d), dtype=np.float64)
    t = np.arange(context_len)
    logical = t // block_size
    offset = t % block_size
    pid = np.asarray(block_table_row, dtype=np.int64)[logical]
    if pid.min() < 0 or pid.max() >= nb:
        raise IndexError("block table entry outside the block pool")
    rows = k_rows_at(cache, pid, offset) if kind == "k" else v_rows_at(cache, pid, offset, block_size)
    return to_float64(rows, dtype)


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def attend_contiguous(q_seq: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray,
                      scale: float) -> np.ndarray:
    """Single-query softmax attention of every query head over contiguous rows.

    q_seq: float64 [num_heads, D]; k_rows, v_rows: float64 [L, num_kv_heads, D].
    Query head h reads KV head h // g with g = num_heads // num_kv_heads
    (contiguous groups of query heads share one KV head). For each head:
    x = scale * K q, p = exp(x - max x), out = (p V) / sum(p). With L = 0 the
    output row is 0 (an empty weighted sum). Paging does not change this value:
    it only changes where the rows live ([aiqz] "常见误区": K and V are neither
    compressed nor reduced in precision; [lihaoran] "块表把逻辑顺序映射到物理位置":
    attention still covers the whole visible history).
    """
    hq, d = q_seq.shape
    n, hkv, d2 = k_rows.shape
    if d2 != d or v_rows.shape != k_rows.shape:
        raise ValueError("shape mismatch")
    if hq % hkv != 0:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    g = hq // hkv
    out = np.zeros((hq, d), dtype=np.float64)
    if n == 0:
        return out
    for h in range(hq):
        kv = h // g
        x = scale * (k_rows[:, kv, :] @ q_seq[h])
        p = np.exp(x - x.max())
        out[h] = (p @ v_rows[:, kv, :]) / p.sum()
    return out


def _check_decode_args(q, k_cache, v_cache, block_tables, context_lens, block_size, dtype,
                       one_row_per_seq=True):
    _check_storage(q, dtype, "q")
    _check_storage(k_cache, dtype, "k_cache")
    _check_storage(v_cache, dtype, "v_cache")
    rows, hq, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    if d2 != d or bs != block_size:
        raise ValueError("cache shape does not match q / block_size")
    if v_cache.shape != v_cache_shape(nb, hkv, block_size, d):
        raise ValueError("v_cache shape does not match the transposed tile layout")
    if len(context_lens) != len(block_tables) or (one_row_per_seq and len(context_lens) != rows):
        raise ValueError("one block table and one context length per sequence")
    for L in context_lens:
        if L < 0:
            raise ValueError("negative context length")
        blocks, _ = block_layout(int(L), block_size)
        if blocks > np.asarray(block_tables).shape[1]:
            raise ValueError("block table too short for context length")


def paged_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                 block_tables: np.ndarray, context_lens, scale: float,
                 block_size: int, dtype: str) -> np.ndarray:
    """Paged decode attention, float64 [num_seqs, num_heads, head_dim].

    For each sequence: gather its K and V rows through its block table
    (``gather_rows``), then run ``attend_contiguous``. This is the operator of
    [aiqz] "vLLM 工程落地" / [cf-1] 5.1 (attention that first looks up the
    block table and then reads block data), evaluated by its definition.
    """
    _check_decode_args(q, k_cache, v_cache, block_tables, context_lens, block_size, dtype)
    s = q.shape[0]
    out = np.zeros(q.shape, dtype=np.float64)
    for i in range(s):
        L = int(context_lens[i])
        k_rows = gather_rows(k_cache, block_tables[i], L, block_size, dtype, "k")
        v_rows = gather_rows(v_cache, block_tables[i], L, block_size, dtype, "v")
        out[i] = attend_contiguous(to_float64(q[i], dtype), k_rows, v_rows, scale)
    return out


def paged_prefill(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                  block_tables: np.ndarray, context_lens, query_start, scale: float,
                  block_size: int, dtype: str) -> np.ndarray:
    """Paged prefill (multi-token query) attention, float64 [total_q, num_heads, D].

    Sequence s holds L_s = context_lens[s] tokens in its blocks, the last
    M_s = query_start[s + 1] - query_start[s] of them new (their K and V
    already written to the cache). Its i-th new token, at position
    p = L_s - M_s + i, attends to tokens 0..p: the visible history up to and
    including itself ([lihaoran] "块表把逻辑顺序映射到物理位置": attention
    covers the whole visible history; for a token of the prompt, what it can
    see is what precedes it). Each query row is ``attend_contiguous`` over the
    first p + 1 gathered rows; q rows of sequence s are
    q[query_start[s]:query_start[s + 1]].
    """
    starts = [int(x) for x in query_start]
    s = len(starts) - 1
    if s < 0 or q.shape[0] != starts[-1] or any(b < a for a, b in zip(starts, starts[1:])):
        raise ValueError("query_start must be non-decreasing, from 0 to the number of query rows")
    if starts[0] != 0:
        raise ValueError("query_start[0] must be 0")
    _check_decode_args(q, k_cache, v_cache, block_tables, context_lens, block_size, dtype,
                       one_row_per_seq=False)
    if len(context_lens) != s:
        raise ValueError("one context length per sequence")
    out = np.zeros(q.shape, dtype=np.float64)
    for i in range(s):
        L = int(context_lens[i])
        m = starts[i + 1] - starts[i]
        if m > L:
            raise ValueError("more new tokens than the sequence holds")
        k_rows = gather_rows(k_cache, block_tables[i], L, block_size, dtype, "k")
        v_rows = gather_rows(v_cache, block_tables[i], L, block_size, dtype, "v")
        for j in range(m):
            p = L - m + j
            out[starts[i] + j] = attend_contiguous(to_float64(q[starts[i] + j], dtype), k_rows[:p + 1],
                                                   v_rows[:p + 1], scale)
    return out


# --------------------------------------------------------------------------
# Split over context partitions and log-sum-exp merge
# --------------------------------------------------------------------------

def partition_stats(q_head: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray,
                    scale: float) -> tuple[float, float, np.ndarray]:
    """(m, l, o) of one query head over one range of rows of its KV head.

    m = max of the logits x = scale * K q, l = sum exp(x - m),
    o = sum exp(x - m) v / l. An empty range gives (-inf, 0, 0).
    k_rows, v_rows: float64 [n, D] of the single KV head this query head reads.
    """
    d = q_head.shape[0]
    if k_rows.shape[0] == 0:
        return -math.inf, 0.0, np.zeros(d, dtype=np.float64)
    x = scale * (k_rows @ q_head)
    m = float(x.max())
    p = np.exp(x - m)
    l_sum = float(p.sum())
    return m, l_sum, (p @ v_rows) / l_sum


def lse_merge(parts) -> np.ndarray:
    """Merge per-partition (m_p, l_p, o_p) into the softmax over their union.

    M = max_p m_p, w_p = l_p * exp(m_p - M), result = sum_p w_p o_p / sum_p w_p.
    Partitions with l_p = 0 (empty) carry no weight and are skipped; if every
    partition is empty the result is 0. The identity holds because
    sum_p l_p exp(m_p - M) is the global softmax denominator scaled by
    exp(-M) and w_p o_p the matching share of the numerator.
    """
    parts = list(parts)
    live = [(m, l_sum, o) for (m, l_sum, o) in parts if l_sum > 0.0]
    d = parts[0][2].shape[0]
    if not live:
        return np.zeros(d, dtype=np.float64)
    big_m = max(m for m, _, _ in live)
    num = np.zeros(d, dtype=np.float64)
    den = 0.0
    for m, l_sum, o in live:
        w = l_sum * math.exp(m - big_m)
        num += w * o
        den += w
    return num / den


def paged_decode_partitioned(q, k_cache, v_cache, block_tables, context_lens, scale,
                             block_size, dtype, partition_size) -> np.ndarray:
    """Paged decode computed per ``partition_size``-token range and merged with
    ``lse_merge``. Used only to pin the merge formula against ``paged_decode``;
    it never produces a reference output for the GPU path."""
    _check_decode_args(q, k_cache, v_cache, block_tables, context_lens, block_size, dtype)
    if partition_size <= 0:
        raise ValueError("partition_size must be positive")
    s, hq, d = q.shape
    hkv = k_cache.shape[1]
    g = hq // hkv
    out = np.zeros(q.shape, dtype=np.float64)
    for i in range(s):
        L = int(context_lens[i])
        k_rows = gather_rows(k_cache, block_tables[i], L, block_size, dtype, "k")
        v_rows = gather_rows(v_cache, block_tables[i], L, block_size, dtype, "v")
        qi = to_float64(q[i], dtype)
        nparts = max(1, -(-L // partition_size))
        for h in range(hq):
            kv = h // g
            parts = []
            for p in range(nparts):
                lo, hi = p * partition_size, min(L, (p + 1) * partition_size)
                parts.append(partition_stats(qi[h], k_rows[lo:hi, kv, :], v_rows[lo:hi, kv, :], scale))
            out[i, h] = lse_merge(parts)
    return out


# --------------------------------------------------------------------------
# Cache maintenance: token write and copy-on-write block copy
# --------------------------------------------------------------------------

def write_cache(k: np.ndarray, v: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                slot_mapping, block_size: int) -> tuple[np.ndarray, np.ndarray]:
    """Write each new token's K and V rows into its slot; returns new caches.

    For token i with slot_i >= 0: pid, off = divmod(slot_i, B), the K row at
    (pid, off) becomes k[i] and the V row at (pid, off) becomes v[i] (in the
    transposed tile layout). A slot of -1 means the token is skipped.
    Elements are moved as stored (no conversion), so the result is defined bit
    for bit. This stores each sequence's newest token, after any copy of a
    shared block ([aiqz] "前缀共享机制");
    the slot is the (pid, off) pair of [aiqz] "块表映射机制" flattened as
    pid * B + off.
    Preconditions (raise): equal storage dtypes, slots in {-1} U [0, NB * B),
    non-negative slots pairwise distinct.
    """
    if not (k.dtype == v.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("all arrays must share one storage dtype")
    nb, hkv, bs, d = k_cache.shape
    if bs != block_size or v_cache.shape != v_cache_shape(nb, hkv, block_size, d):
        raise ValueError("cache shapes do not match block_size")
    slots = np.asarray(slot_mapping, dtype=np.int64)
    if k.shape != (len(slots), hkv, d) or v.shape != k.shape:
        raise ValueError("k/v must be [num_tokens, num_kv_heads, head_dim]")
    live = slots[slots >= 0]
    if np.any(slots < -1) or np.any(live >= nb * block_size):
        raise IndexError("slot outside the block pool")
    if len(np.unique(live)) != len(live):
        raise ValueError("duplicate slot in slot_mapping")
    t = v_tile(block_size)
    k_new = k_cache.copy()
    v_new = v_cache.copy()
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        pid, off = divmod(int(slot), block_size)
        k_new[pid, :, off, :] = k[i]
        v_new[pid, :, off // t, :, off % t] = v[i]
    return k_new, v_new


def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray,
                src_dst_pairs) -> tuple[np.ndarray, np.ndarray]:
    """Copy whole physical blocks src -> dst in both caches; returns new caches.

    The copy of copy-on-write ([aiqz] "前缀共享机制"; [cf-1] 4.2): a new block
    receives the old block's full contents -- every KV head and all B slots,
    including slots past the sequence's end -- before the new token is written
    into it. Pairs act as if applied at once. Preconditions (raise): ids in
    range, every dst distinct, no dst equal to any src.
    """
    if k_cache.shape[0] != v_cache.shape[0] or k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache must have the same block count and dtype")
    nb = k_cache.shape[0]
    pairs = np.asarray(src_dst_pairs, dtype=np.int64).reshape(-1, 2)
    if pairs.size and (pairs.min() < 0 or pairs.max() >= nb):
        raise IndexError("block id outside the block pool")
    src, dst = pairs[:, 0], pairs[:, 1]
    if len(np.unique(dst)) != len(dst):
        raise ValueError("duplicate destination block")
    if np.intersect1d(src, dst).size:
        raise ValueError("a destination block is also a source block")
    k_new = k_cache.copy()
    v_new = v_cache.copy()
    for s_id, d_id in pairs:
        k_new[d_id] = k_cache[s_id]
        v_new[d_id] = v_cache[s_id]
    return k_new, v_new


# --------------------------------------------------------------------------
# Several layers at once
# --------------------------------------------------------------------------

def write_cache_layers(k: np.ndarray, v: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                       slot_mapping, block_size: int) -> tuple[np.ndarray, np.ndarray]:
    """``write_cache`` applied to every layer with the one slot mapping:
    k, v [L, num_tokens, Hkv, D]; k_cache [L, NB, Hkv, B, D]; v_cache
    [L, NB, Hkv, B/T, D, T]. A token lives at the same slot in every layer's
    cache (its position in the sequence fixes the slot, [aiqz] "块表映射机制"),
    and each layer's rows are its own. Returns new caches."""
    if k_cache.ndim != 5 or v_cache.ndim != 6 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("layered arrays need a leading layer axis")
    n_layers = k_cache.shape[0]
    if v_cache.shape[0] != n_layers or k.shape[0] != n_layers or v.shape[0] != n_layers:
        raise ValueError("one slice per layer")
    out_k, out_v = [], []
    for layer in range(n_layers):
        kc, vc = write_cache(k[layer], v[layer], k_cache[layer], v_cache[layer], slot_mapping, block_size)
        out_k.append(kc)
        out_v.append(vc)
    return np.stack(out_k), np.stack(out_v)


def copy_blocks_layers(k_cache: np.ndarray, v_cache: np.ndarray,
                       src_dst_pairs) -> tuple[np.ndarray, np.ndarray]:
    """``copy_blocks`` applied to every layer with the same pairs: a block
    shared by sequences is shared in every layer, so copy-on-write copies it
    in all of them ([aiqz] "前缀共享机制"). Returns new caches."""
    if k_cache.ndim != 5 or v_cache.ndim != 6 or k_cache.shape[0] != v_cache.shape[0]:
        raise ValueError("layered caches need the same leading layer axis")
    pairs = [copy_blocks(k_cache[layer], v_cache[layer], src_dst_pairs) for layer in range(k_cache.shape[0])]
    return np.stack([p[0] for p in pairs]), np.stack([p[1] for p in pairs])
