"""Host-side block pool used to build synthetic block tables, slot mappings and
copy-on-write pairs.

This is input generation, not the decode path: the GPU library receives the
tables and pairs this produces as plain integer arrays. The rules it follows
are the block manager's as the pages describe it:
  * a sequence holds ceil(tokens / B) blocks and takes a new one only when
    its next token falls past its last block (aiqz.cc tutorial, section
    分页核心思想; cf-1.com blog 3.2);
  * token t of a sequence sits at logical block t // B, offset t % B (aiqz.cc,
    section 块表映射机制);
  * sequences may list the same physical block (prefix sharing); a block is
    free when no sequence lists it (aiqz.cc, section 前缀共享机制);
  * a token written into a block that other sequences still list goes into a
    private copy of that block first: copy-on-write (aiqz.cc 前缀共享机制;
    cf-1.com 4.2);
  * freeing a sequence drops its hold on each of its blocks (cf-1.com 3.2);
  * a consistency check recounts every block's holders from the tables
    (cf-1.com 4.3).

Design. Each sequence is a span: its physical blocks in logical order and the
number of tokens they hold. Every operation is a growth of a span by n tokens
(a prompt is growth from zero) that first counts the blocks it will take, so
a batch of appends either fits the free queue as a whole or changes nothing,
as the native manager does. With ``free_order=None`` the free queue hands
out the lowest id first.
"""

from __future__ import annotations

from collections import Counter, deque


class PoolExhausted(RuntimeError):
    pass


class _Span:
    __slots__ = ("blocks", "length")

    def __init__(self, blocks, length):
        self.blocks = blocks   # physical block of each logical block
        self.length = length   # tokens held


class HostBlockPool:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("invalid size")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must list every block of the pool once")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self._holders = [0] * num_blocks   # sequences whose table lists the block
        self._queue = deque(order)         # blocks nobody lists, in hand-out order
        self._spans: dict = {}
        self.allocations = 0               # blocks handed out so far

    # -- views ------------------------------------------------------------
    @property
    def refs(self) -> list:
        """Holders of every block (its reference count)."""
        return list(self._holders)

    @property
    def tables(self) -> dict:
        return {s: list(sp.blocks) for s, sp in self._spans.items()}

    @property
    def used(self) -> dict:
        return {s: sp.length for s, sp in self._spans.items()}

    @property
    def free(self) -> tuple:
        """Free blocks in the order they will be handed out."""
        return tuple(self._queue)

    def tokens(self, seq) -> int:
        return self._spans[seq].length

    def blocks_of(self, seq) -> list:
        return list(self._spans[seq].blocks)

    # -- block bookkeeping -------------------------------------------------
    def _blocks_for(self, tokens: int) -> int:
        return -(-tokens // self.block_size)

    def _claim(self) -> int:
        pid = self._queue.popleft()
        self._holders[pid] = 1
        self.allocations += 1
        return pid

    def _release(self, pid: int) -> None:
        if self._holders[pid] <= 0:
            raise RuntimeError(f"block {pid} released more often than it was held")
        self._holders[pid] -= 1
        if self._holders[pid] == 0:
            self._queue.append(pid)

    def _new_span(self, seq) -> _Span:
        if seq in self._spans:
            raise KeyError(f"sequence {seq!r} exists")
        sp = _Span([], 0)
        self._spans[seq] = sp
        return sp

    def _grow(self, sp: _Span, n: int):
        """Reserve the next n token slots of span ``sp`` (the caller has
        checked that the free queue covers it). Returns the copy-on-write
        pair (src, dst) if the first new token fell into a block other
        sequences still list, else None."""
        pair = None
        b, off = divmod(sp.length, self.block_size)
        if n > 0 and off != 0 and self._holders[sp.blocks[b]] > 1:
            old = sp.blocks[b]
            sp.blocks[b] = self._claim()
            self._release(old)
            pair = (old, sp.blocks[b])
        for _ in range(self._blocks_for(sp.length + n) - len(sp.blocks)):
            sp.blocks.append(self._claim())
        sp.length += n
        return pair

    # -- sequence operations -------------------------------------------------
    def prefill(self, seq, num_tokens: int) -> list:
        """A new sequence holding ``num_tokens`` tokens in fresh blocks."""
        if self._blocks_for(num_tokens) > len(self._queue):
            raise PoolExhausted(f"{self._blocks_for(num_tokens)} blocks needed, {len(self._queue)} free")
        sp = self._new_span(seq)
        self._grow(sp, num_tokens)
        return list(sp.blocks)

    def share(self, seq, src, num_tokens: int) -> list:
        """A new sequence whose first ``num_tokens`` tokens are those of
        ``src``, read from the same blocks."""
        base = self._spans[src]
        if num_tokens > base.length:
            raise ValueError("cannot share more tokens than the source holds")
        blocks = base.blocks[: self._blocks_for(num_tokens)]
        sp = self._new_span(seq)
        for pid in blocks:
            self._holders[pid] += 1
        sp.blocks = list(blocks)
        sp.length = num_tokens
        return list(blocks)

    def append_batch(self, seqs):
        """One new token for each sequence of ``seqs``, in order, all or
        nothing. Returns (slots, pairs): the slot (block * B + offset) of
        every new token, and the copy-on-write pairs (src, dst) in the order
        they were made. A shared partly filled block is copied for every
        sharer that appends before it is the block's last holder; the last
        one writes in place."""
        seqs = list(seqs)
        if len(set(seqs)) != len(seqs):
            raise ValueError("a sequence appears twice in one batch")
        spans = [self._spans[s] for s in seqs]
        need, leaving = 0, Counter()
        for sp in spans:
            b, off = divmod(sp.length, self.block_size)
            if off == 0:
                need += 1
            elif self._holders[sp.blocks[b]] - leaving[sp.blocks[b]] > 1:
                need += 1
                leaving[sp.blocks[b]] += 1
        if need > len(self._queue):
            raise PoolExhausted(f"{need} blocks needed, {len(self._queue)} free")
        slots, pairs = [], []
        for sp in spans:
            t = sp.length
            pair = self._grow(sp, 1)
            if pair is not None:
                pairs.append(pair)
            b, off = divmod(t, self.block_size)
            slots.append(sp.blocks[b] * self.block_size + off)
        return slots, pairs

    def append_token(self, seq):
        """Reserve the slot of the sequence's next token: (slot, pair), pair
        being the copy-on-write (src, dst) the write needs first, or None."""
        slots, pairs = self.append_batch([seq])
        return slots[0], (pairs[0] if pairs else None)

    def free_seq(self, seq) -> None:
        sp = self._spans.pop(seq)
        for pid in sp.blocks:
            self._release(pid)

    # -- accounting ---------------------------------------------------------
    def blocks_in_use(self) -> int:
        return sum(1 for h in self._holders if h > 0)

    def blocks_without_sharing(self) -> int:
        """Blocks the live sequences would take if none shared a block."""
        return sum(self._blocks_for(sp.length) for sp in self._spans.values())

    def check_consistency(self) -> None:
        recount = Counter(pid for sp in self._spans.values() for pid in sp.blocks)
        bad = [pid for pid in range(self.num_blocks) if recount.get(pid, 0) != self._holders[pid]]
        if bad:
            raise AssertionError(f"reference counts disagree with the tables at blocks {bad[:8]}")
        queued = Counter(self._queue)
        if any(c > 1 for c in queued.values()):
            raise AssertionError("a block is on the free list twice")
        for pid, h in enumerate(self._holders):
            if (h == 0) != (pid in queued):
                raise AssertionError(f"block {pid}: count {h} but free-list membership {pid in queued}")
        for s, sp in self._spans.items():
            if len(sp.blocks) != self._blocks_for(sp.length):
                raise AssertionError(f"sequence {s!r}: {len(sp.blocks)} blocks for {sp.length} tokens")
