"""Host-side block pool used to build synthetic block tables, slot mappings and
copy-on-write pairs.

This is input generation, not the decode path: the GPU library receives the
tables and pairs this produces as plain integer arrays. It follows the block
manager described on the pages:
  * on-demand allocation -- a sequence takes a new block only when its last
    block is full (aiqz.cc tutorial, section "分页核心思想"; cf-1.com blog 3.2);
  * prefix sharing by reference counts (aiqz.cc, section "前缀共享机制");
  * copy-on-write on the first write into a block whose count is above one:
    take a new block, copy the old one into it, write the token, drop one
    reference from the old block (aiqz.cc "前缀共享机制"; cf-1.com 4.2);
  * release by decrementing counts and returning blocks at zero, mapping
    removed before the decrement (cf-1.com 3.2);
  * a debug consistency check of every count against the tables (cf-1.com 4.3).
With ``free_order=None`` the free list hands out the lowest id first, the
behaviour of the Python demo in the aiqz.cc tutorial ("Python 演示").
"""

from __future__ import annotations

from collections import deque


class PoolExhausted(RuntimeError):
    pass


class HostBlockPool:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("invalid size")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.refs = [0] * num_blocks
        order = range(num_blocks) if free_order is None else [int(x) for x in free_order]
        self.free = deque(order)
        self.tables: dict = {}
        self.used: dict = {}
        self.allocations = 0

    # -- primitives -------------------------------------------------------
    def _alloc(self) -> int:
        if not self.free:
            raise PoolExhausted("no free block")
        pid = self.free.popleft()
        self._inc_ref(pid)
        self.allocations += 1
        return pid

    def _inc_ref(self, pid: int) -> None:
        self.refs[pid] += 1

    def _dec_ref(self, pid: int) -> None:
        if self.refs[pid] <= 0:
            raise RuntimeError(f"reference count of block {pid} would go negative")
        self.refs[pid] -= 1
        if self.refs[pid] == 0:
            self.free.append(pid)

    # -- sequence operations ---------------------------------------------
    def prefill(self, seq, num_tokens: int) -> list:
        if seq in self.tables:
            raise KeyError(f"sequence {seq!r} exists")
        need = -(-num_tokens // self.block_size)
        self.tables[seq] = [self._alloc() for _ in range(need)]
        self.used[seq] = num_tokens
        return list(self.tables[seq])

    def share(self, seq, src, num_tokens: int) -> list:
        if seq in self.tables:
            raise KeyError(f"sequence {seq!r} exists")
        if num_tokens > self.used[src]:
            raise ValueError("cannot share more tokens than the source holds")
        n = -(-num_tokens // self.block_size)
        shared = self.tables[src][:n]
        for pid in shared:
            self._inc_ref(pid)
        self.tables[seq] = list(shared)
        self.used[seq] = num_tokens
        return list(shared)

    def append_token(self, seq):
        """Reserve the slot of the sequence's next token.

        Returns (slot, cow_pair) where slot = pid * B + offset and cow_pair is
        (src, dst) when the write had to copy a shared block first, else None.
        """
        blocks = self.tables[seq]
        pos = self.used[seq] % self.block_size
        cow = None
        if pos == 0:
            blocks.append(self._alloc())
        else:
            last = blocks[-1]
            if self.refs[last] > 1:
                new_pid = self._alloc()
                blocks[-1] = new_pid
                self._dec_ref(last)
                cow = (last, new_pid)
        self.used[seq] += 1
        return blocks[-1] * self.block_size + pos, cow

    def free_seq(self, seq) -> None:
        blocks = self.tables.pop(seq)
        del self.used[seq]
        for pid in blocks:
            self._dec_ref(pid)

    # -- accounting ---------------------------------------------------------
    def blocks_in_use(self) -> int:
        return sum(1 for r in self.refs if r > 0)

    def blocks_without_sharing(self) -> int:
        return sum(-(-u // self.block_size) for u in self.used.values())

    def check_consistency(self) -> None:
        counts = [0] * self.num_blocks
        for blocks in self.tables.values():
            for pid in blocks:
                counts[pid] += 1
        if counts != self.refs:
            bad = [i for i in range(self.num_blocks) if counts[i] != self.refs[i]]
            raise AssertionError(f"reference counts disagree with the tables at blocks {bad[:8]}")
        free = set(self.free)
        if len(free) != len(self.free):
            raise AssertionError("a block is on the free list twice")
        for i, r in enumerate(self.refs):
            if (r == 0) != (i in free):
                raise AssertionError(f"block {i}: count {r} but free-list membership {i in free}")
