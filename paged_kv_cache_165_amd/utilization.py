"""Contiguous versus paged KV-cache allocation on synthetic request traces.

Host-side only (no GPU). It measures the quantities the PagedAttention
tutorial (aiqz.cc, section 显存收益分析) defines for comparing the two
schemes:

  waste ratio     eta_waste = (M_alloc - M_used) / M_alloc, M counted in token
                  slots (every slot of one layer holds the same bytes);
  paged internal  eta'_int ~ 1 / (2 N_blocks): each request wastes half of
  fragmentation   its last block on average.

Two allocators serve the same trace of requests (arrival step, prompt length,
output length) in discrete steps, each running request producing one token per
step:

  contiguous  a request reserves one contiguous region of prompt + max_new
              slots when it is admitted (its output length is not known in
              advance), first fit over a free list; the region is released
              when it finishes. Waste is the reserved-but-unwritten tail plus
              what cannot be handed out because free space is fragmented.
  paged       blocks of block_size slots on demand, through the native block
              manager (include/pa_blocks.h): the prompt's blocks at admission,
              one more block whenever a request's last block is full. A
              request is admitted only if its prompt's blocks plus one block
              of growth per running request are free (a watermark), and one
              that needs a block when none is free waits that step.

Admission is first come, first served in both; a request is admitted only if
its initial allocation fits, and one that could never fit (longer than the
whole cache) is rejected on arrival. If in some step no running paged request
can get the block it needs, the most recently admitted one is preempted by
recomputation: its blocks are freed and it goes back to the head of the
queue, its generated tokens lost (they count in `preempted_tokens`).
"""

from __future__ import annotations

import bisect
import math
from dataclasses import dataclass

import numpy as np

from .blocks import BlockManager, BlocksExhausted


def waste_ratio(alloc_slots: int, used_slots: int) -> float:
    """eta_waste = (M_alloc - M_used) / M_alloc (0 when nothing is allocated)."""
    return (alloc_slots - used_slots) / alloc_slots if alloc_slots else 0.0


def paged_internal_estimate(mean_blocks: float) -> float:
    """eta'_int ~ 1 / (2 N_blocks): half a block wasted per request."""
    return 1.0 / (2.0 * mean_blocks) if mean_blocks > 0 else 0.0


def static_waste(lengths, block_size: int, reserve: int) -> dict:
    """Waste ratios of a set of resident sequences of the given lengths:
    contiguous with `reserve` slots per sequence, paged with blocks of
    `block_size` (ceil(L / B) blocks per sequence)."""
    lens = np.asarray(lengths, dtype=np.int64)
    if np.any(lens > reserve):
        raise ValueError("a sequence longer than the contiguous reservation")
    used = int(lens.sum())
    blocks = -(-lens // block_size)
    paged_alloc = int(blocks.sum()) * block_size
    return {
        "used_slots": used,
        "contiguous_alloc_slots": int(len(lens) * reserve),
        "paged_alloc_slots": paged_alloc,
        "contiguous_waste": waste_ratio(int(len(lens) * reserve), used),
        "paged_waste": waste_ratio(paged_alloc, used),
        "paged_internal_estimate": paged_internal_estimate(float(blocks.mean()) if len(lens) else 0.0),
    }


@dataclass
class Request:
    arrival: int
    prompt: int
    output: int


def make_trace(num_requests: int, seed: int, *, prompt_median=512, output_median=256, sigma=0.8,
               max_prompt=4096, max_new=2048, arrivals_per_step=0.05) -> list:
    """Seeded synthetic trace: lognormal prompt and output lengths (clipped to
    [1, max_prompt] and [1, max_new]) and Poisson arrivals."""
    rng = np.random.default_rng(seed)
    p = np.clip(np.round(np.exp(rng.normal(math.log(prompt_median), sigma, num_requests))), 1, max_prompt)
    o = np.clip(np.round(np.exp(rng.normal(math.log(output_median), sigma, num_requests))), 1, max_new)
    gaps = rng.exponential(1.0 / arrivals_per_step, num_requests)
    t = np.floor(np.cumsum(gaps)).astype(np.int64)
    return [Request(int(a), int(pp), int(oo)) for a, pp, oo in zip(t, p, o)]


class _FirstFit:
    """Contiguous allocator over [0, capacity): sorted free list of (start, length)."""

    def __init__(self, capacity: int):
        self.free = [(0, capacity)]

    def alloc(self, n: int):
        for i, (start, length) in enumerate(self.free):
            if length >= n:
                if length == n:
                    self.free.pop(i)
                else:
                    self.free[i] = (start + n, length - n)
                return start
        return None

    def release(self, start: int, n: int) -> None:
        i = bisect.bisect_left(self.free, (start, 0))
        self.free.insert(i, (start, n))
        # merge with neighbours
        if i + 1 < len(self.free) and self.free[i][0] + self.free[i][1] == self.free[i + 1][0]:
            self.free[i] = (self.free[i][0], self.free[i][1] + self.free[i + 1][1])
            self.free.pop(i + 1)
        if i > 0 and self.free[i - 1][0] + self.free[i - 1][1] == self.free[i][0]:
            self.free[i - 1] = (self.free[i - 1][0], self.free[i - 1][1] + self.free[i][1])
            self.free.pop(i)

    def largest(self) -> int:
        return max((length for _, length in self.free), default=0)


def simulate(trace, capacity_slots: int, policy: str, *, block_size: int = 16, max_new: int = 2048,
             max_steps: int = 1_000_000) -> dict:
    """Serve `trace` with `policy` ("contiguous" or "paged") on a cache of
    `capacity_slots` token slots; every running request generates one token
    per step. Returns time averages over the steps with at least one running
    request: waste ratio, running requests, slots in use, plus totals."""
    if policy not in ("contiguous", "paged"):
        raise ValueError("policy is 'contiguous' or 'paged'")
    pending = sorted(trace, key=lambda r: r.arrival)
    queue: list = []
    running: dict = {}  # id -> [request, generated tokens, contiguous start or None]
    order: list = []    # running ids in admission order
    if policy == "paged":
        nb = capacity_slots // block_size
        bm = BlockManager(nb, block_size)
    else:
        ff = _FirstFit(capacity_slots)
    nxt = 0
    step = 0
    done = 0
    rejected = 0
    preempted_tokens = 0
    waste_sum = run_sum = alloc_sum = 0.0
    busy_steps = 0
    stalls = 0
    generated = 0
    wait_sum = 0
    while (nxt < len(pending) or queue or running) and step < max_steps:
        while nxt < len(pending) and pending[nxt].arrival <= step:
            r = pending[nxt]
            fits = (r.prompt + max_new <= capacity_slots if policy == "contiguous"
                    else -(-(r.prompt + r.output) // block_size) <= capacity_slots // block_size)
            if fits:
                queue.append((nxt, r))
            else:
                rejected += 1
            nxt += 1
        # admission, first come first served
        while queue:
            rid, r = queue[0]
            if policy == "paged":
                # watermark: the prompt's blocks plus one block of growth per
                # running request (and the new one) must be free
                if bm.num_free() < -(-r.prompt // block_size) + len(running) + 1:
                    break
                bm.prefill(rid, r.prompt)
                start = None
            else:
                start = ff.alloc(r.prompt + max_new)
                if start is None:
                    break
            queue.pop(0)
            running[rid] = [r, 0, start]
            order.append(rid)
            wait_sum += step - r.arrival
        # one token per running request
        finished = []
        if policy == "paged":
            progressed = False
            ids = list(running)
            try:
                bm.append(ids)  # all-or-nothing: the common case, one call
                grown = ids
            except BlocksExhausted:
                grown = []
                for rid in ids:
                    try:
                        bm.append([rid])
                        grown.append(rid)
                    except BlocksExhausted:
                        stalls += 1
            for rid in grown:
                progressed = True
                running[rid][1] += 1
                generated += 1
                if running[rid][1] == running[rid][0].output:
                    finished.append(rid)
            if running and not progressed:
                victim = order.pop()
                r, gen, _ = running.pop(victim)
                bm.free(victim)
                preempted_tokens += gen
                queue.insert(0, (victim, r))
            alloc = bm.blocks_in_use() * block_size
        else:
            for rid, st in running.items():
                st[1] += 1
                generated += 1
                if st[1] == st[0].output:
                    finished.append(rid)
            alloc = sum(st[0].prompt + max_new for st in running.values())
        used = sum(st[0].prompt + st[1] for st in running.values())
        if running:
            busy_steps += 1
            waste_sum += waste_ratio(alloc, used)
            run_sum += len(running)
            alloc_sum += alloc
        for rid in finished:
            st = running.pop(rid)
            order.remove(rid)
            if policy == "paged":
                bm.free(rid)
            else:
                ff.release(st[2], st[0].prompt + max_new)
            done += 1
        step += 1
    if policy == "paged":
        bm.check()
        bm.close()
    return {
        "policy": policy,
        "steps": step,
        "finished": done,
        "generated_tokens": generated,
        "tokens_per_step": generated / step if step else 0.0,
        "mean_waste": waste_sum / busy_steps if busy_steps else 0.0,
        "mean_running": run_sum / busy_steps if busy_steps else 0.0,
        "mean_alloc_fraction": alloc_sum / busy_steps / capacity_slots if busy_steps else 0.0,
        "mean_queue_wait_steps": wait_sum / done if done else 0.0,
        "stalled_appends": stalls,
        "rejected": rejected,
        "preempted_tokens": preempted_tokens,
    }


def main(argv=None) -> None:
    """Print one JSON line per policy for a seeded trace (defaults: 3000
    requests, lognormal prompts of median 512 and outputs of median 256,
    max_new 2048, one arrival every 2 steps, a cache of 65,536 slots, blocks
    of 16), then the static waste of the resident lengths at the end."""
    import argparse
    import json
    ap = argparse.ArgumentParser(description=main.__doc__)
    ap.add_argument("--requests", type=int, default=3000)
    ap.add_argument("--seed", type=int, default=1680)
    ap.add_argument("--capacity", type=int, default=65536)
    ap.add_argument("--block-size", type=int, default=16)
    ap.add_argument("--max-new", type=int, default=2048)
    ap.add_argument("--arrivals-per-step", type=float, default=0.5)
    a = ap.parse_args(argv)
    trace = make_trace(a.requests, a.seed, max_new=a.max_new, arrivals_per_step=a.arrivals_per_step)
    for policy in ("contiguous", "paged"):
        r = simulate(trace, a.capacity, policy, block_size=a.block_size, max_new=a.max_new)
        r.update(capacity_slots=a.capacity, block_size=a.block_size, max_new=a.max_new, requests=a.requests,
                 seed=a.seed, arrivals_per_step=a.arrivals_per_step)
        print(json.dumps(r), flush=True)


if __name__ == "__main__":
    main()
