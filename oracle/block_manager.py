"""Reference block manager for paged KV caches (test infrastructure).

This module is test infrastructure: only the test suite, the smoke check and
the CPU-baseline leg of the benchmark may import it.  The GPU library never
calls it, and it shares no code with the library's block manager.

What it does, from the pages:

* A request's KV cache lives in fixed-size physical blocks; a per-request
  block table maps logical block j to a physical block; blocks are allocated
  on demand as tokens are generated and returned to the pool when the
  request finishes ("Paged Attention and Memory Efficiency in Production LLM
  Serving", section "How PagedAttention borrows OS paging to eliminate KV
  cache fragmentation"; "PagedAttention in Production", section "Core
  Principle", block-table figure and the paragraph after it;
  "PagedAttention — The KV Cache Problem", section "How It Works").
* The only waste is the unused tail of a sequence's last block (first page,
  same section).
* Requests that share a prefix point their tables at the same physical
  blocks; a sequence that diverges gets a new block, copy-on-write (first
  page, same section; third page, "Why This Matters for Production":
  parallel sampling and beam search share blocks).

Readings where the pages are silent (the library implements the same ones):
* Free blocks are handed out last-freed-first; a fresh pool hands out 0, 1,
  2, ... in order.
* A block is shared when more than one table references it (its reference
  count).  Appending into a shared, partially filled last block first copies
  it: a new block is allocated, the pair (old, new) is reported for the
  device copy, the sequence's table points at the new block and the old
  block's count drops by one.  A full shared block is never written, so a
  new token past it simply starts a new block.
* Appending to a sequence needs every block it will use; when the pool runs
  dry the call fails and changes nothing.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple


class OutOfBlocks(RuntimeError):
    pass


@dataclass
class _Seq:
    table: List[int] = field(default_factory=list)
    length: int = 0


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[List[int]] = None):
        """free_order: the free list, next block to hand out first (default 0, 1, 2, ...)."""
        if num_blocks < 0 or block_size < 1:
            raise ValueError("bad pool size")
        self.block_size = block_size
        self.num_blocks = num_blocks
        order = list(range(num_blocks)) if free_order is None else list(free_order)
        self._free = list(reversed(order))  # a stack: the end of the list is handed out next
        self.refcount = [0] * num_blocks
        self.seqs: Dict[int, _Seq] = {}

    # -- pool ---------------------------------------------------------------
    def num_free(self) -> int:
        return len(self._free)

    def _take(self) -> int:
        b = self._free.pop()
        self.refcount[b] = 1
        return b

    def _release(self, b: int):
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            self._free.append(b)

    # -- sequences ----------------------------------------------------------
    def add(self, seq: int):
        if seq in self.seqs:
            raise KeyError(f"sequence {seq} exists")
        self.seqs[seq] = _Seq()

    def fork(self, parent: int, child: int):
        """The child shares every block of the parent (copy-on-write later)."""
        if child in self.seqs:
            raise KeyError(f"sequence {child} exists")
        p = self.seqs[parent]
        for b in p.table:
            self.refcount[b] += 1
        self.seqs[child] = _Seq(list(p.table), p.length)

    def append(self, seq: int, n: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        """Reserve slots for n new tokens of seq.  Returns (slots, copy pairs);
        a copy pair (src, dst) must be copied on the device before the new rows
        are written."""
        s = self.seqs[seq]
        bs = self.block_size
        if n < 0:
            raise ValueError("n < 0")
        if n == 0:
            return [], []
        cow = s.length % bs != 0 and self.refcount[s.table[-1]] > 1
        new_blocks = (s.length + n + bs - 1) // bs - len(s.table)
        if self._needed(seq, n) > len(self._free):
            raise OutOfBlocks(f"sequence {seq}: {self._needed(seq, n)} blocks needed, {len(self._free)} free")
        pairs = []
        if cow:
            old = s.table[-1]
            new = self._take()
            self._release(old)
            s.table[-1] = new
            pairs.append((old, new))
        for _ in range(new_blocks):
            s.table.append(self._take())
        slots = [s.table[t // bs] * bs + t % bs for t in range(s.length, s.length + n)]
        s.length += n
        return slots, pairs

    def _needed(self, seq: int, n: int) -> int:
        s = self.seqs[seq]
        bs = self.block_size
        if n == 0:
            return 0
        cow = s.length % bs != 0 and self.refcount[s.table[-1]] > 1
        return (s.length + n + bs - 1) // bs - len(s.table) + (1 if cow else 0)

    def append_batch(self, seqs, n_tokens) -> Tuple[List[int], List[Tuple[int, int]]]:
        """Append n_tokens[i] tokens to seqs[i], in order.  All or nothing: the
        blocks the batch needs, counted before any of it is applied, must be
        free."""
        seqs = [int(x) for x in seqs]
        n_tokens = [int(x) for x in n_tokens]
        if len(set(seqs)) != len(seqs):
            raise ValueError("a sequence appears twice in the batch")
        for x in seqs:
            if x not in self.seqs:
                raise KeyError(x)
        if any(n < 0 for n in n_tokens):
            raise ValueError("n < 0")
        need = sum(self._needed(x, n) for x, n in zip(seqs, n_tokens))
        if need > len(self._free):
            raise OutOfBlocks(f"{need} blocks needed, {len(self._free)} free")
        slots, pairs = [], []
        for x, n in zip(seqs, n_tokens):
            sl, pr = self.append(x, n)
            slots += sl
            pairs += pr
        return slots, pairs

    def free(self, seq: int):
        s = self.seqs.pop(seq)
        for b in s.table:
            self._release(b)

    def evict(self, seq: int, sink_tokens: int, window_tokens: int) -> int:
        """Sliding window with attention sinks, whole blocks at a time ("Paged
        Attention and Memory Efficiency in Production LLM Serving", section
        "Eviction, compression, and the challenge of fitting more KV cache
        into less memory": the first few tokens are kept as attention sinks
        next to a window of recent tokens, and eviction works on whole blocks
        of the paged layout).  A block may go only if none of its positions is
        among the first sink_tokens or the last window_tokens, and the block
        holding the newest position (the one the next token goes into) always
        stays; the blocks that go leave the table, which keeps its order.
        Returns the number of positions dropped."""
        s = self.seqs[seq]
        if sink_tokens < 0 or window_tokens < 0:
            raise ValueError("negative sink or window")
        bs, L = self.block_size, s.length
        keep = []
        for j, b in enumerate(s.table):
            first, last = j * bs, min(L, (j + 1) * bs) - 1  # positions block j holds
            in_sink = first < sink_tokens
            in_window = last >= L - window_tokens
            newest = j == len(s.table) - 1
            keep.append(in_sink or in_window or newest)
        gone = [j for j, k in enumerate(keep) if not k]
        assert all((j + 1) * bs <= L for j in gone)  # only full blocks can go
        for j in gone:
            self._release(s.table[j])
        s.table = [b for b, k in zip(s.table, keep) if k]
        s.length -= len(gone) * bs
        return len(gone) * bs

    def table(self, seq: int) -> List[int]:
        return list(self.seqs[seq].table)

    def length(self, seq: int) -> int:
        return self.seqs[seq].length

    # -- accounting -----------------------------------------------------------
    def stats(self) -> dict:
        """Token slots held by live sequences' tables (counting a shared block
        once per table that references it) against the tokens they hold, and
        the physical blocks in use."""
        held = sum(len(s.table) for s in self.seqs.values()) * self.block_size
        used = sum(s.length for s in self.seqs.values())
        in_use = self.num_blocks - len(self._free)
        shared = sum(1 for c in self.refcount if c > 1)
        return {"blocks_in_use": in_use, "blocks_free": len(self._free), "shared_blocks": shared,
                "slots_held": held, "tokens": used,
                "tail_waste": (held - used) / held if held else 0.0}
