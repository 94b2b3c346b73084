"""Host-side physical block pool with reference counts, fork and copy-on-write.

This is support code: it decides which physical block every logical block of
every sequence uses, which is what the Block Tables handed to the kernels hold.
It follows:

* "PagedAttention技术解析" section 2.1: each physical block carries a reference
  count and an allocation flag; allocation from a pool of free blocks is O(1);
  a child sequence can share its parent's blocks (a fork).
* Same page, section 4.2: a block is returned to the free pool as soon as its
  reference count drops to zero; a pool of free blocks is kept to make
  allocation cheap.
* "PagedAttention核心思想" section 2.4.3: shared blocks are read-only; a write
  into a block whose reference count is above one first copies the block
  (copy-on-write).  Reading taken: the writer that finds the count above one
  copies the block's valid tokens to a fresh block, drops its reference to the
  old one and repoints its table entry; a writer that finds the count at one
  writes in place.  The end state holds the same data whichever fork goes first.
* "VLLM中PagedAttention如何降低显存碎片？" section 三 items 7-8: the pool is carved
  into equal frames up front and handed out slab-style; common prompt prefixes
  are shared across requests.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np


class PoolExhausted(RuntimeError):
    """Raised when an allocation finds no free block."""


class BlockPool:
    """Fixed pool of ``num_blocks`` equal blocks handed out from a free list."""

    def __init__(self, num_blocks: int, order: Optional[Sequence[int]] = None):
        if num_blocks <= 0:
            raise ValueError("num_blocks must be positive")
        self.num_blocks = int(num_blocks)
        order = list(range(num_blocks)) if order is None else [int(b) for b in order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("order must be a permutation of the block ids")
        # pop() from the end is O(1); reverse so that order[0] is handed out first
        self._free: List[int] = order[::-1]
        self.ref = np.zeros(num_blocks, dtype=np.int64)

    @property
    def num_free(self) -> int:
        return len(self._free)

    def alloc(self) -> int:
        if not self._free:
            raise PoolExhausted("no free block left in the pool")
        b = self._free.pop()
        assert self.ref[b] == 0
        self.ref[b] = 1
        return b

    def incref(self, b: int) -> None:
        if self.ref[b] <= 0:
            raise ValueError(f"block {b} is not allocated")
        self.ref[b] += 1

    def decref(self, b: int) -> None:
        if self.ref[b] <= 0:
            raise ValueError(f"block {b} is not allocated (double free?)")
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self._free.append(b)

    def is_allocated(self, b: int) -> bool:
        return bool(self.ref[b] > 0)


@dataclass
class Sequence_:
    """One request: its Block Table (logical -> physical) and token count."""
    table: List[int] = field(default_factory=list)
    length: int = 0


@dataclass
class CowCopy:
    """A block copy the caller must perform on the device before the write."""
    src: int
    dst: int
    valid_tokens: int


class BlockManager:
    """Sequences over a ``BlockPool``: append, fork, copy-on-write, release."""

    def __init__(self, pool: BlockPool, block_size: int):
        if block_size <= 0:
            raise ValueError("block_size must be positive")
        self.pool = pool
        self.block_size = int(block_size)
        self.seqs: List[Sequence_] = []

    def new_sequence(self) -> int:
        self.seqs.append(Sequence_())
        return len(self.seqs) - 1

    def fork(self, parent: int) -> int:
        """New sequence sharing every block of ``parent`` (reference counted)."""
        p = self.seqs[parent]
        for b in p.table:
            self.pool.incref(b)
        self.seqs.append(Sequence_(table=list(p.table), length=p.length))
        return len(self.seqs) - 1

    def fork_many(self, parent: int, n: int) -> List[int]:
        """``n`` new sequences sharing every block of ``parent`` (parallel
        sampling or beam width ``n``): one reference count update per block."""
        if n < 0:
            raise ValueError("n must be non-negative")
        p = self.seqs[parent]
        for b in p.table:
            if self.pool.ref[b] <= 0:
                raise ValueError(f"block {b} is not allocated")
            self.pool.ref[b] += n
        first = len(self.seqs)
        self.seqs.extend(Sequence_(table=list(p.table), length=p.length) for _ in range(n))
        return list(range(first, first + n))

    def append_batch(self, sids: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
        """One new token for each sequence of ``sids``, in order.

        Returns the slot of every token (int64, the ``slot_mapping`` of the KV
        write) and the (src, dst) block pairs to copy (int64 [k, 2], the
        argument of the device block copy).  Sources and destinations are
        disjoint (a destination is freshly allocated), but a source can be
        written in the same batch: the last sequence still referencing it
        appends in place, into the row just past the copied ones.  So the copies
        must complete before the KV write of the batch: issue the block copy
        first, on the same stream as the write.
        """
        slots = np.empty(len(sids), dtype=np.int64)
        pairs = []
        for n, sid in enumerate(sids):
            slots[n], cow = self.append_token(sid)
            if cow is not None:
                pairs.append((cow.src, cow.dst))
        return slots, np.array(pairs, dtype=np.int64).reshape(-1, 2)

    def append_token(self, sid: int) -> Tuple[int, Optional[CowCopy]]:
        """Reserve the slot of the sequence's next token.

        Returns ``(slot, cow)`` with ``slot = physical_block * block_size +
        offset``; ``cow`` is a copy the caller must carry out first when the
        last block was shared.
        """
        s = self.seqs[sid]
        off = s.length % self.block_size
        cow = None
        if off == 0:
            s.table.append(self.pool.alloc())
        else:
            last = s.table[-1]
            if self.pool.ref[last] > 1:
                dst = self.pool.alloc()
                self.pool.decref(last)
                s.table[-1] = dst
                cow = CowCopy(src=last, dst=dst, valid_tokens=off)
        slot = s.table[-1] * self.block_size + off
        s.length += 1
        return slot, cow

    def release(self, sid: int) -> None:
        """Drop the sequence's references; blocks reaching zero are freed."""
        s = self.seqs[sid]
        for b in s.table:
            self.pool.decref(b)
        s.table = []
        s.length = 0

    def table_refs(self) -> np.ndarray:
        """Reference count implied by the tables (for invariant checks)."""
        cnt = np.zeros(self.pool.num_blocks, dtype=np.int64)
        for s in self.seqs:
            for b in s.table:
                cnt[b] += 1
        return cnt


def preallocation_waste(used_tokens: float, reserved_tokens: float) -> float:
    """Fraction of a contiguous per-request reservation left unused.

    "PagedAttention核心思想" section 2.4.2 works this out for requests that use
    128 tokens of a 2048-token reservation; the CSDN answer, section 一, for 8k
    of a 32k reservation.
    """
    if reserved_tokens <= 0:
        raise ValueError("reserved_tokens must be positive")
    return 1.0 - float(used_tokens) / float(reserved_tokens)


def paged_waste_tokens(length: int, block_size: int) -> int:
    """Unused slots when a sequence of ``length`` tokens is held in blocks."""
    nblocks = -(-length // block_size)
    return nblocks * block_size - length
