"""Host-side block manager that feeds block tables, slot mappings and
copy-on-write pairs to the GPU kernels.

It is not on the GPU hot path: it decides *where* tokens go, the kernels move
and read the bytes.  Behaviour follows the pages:

* a sequence of n tokens holds ceil(n / block_size) blocks, and a new block
  is taken only when the last one is full, from wherever a free block is
  (gufacode.com "PagedAttention:KV cache 的页表革命", section "按需分配 demo";
  ultralytics.com glossary "PagedAttention", section "페이징의 작동 방식");
* the free list is first-in first-out, as in the pool example of that
  ultralytics section, where free blocks are popped from the front;
* a finished sequence's blocks return to the pool (zerocoder.ru "Что такое
  PagedAttention", worked trace; vasteelab.pages.dev "PagedAttentionとは？",
  section "tokenを固定長blockへ分ける");
* several tables may name the same physical block; each block carries a
  reference count, and a sequence that must write into a block that others
  still reference first receives a private copy (vasteelab.pages.dev,
  section "Copy-on-Writeで共通prefixを共有できる"; ultralytics.com, section
  "시퀀스 간 블록 공유"; gufacode.com, section "前缀共享:Copy-on-Write");
* the structural checks of zerocoder.ru's worked trace: tables name existing
  blocks, reference counts agree with the tables, and freeing leaves no
  dangling entries;
* when the pool runs out, every block of a sequence can be moved to a swap
  area in host memory and its GPU blocks freed, then brought back later into
  whatever GPU blocks are free (gufacode.com, section "Swap 到 CPU:兜底溢出";
  vasteelab.pages.dev, section "blockが足りなくなったとき");
* under a sliding attention window, blocks that lie wholly before the window
  are released (zerocoder.ru, section "Где подход не решает задачу";
  vasteelab.pages.dev, section "hybrid modelではblock設計が複雑になる"); their
  table entries stay as RELEASED placeholders so logical block j is still
  entry j, and the windowed decode never reads them.
"""

from __future__ import annotations

from collections import deque
from dataclasses import dataclass
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np


class OutOfBlocks(RuntimeError):
    """The pool has no free block left."""


class AllocatorError(RuntimeError):
    """A request that would break the allocator's invariants."""


@dataclass
class AllocatorStats:
    total_blocks: int
    used_blocks: int
    free_blocks: int
    shared_blocks: int          # physical blocks referenced by more than one table
    cow_copies: int             # copy-on-write pairs emitted so far
    waste_slots: int            # unused slots in the last block of every sequence
    tokens: int                 # sum of sequence lengths


RELEASED = -1   # table entry of a block released under a sliding window


class BlockAllocator:
    """Free list + reference counts + per-sequence block tables (+ an
    optional host swap area of ``host_blocks`` blocks)."""

    def __init__(self, num_blocks: int, block_size: int,
                 free_order: Optional[Iterable[int]] = None, host_blocks: int = 0):
        if num_blocks <= 0:
            raise ValueError("num_blocks must be positive")
        if block_size <= 1 or block_size & (block_size - 1):
            raise ValueError("block_size must be a power of two greater than one")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if len(order) != len(set(order)) or any(b < 0 or b >= num_blocks for b in order):
            raise ValueError("free_order must list distinct block ids inside the pool")
        self._free: deque = deque(order)
        # blocks left off the initial free list belong to someone else (as in
        # a pool whose other blocks other requests already hold)
        self._reserved = frozenset(range(num_blocks)) - frozenset(order)
        self._refcount = np.zeros(num_blocks, dtype=np.int64)
        self._tables: Dict[int, List[int]] = {}
        self._lengths: Dict[int, int] = {}
        self._cow_copies = 0
        self.host_blocks = 0
        self._host_free: deque = deque()
        self._swapped: Dict[int, Tuple[List[int], int]] = {}   # seq -> (host table, length)
        self.add_host_area(host_blocks)

    def add_host_area(self, host_blocks: int) -> None:
        """Grow the host swap area by ``host_blocks`` slots (ids continue
        from the current size)."""
        if host_blocks < 0:
            raise ValueError("host_blocks must be >= 0")
        self._host_free.extend(range(self.host_blocks, self.host_blocks + host_blocks))
        self.host_blocks += host_blocks

    # -- queries ---------------------------------------------------------

    def block_table(self, seq_id: int) -> List[int]:
        return list(self._tables[seq_id])

    def length(self, seq_id: int) -> int:
        return self._lengths[seq_id]

    def refcount(self, block: int) -> int:
        return int(self._refcount[block])

    def free_block_ids(self) -> List[int]:
        return list(self._free)

    @property
    def num_free(self) -> int:
        return len(self._free)

    def sequences(self) -> List[int]:
        return list(self._tables)

    def slot(self, seq_id: int, pos: int) -> int:
        """Flat pool slot of position ``pos``: block * block_size + offset."""
        if not 0 <= pos < self._lengths[seq_id]:
            raise AllocatorError(f"position {pos} outside sequence {seq_id}")
        table = self._tables[seq_id]
        if table[pos // self.block_size] == RELEASED:
            raise AllocatorError(f"position {pos} lies in a released block")
        return table[pos // self.block_size] * self.block_size + pos % self.block_size

    def slots(self, seq_id: int, start: int, stop: int) -> np.ndarray:
        """Slots of positions [start, stop) as int64."""
        if not 0 <= start <= stop <= self._lengths[seq_id]:
            raise AllocatorError("slot range outside the sequence")
        table = np.asarray(self._tables[seq_id], dtype=np.int64)
        pos = np.arange(start, stop, dtype=np.int64)
        if (table[pos // self.block_size] == RELEASED).any():
            raise AllocatorError("slot range reaches a released block")
        return table[pos // self.block_size] * self.block_size + pos % self.block_size

    def tables_array(self, seq_ids: Sequence[int], max_blocks: Optional[int] = None,
                     pad: int = 0) -> np.ndarray:
        """``int32 [len(seq_ids), max_blocks]`` table, padded with ``pad``."""
        rows = [self._tables[s] for s in seq_ids]
        width = max((len(r) for r in rows), default=0) if max_blocks is None else max_blocks
        out = np.full((len(rows), max(width, 1)), pad, dtype=np.int32)
        for i, r in enumerate(rows):
            if len(r) > width:
                raise AllocatorError("max_blocks smaller than a table")
            out[i, :len(r)] = r
        return out

    def swapped(self) -> List[int]:
        return list(self._swapped)

    @property
    def num_host_free(self) -> int:
        return len(self._host_free)

    def stats(self) -> AllocatorStats:
        used = int((self._refcount > 0).sum())
        return AllocatorStats(
            total_blocks=self.num_blocks,
            used_blocks=used,
            free_blocks=len(self._free),
            shared_blocks=int((self._refcount > 1).sum()),
            cow_copies=self._cow_copies,
            waste_slots=sum(len(t) * self.block_size - self._lengths[s]
                            for s, t in self._tables.items() if t),
            tokens=sum(self._lengths.values()),
        )

    # -- mutations -------------------------------------------------------

    def _take(self) -> int:
        if not self._free:
            raise OutOfBlocks("no free block in the pool")
        b = self._free.popleft()
        self._refcount[b] = 1
        return b

    def _release(self, b: int) -> None:
        if self._refcount[b] <= 0:
            raise AllocatorError(f"reference count underflow on block {b}")
        self._refcount[b] -= 1
        if self._refcount[b] == 0:
            self._free.append(b)

    def add_sequence(self, seq_id: int, num_tokens: int = 0) -> List[int]:
        """Register a sequence holding ``num_tokens`` tokens (a prompt)."""
        if seq_id in self._tables or seq_id in self._swapped:
            raise AllocatorError(f"sequence {seq_id} exists")
        need = -(-num_tokens // self.block_size)
        if need > len(self._free):
            raise OutOfBlocks(f"sequence needs {need} blocks, {len(self._free)} free")
        self._tables[seq_id] = [self._take() for _ in range(need)]
        self._lengths[seq_id] = int(num_tokens)
        return self.block_table(seq_id)

    def append_tokens(self, seq_id: int, count: int = 1) -> Tuple[np.ndarray, List[Tuple[int, int]]]:
        """Grow a sequence by ``count`` tokens.

        Returns the new tokens' slots and the copy-on-write pairs the caller
        must apply (``pa_copy_blocks``) before writing them: a token that
        lands in a partly filled last block that other tables share triggers
        a copy of that block to a fresh one.

        The call is all or nothing: the fresh blocks it needs (one per block
        boundary crossed, plus one for a copy-on-write of a shared partly
        filled last block, which can only concern the first new token) are
        counted first, and OutOfBlocks is raised before anything changes.
        """
        if count < 0:
            raise AllocatorError("count must be >= 0")
        table = self._tables[seq_id]
        start = self._lengths[seq_id]
        fresh = -(-(start + count) // self.block_size) - -(-start // self.block_size)
        cow = count > 0 and start % self.block_size != 0 and \
            self._refcount[table[start // self.block_size]] > 1
        if fresh + int(cow) > len(self._free):
            raise OutOfBlocks(f"append of {count} tokens needs {fresh + int(cow)} blocks, "
                              f"{len(self._free)} free")
        pairs: List[Tuple[int, int]] = []
        slots = np.empty(count, dtype=np.int64)
        for i in range(count):
            pos = self._lengths[seq_id]
            if pos % self.block_size == 0:
                table.append(self._take())
            else:
                pair = self.copy_on_write(seq_id, pos // self.block_size)
                if pair is not None:
                    pairs.append(pair)
            self._lengths[seq_id] = pos + 1
            slots[i] = table[pos // self.block_size] * self.block_size + pos % self.block_size
        return slots, pairs

    def copy_on_write(self, seq_id: int, logical_block: int) -> Optional[Tuple[int, int]]:
        """Give ``seq_id`` a private copy of one of its blocks if it is shared.

        Returns ``(src, dst)`` for the block copy, or None if the block was
        already private.
        """
        table = self._tables[seq_id]
        src = table[logical_block]
        if self._refcount[src] <= 1:
            return None
        dst = self._take()
        self._refcount[src] -= 1
        table[logical_block] = dst
        self._cow_copies += 1
        return (src, dst)

    def fork(self, parent_id: int, child_id: int) -> List[int]:
        """New sequence sharing every block of ``parent_id`` (refcounts + 1)."""
        if child_id in self._tables or child_id in self._swapped:
            raise AllocatorError(f"sequence {child_id} exists")
        table = list(self._tables[parent_id])
        for b in table:
            if b != RELEASED:
                self._refcount[b] += 1
        self._tables[child_id] = table
        self._lengths[child_id] = self._lengths[parent_id]
        return list(table)

    def free(self, seq_id: int) -> None:
        """Return a finished sequence's blocks (shared ones lose one reference)."""
        if seq_id in self._swapped:
            host, _ = self._swapped.pop(seq_id)
            self._host_free.extend(h for h in host if h != RELEASED)
            return
        if seq_id not in self._tables:
            raise AllocatorError(f"sequence {seq_id} unknown or already freed")
        for b in self._tables.pop(seq_id):
            if b != RELEASED:
                self._release(b)
        del self._lengths[seq_id]

    # -- sliding window --------------------------------------------------

    def release_before_window(self, seq_id: int, window: int) -> List[int]:
        """Release the blocks of ``seq_id`` that lie wholly before its sliding
        window: with n tokens the window starts at lo = max(0, n - window), so
        logical blocks j < lo // block_size hold no position the next decode
        step reads.  Their entries become RELEASED; shared blocks lose one
        reference.  Returns the block ids released by this call."""
        if window <= 0:
            return []
        table = self._tables[seq_id]
        lo = max(0, self._lengths[seq_id] - window)
        out = []
        for j in range(lo // self.block_size):
            b = table[j]
            if b != RELEASED:
                self._release(b)
                table[j] = RELEASED
                out.append(b)
        return out

    # -- swap to the host area ---------------------------------------------

    def swap_out(self, seq_id: int) -> List[Tuple[int, int]]:
        """Move every block of ``seq_id`` to host slots and free its GPU
        blocks (shared ones lose one reference).  Returns the (GPU block,
        host slot) copies to apply, e.g. with pa_swap_blocks, on the stream
        ahead of any later write into the freed blocks.  All or nothing:
        OutOfBlocks if the host area lacks the slots."""
        table = self._tables[seq_id]
        live = [b for b in table if b != RELEASED]
        if len(live) > len(self._host_free):
            raise OutOfBlocks(f"swap-out needs {len(live)} host slots, {len(self._host_free)} free")
        host = [RELEASED if b == RELEASED else self._host_free.popleft() for b in table]
        for b in live:
            self._release(b)
        self._swapped[seq_id] = (host, self._lengths.pop(seq_id))
        del self._tables[seq_id]
        return [(b, h) for b, h in zip(table, host) if b != RELEASED]

    def swap_in(self, seq_id: int) -> List[Tuple[int, int]]:
        """Bring a swapped-out sequence back into free GPU blocks.  Returns
        the (host slot, GPU block) copies to apply before the sequence is
        read; its host slots are free again once those copies are ordered
        ahead of any later swap-out on the same stream.  All or nothing."""
        if seq_id not in self._swapped:
            raise AllocatorError(f"sequence {seq_id} is not swapped out")
        host, n = self._swapped[seq_id]
        live = [h for h in host if h != RELEASED]
        if len(live) > len(self._free):
            raise OutOfBlocks(f"swap-in needs {len(live)} blocks, {len(self._free)} free")
        table = [RELEASED if h == RELEASED else self._take() for h in host]
        del self._swapped[seq_id]
        self._tables[seq_id] = table
        self._lengths[seq_id] = n
        self._host_free.extend(live)
        return [(h, b) for h, b in zip(host, table) if h != RELEASED]

    # -- structural checks -----------------------------------------------

    def check(self) -> None:
        """Raise AllocatorError unless the structure is consistent."""
        counts = np.zeros(self.num_blocks, dtype=np.int64)
        for s, table in self._tables.items():
            if len(table) != -(-self._lengths[s] // self.block_size):
                raise AllocatorError(f"sequence {s}: table does not cover its tokens")
            live = [b for b in table if b != RELEASED]
            if table[:len(table) - len(live)] != [RELEASED] * (len(table) - len(live)):
                raise AllocatorError(f"sequence {s}: released entries must be a prefix")
            if table and table[-1] == RELEASED:
                raise AllocatorError(f"sequence {s}: the last block was released")
            for b in live:
                if not 0 <= b < self.num_blocks:
                    raise AllocatorError(f"sequence {s}: block {b} outside the pool")
                counts[b] += 1
        host_used = [h for host, _ in self._swapped.values() for h in host if h != RELEASED]
        if set(self._swapped) & set(self._tables):
            raise AllocatorError("a sequence is both resident and swapped out")
        if len(set(host_used)) != len(host_used) or set(host_used) & set(self._host_free) or \
                len(host_used) + len(self._host_free) != self.host_blocks or \
                any(not 0 <= h < self.host_blocks for h in host_used):
            raise AllocatorError("host swap slots are inconsistent")
        if not np.array_equal(counts, self._refcount):
            raise AllocatorError("reference counts disagree with the tables")
        free = list(self._free)
        if len(set(free)) != len(free):
            raise AllocatorError("a block is on the free list twice")
        if any(counts[b] for b in free):
            raise AllocatorError("a referenced block is on the free list")
        if any(counts[b] or b in free for b in self._reserved):
            raise AllocatorError("a block held outside this allocator is in use here")
        if len(free) + int((counts > 0).sum()) + len(self._reserved) != self.num_blocks:
            raise AllocatorError("a block is neither free nor referenced")
