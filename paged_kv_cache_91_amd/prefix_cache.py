"""Host prefix-cache lookup: full KV blocks keyed by content so that a new
request whose prompt starts like an earlier one reuses that request's
blocks instead of computing them again.

It sits on the host beside the block allocator and feeds the same kernels:
a hit hands out block ids (reference counts go up, as for any shared block),
and only the positions after the cached prefix need K/V computed and
written, which is a chunked prefill (``pa_prefill`` with L = n - cached).

Behaviour follows the pages:

* a full block is identified by its parent block's key, the tokens it holds
  and the conditions that change its K/V (vasteelab.pages.dev
  "PagedAttentionとは？", section "Prefix Cachingとの違い": the parent block's
  hash, the block's tokens, the LoRA id, multimodal input hashes); chaining
  through the parent means a block matches only when the whole prefix before
  it matches;
* hashing whole blocks extends sharing across requests (ultralytics.com
  "PagedAttention", section "시퀀스 간 블록 공유"), and blocks fill up before
  they are entered (zerocoder.ru "Что такое PagedAttention": blocks with
  computed state go into the lookup structure as they fill; a new request is
  looked up and matching blocks are reused instead of computed);
* blocks nobody references stay cached on the free list until a fresh block
  is needed; eviction takes uncached free blocks first, then cached ones by
  priority 0 .. 100, least recently released first among equal priorities
  (zerocoder.ru, the TensorRT LLM reuse paragraph).  The pages do not say
  which end of the priority range goes first; here the lowest does.
"""

from __future__ import annotations

import hashlib
import struct
from typing import Dict, List, Optional, Sequence, Tuple


from .allocator import AllocatorError, BlockAllocator, OutOfBlocks

ROOT_KEY = b"\x00" * 16          # parent key of a sequence's first block


def block_key(parent: bytes, tokens: Sequence[int], extra: bytes = b"") -> bytes:
    """Key of one full block: a 16-byte digest of the parent block's key, the
    block's token ids and ``extra`` (the conditions that change K/V: adapter
    id, multimodal input hashes, ...)."""
    h = hashlib.blake2b(digest_size=16)
    h.update(parent)
    h.update(struct.pack(f"<{len(tokens)}q", *[int(t) for t in tokens]))
    h.update(struct.pack("<q", len(extra)))
    h.update(extra)
    return h.digest()


class PrefixCachingAllocator(BlockAllocator):
    """BlockAllocator whose full blocks can be found again by content."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None, host_blocks: int = 0):
        super().__init__(num_blocks, block_size, free_order=free_order, host_blocks=host_blocks)
        self._key_of: Dict[int, bytes] = {}          # cached block -> key
        self._block_of: Dict[bytes, int] = {}        # key -> cached block
        self._priority: Dict[int, int] = {}          # cached block -> eviction priority
        self._released_at: Dict[int, int] = {}       # cached free block -> release tick
        self._tick = 0
        self.hits = 0                                # blocks reused by lookups
        self.misses = 0                              # full prompt blocks that had to be computed

    # -- keys ----------------------------------------------------------------

    def prompt_keys(self, tokens: Sequence[int], extra: bytes = b"") -> List[bytes]:
        """Keys of the full blocks of ``tokens``, each chained to the one before."""
        keys, parent = [], ROOT_KEY
        bs = self.block_size
        for i in range(len(tokens) // bs):
            parent = block_key(parent, tokens[i * bs:(i + 1) * bs], extra)
            keys.append(parent)
        return keys

    def cached_blocks(self) -> int:
        return len(self._block_of)

    # -- allocation with lookup ----------------------------------------------

    def add_prompt(self, seq_id: int, tokens: Sequence[int], extra: bytes = b"") -> Tuple[List[int], int]:
        """Register a sequence holding the prompt ``tokens``: the longest
        chain of its full blocks already cached is reused, the rest comes
        from the free pool.  Returns (block table, cached positions): K/V
        must be computed and written only for positions from the second
        value on.  At least the last prompt position is always computed
        (its query is needed), so a fully cached prompt keeps its last
        block fresh.  All or nothing: OutOfBlocks leaves no trace."""
        if seq_id in self._tables or seq_id in self._swapped:
            raise AllocatorError(f"sequence {seq_id} exists")
        n, bs = len(tokens), self.block_size
        keys = self.prompt_keys(tokens, extra)
        hit = []
        for key in keys:
            b = self._block_of.get(key)
            if b is None:
                break
            hit.append(b)
        if hit and len(hit) * bs >= n:          # keep the last position's block computed
            hit.pop()
        need = -(-n // bs) - len(hit)
        revived = sum(1 for b in hit if self._refcount[b] == 0)
        if need > len(self._free) - revived:
            raise OutOfBlocks(f"prompt needs {need} fresh blocks, {len(self._free) - revived} free")
        for b in hit:
            if self._refcount[b] == 0:           # cached but free: back in use
                self._free.remove(b)
                self._released_at.pop(b, None)
            self._refcount[b] += 1
        table = hit + [self._take() for _ in range(need)]
        self._tables[seq_id] = table
        self._lengths[seq_id] = n
        self.hits += len(hit)
        self.misses += len(keys) - len(hit)
        return list(table), len(hit) * bs

    def commit(self, seq_id: int, tokens: Sequence[int], extra: bytes = b"", priority: int = 35) -> int:
        """Enter the full blocks of ``seq_id`` (whose first positions hold
        ``tokens``, K/V written) into the cache; a key already cached keeps
        its block.  Returns how many blocks were entered."""
        if not 0 <= priority <= 100:
            raise ValueError("priority must be in [0, 100]")
        if seq_id not in self._tables:
            raise AllocatorError(f"sequence {seq_id} is not resident")
        table = self._tables[seq_id]
        if len(tokens) > self._lengths[seq_id]:
            raise AllocatorError("more tokens than the sequence holds")
        added = 0
        for i, key in enumerate(self.prompt_keys(tokens, extra)):
            b = table[i]
            if key in self._block_of or b in self._key_of or b < 0:
                continue
            self._block_of[key] = b
            self._key_of[b] = key
            self._priority[b] = priority
            added += 1
        return added

    # -- eviction --------------------------------------------------------------

    def _release(self, b: int) -> None:
        super()._release(b)
        if self._refcount[b] == 0 and b in self._key_of:
            self._tick += 1
            self._released_at[b] = self._tick

    def _take(self) -> int:
        """A fresh block: uncached free blocks first (in free-list order),
        else the cached free block of lowest priority, least recently
        released first; its cache entry is dropped."""
        if not self._free:
            raise OutOfBlocks("no free block in the pool")
        for b in self._free:
            if b not in self._key_of:
                self._free.remove(b)
                self._refcount[b] = 1
                return b
        victim = min(self._free, key=lambda b: (self._priority[b], self._released_at.get(b, 0)))
        self._free.remove(victim)
        key = self._key_of.pop(victim)
        del self._block_of[key]
        del self._priority[victim]
        self._released_at.pop(victim, None)
        self._refcount[victim] = 1
        return victim

    def copy_on_write(self, seq_id: int, logical_block: int) -> Optional[Tuple[int, int]]:
        """As BlockAllocator's; a cached block is never written in place, so
        a sequence about to write into a cached block it holds alone gets a
        private copy too."""
        table = self._tables[seq_id]
        src = table[logical_block]
        if self._refcount[src] <= 1 and src not in self._key_of:
            return None
        dst = self._take()
        self._refcount[src] -= 1
        if self._refcount[src] == 0:
            self._free.append(src)
            self._tick += 1
            self._released_at[src] = self._tick
        table[logical_block] = dst
        self._cow_copies += 1
        return (src, dst)

    def check(self) -> None:
        super().check()
        if set(self._key_of) != set(self._block_of.values()) or len(self._key_of) != len(self._block_of):
            raise AllocatorError("cache maps disagree")
        for key, b in self._block_of.items():
            if self._key_of.get(b) != key:
                raise AllocatorError("cache maps disagree")
        free = set(self._free)
        for b in self._released_at:
            if b not in free or b not in self._key_of:
                raise AllocatorError("a release time for a block that is not a free cached block")
