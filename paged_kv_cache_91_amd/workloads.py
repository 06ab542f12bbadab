"""Seeded synthetic inputs for the paged decode path.

This module only draws inputs.  It holds none of the method's arithmetic: no
attention, no quantisation and no per-token scatter.  Block contents are
drawn per logical block and dropped into the pool at the block ids the
allocator hands out.  The same host arrays feed the GPU library and the
float64 oracle.

Recipe (per workload, from one integer seed):

1. context lengths, from ``numpy.random.default_rng(seed)``;
2. the pool's free list, a random permutation of all block ids from the
   same generator; sequences take blocks from it in sequence order;
3. K and V block contents, then q (and new-token rows where a workload has
   them), as float32 N(0, 1) from counter-keyed streams
   ``default_rng([seed, stream, chunk])``, cast to the storage dtype with
   round-to-nearest-even.

Storage dtypes follow the oracle's conventions: f32 -> float32,
f16 -> float16, bf16 -> uint16 bit patterns, fp8_e4m3 -> uint8 codes.

The five named workloads mirror the decode shapes the pages discuss: a tiny
fp32 case shaped like zerocoder.ru's worked example (block 4, lengths 6 and
3), a Llama-3-8B-shaped GQA layer at block 16 (gufacode.com's sizing example
model; the default block size of 16 from ultralytics.com), a 13B-shaped MHA
layer with a heavy-tailed length mix plus a one-token cache write, a shared
80-token system prompt with copy-on-write (gufacode.com, section
"前缀共享:Copy-on-Write"), and a long-context fp8 cache (ultralytics.com,
section "관련 기법").
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import numpy as np
import torch

from .allocator import BlockAllocator

ELEMENT_SIZE = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}
STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8_e4m3": np.uint8}
NAN_BITS = {"f32": np.float32(np.nan), "f16": np.float16(np.nan),
            "bf16": np.uint16(0x7FC0), "fp8_e4m3": np.uint8(0x7F)}

# stream ids for the counter-keyed generators
_S_K, _S_V, _S_Q, _S_NEWK, _S_NEWV = 1, 2, 3, 4, 5
_CHUNK = 1 << 20


# ---------------------------------------------------------------------------
# random streams
# ---------------------------------------------------------------------------

def normal_f32(seed: int, stream: int, count: int) -> np.ndarray:
    """``count`` float32 N(0,1) values from stream ``stream`` of ``seed``.

    Chunk i of 2**20 values comes from ``default_rng([seed, stream, i])``, so
    the result does not depend on how many threads fill it.
    """
    out = np.empty(count, dtype=np.float32)
    nchunks = -(-count // _CHUNK)

    def fill(i):
        lo, hi = i * _CHUNK, min(count, (i + 1) * _CHUNK)
        np.random.default_rng([seed, stream, i]).standard_normal(
            out=out[lo:hi], dtype=np.float32)

    workers = max(1, min(16, len(os.sched_getaffinity(0)), nchunks))
    if workers == 1:
        for i in range(nchunks):
            fill(i)
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def cast_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to a storage dtype (nearest, ties to even)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float32).astype(np.float16)
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(f"cannot draw values directly in {dtype}")


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Float32 value of bf16 bit patterns (used for the fp8 scale's amax)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# workload container
# ---------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    q_dtype: str
    kv_dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    q: np.ndarray                      # [S, Hq, D] storage dtype
    k_pool: np.ndarray                 # [N, Hkv, bs, D] storage dtype
    v_pool: np.ndarray
    block_tables: np.ndarray           # int32 [S, maxb]
    context_lens: np.ndarray           # int32 [S]
    scale: float                       # float32 softmax scale
    k_scale: float = 1.0               # float32 per-tensor scales (fp8 pools)
    v_scale: float = 1.0
    partition_size: int = 0
    # write side: rows [T, Hkv, D] in write_src_dtype, slots int64 [T]
    write_src_dtype: Optional[str] = None
    write_k: Optional[np.ndarray] = None
    write_v: Optional[np.ndarray] = None
    slot_mapping: Optional[np.ndarray] = None
    # copy side: int64 [P, 2]; tables as they were before the copy
    copy_pairs: Optional[np.ndarray] = None
    tables_before_copy: Optional[np.ndarray] = None
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.q.shape[0])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes one decode reads: exactly context_len
        positions per sequence, all KV heads, K and V."""
        per_pos = 2 * self.num_kv_heads * self.head_dim * ELEMENT_SIZE[self.kv_dtype]
        return int(self.context_lens.astype(np.int64).sum()) * per_pos


# ---------------------------------------------------------------------------
# generic builder
# ---------------------------------------------------------------------------

def _draw_contents(seed: int, stream: int, nblocks: int, hkv: int, bs: int, d: int,
                   dtype: str) -> np.ndarray:
    vals = normal_f32(seed, stream, nblocks * hkv * bs * d)
    return cast_f32(vals, dtype).reshape(nblocks, hkv, bs, d)


def _place(pool_shape, dtype, used_ids, contents, fill_nan) -> np.ndarray:
    if fill_nan:
        pool = np.full(pool_shape, NAN_BITS[dtype], dtype=STORAGE[dtype])
    else:
        pool = np.zeros(pool_shape, dtype=STORAGE[dtype])
    if len(used_ids):
        pool[used_ids] = contents
    return pool


def _poison_tails(pool, tables, lens, bs, dtype):
    """NaN the slots at and after context_len inside each last block."""
    for s, n in enumerate(lens):
        n = int(n)
        if n % bs:
            pool[tables[s, n // bs], :, n % bs:, :] = NAN_BITS[dtype]


def build_decode(seed: int, *, name: str, q_dtype: str, kv_dtype: str,
                 num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                 num_blocks: int, context_lens: Sequence[int], partition_size: int = 0,
                 rng: Optional[np.random.Generator] = None, poison: bool = False,
                 max_blocks_per_seq: Optional[int] = None) -> Workload:
    """Random-content paged decode workload.

    ``rng`` must be the generator the lengths came from (the permutation is
    drawn next from it); block contents come from counter streams.  With
    ``poison`` every slot no sequence may read (unused blocks, the tail of
    each last block) holds NaN, and table padding names a NaN block.
    """
    if rng is None:
        rng = np.random.default_rng(seed)
    lens = np.asarray(context_lens, dtype=np.int32)
    perm = rng.permutation(num_blocks)
    alloc = BlockAllocator(num_blocks, block_size, free_order=perm)
    for s, n in enumerate(lens):
        alloc.add_sequence(s, int(n))
    need = [math.ceil(int(n) / block_size) for n in lens]
    maxb = max_blocks_per_seq or max(max(need, default=1), 1)
    pad = 0
    if poison:
        if alloc.num_free == 0:
            raise ValueError("poisoned workload needs one spare block")
        pad = alloc.free_block_ids()[0]
    tables = alloc.tables_array(range(len(lens)), maxb, pad=pad)
    used = np.concatenate([np.asarray(alloc.block_table(s), dtype=np.int64)
                           for s in range(len(lens))] or [np.zeros(0, np.int64)])
    pool_shape = (num_blocks, num_kv_heads, block_size, head_dim)
    draw_dtype = "bf16" if kv_dtype == "fp8_e4m3" else kv_dtype
    if kv_dtype == "fp8_e4m3":
        raise ValueError("fp8 pools are filled through the cache write (see config5)")
    kc = _draw_contents(seed, _S_K, len(used), num_kv_heads, block_size, head_dim, draw_dtype)
    vc = _draw_contents(seed, _S_V, len(used), num_kv_heads, block_size, head_dim, draw_dtype)
    k_pool = _place(pool_shape, kv_dtype, used, kc, poison)
    v_pool = _place(pool_shape, kv_dtype, used, vc, poison)
    del kc, vc
    if poison:
        _poison_tails(k_pool, tables, lens, block_size, kv_dtype)
        _poison_tails(v_pool, tables, lens, block_size, kv_dtype)
    q = cast_f32(normal_f32(seed, _S_Q, len(lens) * num_q_heads * head_dim),
                 q_dtype).reshape(len(lens), num_q_heads, head_dim)
    return Workload(
        name=name, q_dtype=q_dtype, kv_dtype=kv_dtype, num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
        num_blocks=num_blocks, q=q, k_pool=k_pool, v_pool=v_pool, block_tables=tables,
        context_lens=lens, scale=float(np.float32(1.0 / math.sqrt(head_dim))),
        partition_size=partition_size,
        meta={"seed": seed, "alloc": alloc.stats(), "poison": poison, "pad_block": pad, "allocator": alloc})


def relocate(wl: Workload, seed: int) -> Workload:
    """Same logical contents under a fresh random bijection of block ids.

    Every block b moves to ``perm[b]`` and the tables are renamed to match,
    so each sequence sees exactly the same K/V in the same logical order.
    """
    perm = np.random.default_rng(seed).permutation(wl.num_blocks)
    k_pool = np.empty_like(wl.k_pool)
    v_pool = np.empty_like(wl.v_pool)
    k_pool[perm] = wl.k_pool
    v_pool[perm] = wl.v_pool
    tables = perm[wl.block_tables].astype(np.int32)
    out = replace(wl, k_pool=k_pool, v_pool=v_pool, block_tables=tables,
                  meta=dict(wl.meta, relocated=seed))
    if wl.slot_mapping is not None:
        bs = wl.block_size
        out.slot_mapping = perm[wl.slot_mapping // bs] * bs + wl.slot_mapping % bs
    if wl.copy_pairs is not None:
        out.copy_pairs = perm[wl.copy_pairs]
        out.tables_before_copy = perm[wl.tables_before_copy].astype(np.int32)
    return out


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def config1(seed: int = 1, poison: bool = False) -> Workload:
    """Tiny fp32 decode: 1 head, head_dim 8, block 4, pool 16, lengths 6 and 3
    on random distinct blocks (the shape of zerocoder.ru's worked example)."""
    rng = np.random.default_rng(seed)
    return build_decode(seed, name="tiny-fp32", q_dtype="f32", kv_dtype="f32",
                        num_q_heads=1, num_kv_heads=1, head_dim=8, block_size=4,
                        num_blocks=16, context_lens=[6, 3], rng=rng, poison=poison)


def config2(seed: int = 2, num_seqs: int = 64, ctx_range=(128, 2048),
            num_blocks: int = 16384, partition_size: int = 0,
            poison: bool = False) -> Workload:
    """Llama-3-8B-shaped decode layer, bf16: 32 q heads on 8 KV heads,
    head_dim 128, block 16, lengths uniform in ``ctx_range`` (inclusive)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(ctx_range[0], ctx_range[1] + 1, size=num_seqs)
    return build_decode(seed, name="llama3-8b-gqa4-bf16", q_dtype="bf16", kv_dtype="bf16",
                        num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                        num_blocks=num_blocks, context_lens=lens,
                        partition_size=partition_size, rng=rng, poison=poison)


def lognormal_lengths(rng, num_seqs, median=512, sigma=1.0, lo=16, hi=4096):
    """Heavy-tailed length mix: clip(rint(exp(ln(median) + sigma Z)), lo, hi)."""
    z = rng.standard_normal(num_seqs)
    return np.clip(np.rint(np.exp(math.log(median) + sigma * z)), lo, hi).astype(np.int64)


def config3(seed: int = 3, num_seqs: int = 256, num_blocks: int = 65536,
            length_cap: int = 4096, poison: bool = False) -> Workload:
    """13B-shaped MHA decode, fp16: 40 heads, head_dim 128, block 16,
    lognormal lengths (median 512, sigma 1, clipped to [16, length_cap]),
    plus a cache write of one new token per sequence at position n-1."""
    rng = np.random.default_rng(seed)
    lens = lognormal_lengths(rng, num_seqs, hi=length_cap)
    wl = build_decode(seed, name="13b-mha-fp16", q_dtype="f16", kv_dtype="f16",
                      num_q_heads=40, num_kv_heads=40, head_dim=128, block_size=16,
                      num_blocks=num_blocks, context_lens=lens, rng=rng, poison=poison)
    bs = wl.block_size
    pos = wl.context_lens.astype(np.int64) - 1
    rows = np.arange(num_seqs)
    wl.slot_mapping = wl.block_tables[rows, pos // bs].astype(np.int64) * bs + pos % bs
    shape = (num_seqs, wl.num_kv_heads, wl.head_dim)
    wl.write_src_dtype = "f16"
    wl.write_k = cast_f32(normal_f32(seed, _S_NEWK, int(np.prod(shape))), "f16").reshape(shape)
    wl.write_v = cast_f32(normal_f32(seed, _S_NEWV, int(np.prod(shape))), "f16").reshape(shape)
    return wl


def config4(seed: int = 4, num_seqs: int = 64, prefix_tokens: int = 80,
            suffix_range=(1, 300), num_cow: int = 16, num_blocks: int = 16384,
            poison: bool = False) -> Workload:
    """Shared-prefix decode with copy-on-write, bf16, Llama-3-8B head shape.

    Sequence 0 holds an 80-token system prompt (5 blocks of 16); the other
    sequences fork it (refcount 64 on each prompt block) and grow private
    suffixes uniform in ``suffix_range``.  Sequences 0..num_cow-1 then take
    a private copy of the last prompt block (the copy pairs); the decode runs
    on the tables after the copy.
    """
    rng = np.random.default_rng(seed)
    suffix = rng.integers(suffix_range[0], suffix_range[1] + 1, size=num_seqs)
    perm = rng.permutation(num_blocks)
    bs, hkv, d = 16, 8, 128
    alloc = BlockAllocator(num_blocks, bs, free_order=perm)
    alloc.add_sequence(0, prefix_tokens)
    for s in range(1, num_seqs):
        alloc.fork(0, s)
    for s in range(num_seqs):
        alloc.append_tokens(s, int(suffix[s]))
    lens = np.array([alloc.length(s) for s in range(num_seqs)], dtype=np.int32)
    maxb = max(len(alloc.block_table(s)) for s in range(num_seqs))
    pad = alloc.free_block_ids()[0] if poison else 0
    tables_before = alloc.tables_array(range(num_seqs), maxb, pad=pad)
    # every physical block any table names, in first-reference order
    used = list(dict.fromkeys(int(b) for s in range(num_seqs) for b in alloc.block_table(s)))
    last_prefix_block = (prefix_tokens - 1) // bs
    pairs = [alloc.copy_on_write(s, last_prefix_block) for s in range(num_cow)]
    pairs = np.array([p for p in pairs if p is not None], dtype=np.int64).reshape(-1, 2)
    alloc.check()
    tables_after = alloc.tables_array(range(num_seqs), maxb, pad=pad)
    shape = (num_blocks, hkv, bs, d)
    used = np.asarray(used, dtype=np.int64)
    kc = _draw_contents(seed, _S_K, len(used), hkv, bs, d, "bf16")
    vc = _draw_contents(seed, _S_V, len(used), hkv, bs, d, "bf16")
    k_pool = _place(shape, "bf16", used, kc, poison)
    v_pool = _place(shape, "bf16", used, vc, poison)
    if poison:
        _poison_tails(k_pool, tables_before, lens, bs, "bf16")
        _poison_tails(v_pool, tables_before, lens, bs, "bf16")
    q = cast_f32(normal_f32(seed, _S_Q, num_seqs * 32 * d), "bf16").reshape(num_seqs, 32, d)
    return Workload(
        name="prefix-cow-bf16", q_dtype="bf16", kv_dtype="bf16", num_q_heads=32,
        num_kv_heads=hkv, head_dim=d, block_size=bs, num_blocks=num_blocks, q=q,
        k_pool=k_pool, v_pool=v_pool, block_tables=tables_after, context_lens=lens,
        scale=float(np.float32(1.0 / math.sqrt(d))), copy_pairs=pairs,
        tables_before_copy=tables_before,
        meta={"seed": seed, "alloc": alloc.stats(), "poison": poison, "pad_block": pad,
              "prefix_blocks": [int(b) for b in tables_before[0, :last_prefix_block + 1]],
              "prefix_refcount_after": alloc.refcount(int(pairs[0, 0])) if len(pairs) else None})


def build_write_filled(seed: int, *, name: str, q_dtype: str, src_dtype: str, kv_dtype: str,
                       num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                       num_blocks: int, context_lens: Sequence[int], partition_size: int = 0,
                       rng: Optional[np.random.Generator] = None,
                       poison: bool = False) -> Workload:
    """Workload whose pools start empty (or NaN when poisoned) and are filled
    by the cache write of every position's K/V row (``write_*`` /
    ``slot_mapping``, rows in sequence order); each side (GPU and oracle)
    performs that write itself.  For an fp8 pool the per-tensor scales are
    max|row value| / 448 over all rows, as float32."""
    if rng is None:
        rng = np.random.default_rng(seed)
    lens = np.asarray(context_lens, dtype=np.int32)
    perm = rng.permutation(num_blocks)
    alloc = BlockAllocator(num_blocks, block_size, free_order=perm)
    slots = []
    for s, n in enumerate(lens):
        alloc.add_sequence(s, int(n))
        slots.append(alloc.slots(s, 0, int(n)))
    maxb = max(max(len(alloc.block_table(s)) for s in range(len(lens))), 1)
    pad = alloc.free_block_ids()[0] if poison else 0
    tables = alloc.tables_array(range(len(lens)), maxb, pad=pad)
    slot_mapping = np.concatenate(slots).astype(np.int64)
    t = len(slot_mapping)
    hkv, d = num_kv_heads, head_dim
    k_rows = cast_f32(normal_f32(seed, _S_K, t * hkv * d), src_dtype).reshape(t, hkv, d)
    v_rows = cast_f32(normal_f32(seed, _S_V, t * hkv * d), src_dtype).reshape(t, hkv, d)
    k_scale = v_scale = 1.0
    if kv_dtype == "fp8_e4m3":
        widen = bf16_bits_to_f32 if src_dtype == "bf16" else (lambda a: np.asarray(a, np.float32))
        k_scale = float(np.float32(np.abs(widen(k_rows)).max()) / np.float32(448.0))
        v_scale = float(np.float32(np.abs(widen(v_rows)).max()) / np.float32(448.0))
    shape = (num_blocks, hkv, block_size, d)
    if poison:
        k_pool = np.full(shape, NAN_BITS[kv_dtype], dtype=STORAGE[kv_dtype])
        v_pool = np.full(shape, NAN_BITS[kv_dtype], dtype=STORAGE[kv_dtype])
    else:
        k_pool = np.zeros(shape, dtype=STORAGE[kv_dtype])
        v_pool = np.zeros(shape, dtype=STORAGE[kv_dtype])
    q = cast_f32(normal_f32(seed, _S_Q, len(lens) * num_q_heads * d), q_dtype).reshape(
        len(lens), num_q_heads, d)
    return Workload(
        name=name, q_dtype=q_dtype, kv_dtype=kv_dtype, num_q_heads=num_q_heads,
        num_kv_heads=hkv, head_dim=d, block_size=block_size, num_blocks=num_blocks, q=q,
        k_pool=k_pool, v_pool=v_pool, block_tables=tables, context_lens=lens,
        scale=float(np.float32(1.0 / math.sqrt(d))), k_scale=k_scale, v_scale=v_scale,
        partition_size=partition_size, write_src_dtype=src_dtype, write_k=k_rows,
        write_v=v_rows, slot_mapping=slot_mapping,
        meta={"seed": seed, "alloc": alloc.stats(), "poison": poison, "pad_block": pad,
              "filled_by_write": True})


def config5(seed: int = 5, num_seqs: int = 32, ctx_range=(8192, 32768),
            num_blocks: int = 32768, partition_size: int = 512,
            poison: bool = False) -> Workload:
    """Long-context split-KV decode over an fp8 e4m3 cache with per-tensor
    scales and bf16 q: 64 q heads on 8 KV heads, head_dim 128, block 32,
    lengths uniform in ``ctx_range``; the pools are filled by the cache write
    of every position's bf16 row (see :func:`build_write_filled`)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(ctx_range[0], ctx_range[1] + 1, size=num_seqs).astype(np.int32)
    return build_write_filled(seed, name="long-ctx-fp8-split", q_dtype="bf16", src_dtype="bf16",
                              kv_dtype="fp8_e4m3", num_q_heads=64, num_kv_heads=8, head_dim=128,
                              block_size=32, num_blocks=num_blocks, context_lens=lens,
                              partition_size=partition_size, rng=rng, poison=poison)


def sequence_rows(wl: Workload, seqs: Sequence[int]) -> np.ndarray:
    """Indices into ``wl.write_k`` of the rows belonging to ``seqs`` when the
    write side holds every position of every sequence in order (config5)."""
    starts = np.concatenate([[0], np.cumsum(wl.context_lens.astype(np.int64))])
    return np.concatenate([np.arange(starts[s], starts[s + 1]) for s in seqs])
