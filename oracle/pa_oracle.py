"""Plain float64 statement of the paged KV-cache hot path (CPU, numpy).

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Nothing here is
blocked, fused or reordered beyond what the definitions below state: K and V
are gathered through the block table into contiguous arrays, then attention is
evaluated naively in float64.

Storage conventions for raw element arrays (the same bits the GPU holds):

====================  =====================================================
dtype name            numpy storage
====================  =====================================================
``"f32"``             ``np.float32``
``"f16"``             ``np.float16``
``"bf16"``            ``np.uint16`` holding bfloat16 bit patterns
``"fp8_e4m3"``        ``np.uint8`` holding OCP e4m3 ("fn") codes
====================  =====================================================

Pools are ``[num_blocks, num_kv_heads, block_size, head_dim]``; block tables
are ``[num_seqs, max_blocks_per_seq]`` int; context lengths ``[num_seqs]``.
"""

from __future__ import annotations

import math

import numpy as np

DTYPES = ("f32", "f16", "bf16", "fp8_e4m3")

# Largest finite OCP e4m3 magnitude: exponent field 1111, mantissa 110.
E4M3_MAX = 448.0


# ---------------------------------------------------------------------------
# fp8 e4m3 codec
#
# [UL] "관련 기법": storing K and V in 8 bits roughly halves cache memory
# against 16-bit storage.  The format itself is the OCP 8-bit e4m3 encoding
# (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, subnormals when
# the exponent field is 0, no infinities, and S.1111.111 reserved for NaN).
# ---------------------------------------------------------------------------

def _e4m3_code_value(code: int) -> float:
    """Value of one e4m3 code, straight from the bit-field definition."""
    negative = bool(code & 0x80)
    exponent = (code >> 3) & 0xF
    mantissa = code & 0x7
    if exponent == 0xF and mantissa == 0x7:
        return math.nan
    if exponent == 0:
        magnitude = (mantissa / 8.0) * 2.0 ** (1 - 7)     # subnormal
    else:
        magnitude = (1.0 + mantissa / 8.0) * 2.0 ** (exponent - 7)
    return -magnitude if negative else magnitude


_E4M3_TABLE = np.array([_e4m3_code_value(c) for c in range(256)], dtype=np.float64)
_E4M3_TABLE.setflags(write=False)


def e4m3_table() -> np.ndarray:
    """Float64 value of each of the 256 e4m3 codes (read-only array)."""
    return _E4M3_TABLE


def e4m3_encode(x) -> np.ndarray:
    """Encode float32 values as e4m3 codes: round to nearest, ties to even,
    saturating to +-448.

    The input is taken as float32 (the precision the GPU quantiser works in).
    Each magnitude is clamped to 448, then the nearest of the 127 finite
    non-negative code values is chosen; on an exact tie the code with an even
    mantissa (an even code number) wins.  The sign bit is copied from the
    input, so -0.0 and negative values that round to zero give 0x80.  NaN
    inputs give 0x7F with the input's sign.
    """
    x32 = np.asarray(x, dtype=np.float32)
    x64 = x32.astype(np.float64)                       # exact widening
    magnitude = np.minimum(np.abs(x64), E4M3_MAX)
    values = _E4M3_TABLE[:127]                         # codes 0x00..0x7E, increasing
    hi = np.clip(np.searchsorted(values, magnitude, side="left"), 1, 126)
    lo = hi - 1
    dist_lo = magnitude - values[lo]
    dist_hi = values[hi] - magnitude
    take_hi = (dist_hi < dist_lo) | ((dist_hi == dist_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    code = np.where(np.isnan(x64), np.uint8(0x7F), code)
    code = code | np.where(np.signbit(x64), np.uint8(0x80), np.uint8(0))
    return code.astype(np.uint8)


# ---------------------------------------------------------------------------
# element decoding
# ---------------------------------------------------------------------------

def to_float64(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored elements (see the storage table)."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(raw, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "fp8_e4m3":
        return _E4M3_TABLE[np.asarray(raw, dtype=np.uint8)]
    raise ValueError(f"unknown dtype {dtype!r}")


def _to_float32(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float32 value of 32/16-bit stored elements."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32)
    if dtype == "f16":
        return np.asarray(raw, dtype=np.float16).astype(np.float32)
    if dtype == "bf16":
        bits = np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32)
    raise ValueError(f"{dtype!r} is not a 32/16-bit source dtype")


# ---------------------------------------------------------------------------
# block arithmetic
# ---------------------------------------------------------------------------

def blocks_needed(num_tokens: int, block_size: int) -> int:
    """Blocks a sequence of ``num_tokens`` occupies: ceil(n / block_size).

    [GC] "按需分配 demo" and [UL] "페이징의 작동 방식": a new block is taken only
    when the last one is full, so n tokens need ceil(n/bs) blocks.
    """
    if num_tokens < 0 or block_size <= 0:
        raise ValueError("num_tokens must be >= 0 and block_size > 0")
    return -(-num_tokens // block_size)


def unused_slots(num_tokens: int, block_size: int) -> int:
    """Slots left empty in the last block ([VL] "memory wasteは最後のblock")."""
    return blocks_needed(num_tokens, block_size) * block_size - num_tokens


def kv_bytes_per_block(block_size: int, num_layers: int, num_heads: int,
                       head_dim: int, dtype_size: int) -> int:
    """KV bytes one block holds across all layers, K and V together.

    [GC] "GPU 上 KV cache 池子有多大": the product of block size, layer count,
    head count, head dimension, 2 (for K and V) and the element size.
    """
    return block_size * num_layers * num_heads * head_dim * 2 * dtype_size


def pool_blocks(pool_bytes: int, bytes_per_block: int) -> int:
    """Whole blocks that fit in a pool of ``pool_bytes`` ([GC], same section)."""
    return pool_bytes // bytes_per_block


# ---------------------------------------------------------------------------
# gather through the block table
# ---------------------------------------------------------------------------

def gather_kv(pool: np.ndarray, table_row: np.ndarray, num_tokens: int) -> np.ndarray:
    """Contiguous ``[num_kv_heads, num_tokens, head_dim]`` view of one
    sequence's cache, read through its block table.

    [GC] "PagedAttention CUDA Kernel": the kernel collects the scattered
    physical blocks named by the table, in logical order, back into a
    contiguous K (and V).  [UL] "페이징의 작동 방식" (PyTorch pool example):
    index the pool with the table, flatten the block and slot axes, and cut
    the result to the sequence length so unused slots of the last block are
    never seen.  [ZC] structural check: every table entry used must name an
    existing block.
    """
    num_blocks, num_kv_heads, block_size, head_dim = pool.shape
    nb = blocks_needed(num_tokens, block_size)
    ids = np.asarray(table_row[:nb], dtype=np.int64)
    if ids.shape[0] != nb:
        raise ValueError("block table shorter than ceil(context_len / block_size)")
    if nb and (ids.min() < 0 or ids.max() >= num_blocks):
        raise ValueError("block table names a block outside the pool")
    blocks = pool[ids]                                   # [nb, Hkv, bs, D]
    per_head = blocks.transpose(1, 0, 2, 3).reshape(num_kv_heads, nb * block_size, head_dim)
    return per_head[:, :num_tokens, :]


def gather_kv_range(pool: np.ndarray, table_row: np.ndarray, start: int, stop: int) -> np.ndarray:
    """Contiguous ``[num_kv_heads, stop - start, head_dim]`` of positions
    start .. stop-1 of one sequence, read through its block table.

    Only the blocks holding those positions are looked up: entries
    ``start // bs .. ceil(stop / bs) - 1``.  Entries before ``start // bs``
    are never read, so a table whose early entries name released blocks
    (the sliding window of zerocoder.ru "Что такое PagedAttention", section
    "Где подход не решает задачу", and vasteelab.pages.dev, section "hybrid
    modelではblock設計が複雑になる": blocks that have left the attention
    window are freed) gathers the same values.  With start = 0 this is
    :func:`gather_kv`.
    """
    num_blocks, num_kv_heads, block_size, head_dim = pool.shape
    if not 0 <= start <= stop:
        raise ValueError("need 0 <= start <= stop")
    first = start // block_size
    last = blocks_needed(stop, block_size)                # one past the last block
    ids = np.asarray(table_row[first:last], dtype=np.int64)
    if ids.shape[0] != last - first:
        raise ValueError("block table shorter than ceil(stop / block_size)")
    if ids.size and (ids.min() < 0 or ids.max() >= num_blocks):
        raise ValueError("block table names a block outside the pool")
    blocks = pool[ids]                                    # [nb, Hkv, bs, D]
    per_head = blocks.transpose(1, 0, 2, 3).reshape(num_kv_heads, ids.shape[0] * block_size, head_dim)
    off = start - first * block_size
    return per_head[:, off:off + (stop - start), :]


# ---------------------------------------------------------------------------
# decode attention
# ---------------------------------------------------------------------------

def _check_decode_shapes(q, k_pool, v_pool, block_tables, context_lens):
    num_seqs, num_q_heads, head_dim = q.shape
    if k_pool.shape != v_pool.shape:
        raise ValueError("K and V pools differ in shape")
    _, num_kv_heads, _, pool_head_dim = k_pool.shape
    if pool_head_dim != head_dim:
        raise ValueError("q and pool head_dim differ")
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    if len(context_lens) != num_seqs or len(block_tables) != num_seqs:
        raise ValueError("block_tables / context_lens length differs from num_seqs")
    return num_seqs, num_q_heads, head_dim, num_kv_heads


def _sequence_kv(k_pool, v_pool, kv_dtype, table_row, n, k_scale, v_scale, start=0):
    """Float64 K and V of positions start .. n-1 of one sequence, ``[Hkv, n - start, D]`` each."""
    if start == 0:
        k = to_float64(gather_kv(k_pool, table_row, n), kv_dtype)
        v = to_float64(gather_kv(v_pool, table_row, n), kv_dtype)
    else:
        k = to_float64(gather_kv_range(k_pool, table_row, start, n), kv_dtype)
        v = to_float64(gather_kv_range(v_pool, table_row, start, n), kv_dtype)
    if kv_dtype == "fp8_e4m3":
        # per-tensor scale: stored code value times the tensor's fp32 scale
        k = k * float(np.float32(k_scale))
        v = v * float(np.float32(v_scale))
    return k, v


def window_start(n: int, window: int) -> int:
    """First position a query at position n-1 sees under a sliding window of
    ``window`` positions (0: no window): max(0, n - window).

    zerocoder.ru, section "Где подход не решает задачу" (a limited attention
    window, whose blocks are released once they leave it) and
    vasteelab.pages.dev, section "hybrid modelではblock設計が複雑になる"
    (sliding-window layers keep only the most recent tokens).  The pages do
    not fix whether the window counts the query's own position; here it does:
    the query and the window - 1 positions before it.
    """
    if window < 0:
        raise ValueError("window must be >= 0")
    return max(0, n - window) if window else 0


def oracle_decode(q, q_dtype, k_pool, v_pool, kv_dtype, block_tables, context_lens,
                  scale, k_scale=1.0, v_scale=1.0, window=0) -> np.ndarray:
    """Single-token decode attention over a paged cache, in float64.

    For each sequence s and query head h (KV head ``h // (Hq/Hkv)``; query
    heads are grouped contiguously onto the KV heads they share, [UL]
    "관련 기법" on grouped-query attention), with n = context_lens[s]:

        z_i   = scale * <q[s,h], K_i>          for i < n
        out   = sum_i softmax(z)_i * V_i

    K and V come from :func:`gather_kv` (table walk in logical order,
    truncated to n).  This is the per-sequence gather-then-attend of [GC]
    "PagedAttention CUDA Kernel", with the explicit ``scale`` factor and the
    truncation to exactly n positions.  Paging is addressing only and leaves
    the attention result unchanged ([PD] "PagedAttention"); the softmax
    subtracts its maximum first, which changes nothing mathematically.
    ``scale`` is taken as the float32 value the GPU receives.  A sequence with
    n = 0 yields a zero row.  With ``window`` > 0 only positions
    :func:`window_start` .. n-1 take part (and only their blocks are read).
    Returns float64 ``[S, Hq, D]``.
    """
    num_seqs, num_q_heads, head_dim, num_kv_heads = _check_decode_shapes(
        q, k_pool, v_pool, block_tables, context_lens)
    group = num_q_heads // num_kv_heads
    scale64 = float(np.float32(scale))
    qf = to_float64(q, q_dtype)
    out = np.zeros((num_seqs, num_q_heads, head_dim), dtype=np.float64)
    for s in range(num_seqs):
        n = int(context_lens[s])
        if n == 0:
            continue
        k, v = _sequence_kv(k_pool, v_pool, kv_dtype, block_tables[s], n, k_scale, v_scale,
                            start=window_start(n, window))
        for h in range(num_q_heads):
            kvh = h // group
            z = scale64 * (k[kvh] @ qf[s, h])
            p = np.exp(z - z.max())
            out[s, h] = (p @ v[kvh]) / p.sum()
    return out


def oracle_prefill(q, q_dtype, k_pool, v_pool, kv_dtype, block_tables, context_lens, query_start,
                   scale, k_scale=1.0, v_scale=1.0, window=0) -> np.ndarray:
    """Causal multi-query attention over a paged cache (a prompt, or a chunk
    of one after a cached prefix), in float64.

    Sequence s holds n = context_lens[s] positions in its blocks, the new
    ones already written.  Its L = query_start[s+1] - query_start[s] queries
    are rows query_start[s] .. query_start[s+1]-1 of ``q`` ([T, Hq, D]) and
    stand for its last L positions: query i sits at position p = n - L + i.
    Each attends positions lo .. p (lo = 0, or p + 1 - window with a sliding
    window), with the scale, grouping and float64 softmax of
    :func:`oracle_decode`:

        out[row, h] = sum_{lo <= j <= p} softmax_j(scale * <q[row, h], K_j>) V_j

    zerocoder.ru, section "Зачем KV cache вообще нужен": in full causal
    attention each position uses the keys and values of the positions before
    it; ultralytics.com "PagedAttention", section "관련 기법": engines run
    FlashAttention-style kernels that read these from the paged blocks.  The
    last query of a sequence is exactly the decode step of
    :func:`oracle_decode`.  Returns float64 ``[T, Hq, D]``.
    """
    num_tokens, num_q_heads, head_dim = q.shape
    num_kv_heads = k_pool.shape[1]
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    group = num_q_heads // num_kv_heads
    qs = np.asarray(query_start, dtype=np.int64)
    if qs.shape != (len(context_lens) + 1,) or qs[0] != 0 or qs[-1] != num_tokens or np.any(np.diff(qs) < 0):
        raise ValueError("query_start must be a nondecreasing [S + 1] prefix sum from 0 to T")
    scale64 = float(np.float32(scale))
    qf = to_float64(q, q_dtype)
    out = np.zeros((num_tokens, num_q_heads, head_dim), dtype=np.float64)
    for s in range(len(context_lens)):
        n, L = int(context_lens[s]), int(qs[s + 1] - qs[s])
        if L > n:
            raise ValueError("a sequence has more queries than positions")
        if L == 0:
            continue
        first = window_start(n - L + 1, window)        # first position the first query sees
        k, v = _sequence_kv(k_pool, v_pool, kv_dtype, block_tables[s], n, k_scale, v_scale, start=first)
        for i in range(L):
            p = n - L + i
            lo = window_start(p + 1, window)
            for h in range(num_q_heads):
                kvh = h // group
                z = scale64 * (k[kvh, lo - first:p + 1 - first] @ qf[qs[s] + i, h])
                e = np.exp(z - z.max())
                out[qs[s] + i, h] = (e @ v[kvh, lo - first:p + 1 - first]) / e.sum()
    return out


def oracle_partials(q, q_dtype, k_pool, v_pool, kv_dtype, block_tables, context_lens,
                    scale, partition_size, k_scale=1.0, v_scale=1.0):
    """Per-partition softmax statistics for split-KV decode, in float64.

    Partition p of a sequence covers positions [p*P, min((p+1)*P, n)).  For
    each (s, h, p):  m = max z_i,  l = sum exp(z_i - m),  o = sum exp(z_i - m) V_i
    over the partition (z as in :func:`oracle_decode`).  Returns
    ``(m, l, o, num_parts)`` with m, l ``[S, Hq, Pmax]``, o ``[S, Hq, Pmax, D]``
    and num_parts ``[S]``; entries of absent partitions are m = -inf, l = 0,
    o = 0.  Splitting the context is not on the pages: it is an exact
    regrouping of the sums in :func:`oracle_decode`.
    """
    num_seqs, num_q_heads, head_dim, num_kv_heads = _check_decode_shapes(
        q, k_pool, v_pool, block_tables, context_lens)
    if partition_size <= 0:
        raise ValueError("partition_size must be positive")
    group = num_q_heads // num_kv_heads
    scale64 = float(np.float32(scale))
    qf = to_float64(q, q_dtype)
    num_parts = np.array([blocks_needed(int(n), partition_size) for n in context_lens],
                         dtype=np.int64)
    pmax = int(num_parts.max()) if num_seqs else 0
    m = np.full((num_seqs, num_q_heads, pmax), -np.inf)
    l = np.zeros((num_seqs, num_q_heads, pmax))
    o = np.zeros((num_seqs, num_q_heads, pmax, head_dim))
    for s in range(num_seqs):
        n = int(context_lens[s])
        if n == 0:
            continue
        k, v = _sequence_kv(k_pool, v_pool, kv_dtype, block_tables[s], n, k_scale, v_scale)
        for h in range(num_q_heads):
            kvh = h // group
            z = scale64 * (k[kvh] @ qf[s, h])
            for p in range(num_parts[s]):
                lo, hi = p * partition_size, min((p + 1) * partition_size, n)
                zp = z[lo:hi]
                m[s, h, p] = zp.max()
                e = np.exp(zp - m[s, h, p])
                l[s, h, p] = e.sum()
                o[s, h, p] = e @ v[kvh, lo:hi]
    return m, l, o, num_parts


def oracle_lse_merge(m, l, o, num_parts) -> np.ndarray:
    """Combine split-KV partials into the decode output, in float64.

    With M = max_p m_p and w_p = exp(m_p - M):  out = sum_p w_p o_p / sum_p w_p l_p,
    summed over p = 0 .. num_parts-1 in increasing p.  A sequence with no
    partition yields a zero row.  Not on the pages (see
    :func:`oracle_partials`).
    """
    num_seqs, num_q_heads, _, head_dim = o.shape
    out = np.zeros((num_seqs, num_q_heads, head_dim))
    for s in range(num_seqs):
        P = int(num_parts[s])
        if P == 0:
            continue
        for h in range(num_q_heads):
            big_m = m[s, h, :P].max()
            w = np.exp(m[s, h, :P] - big_m)
            out[s, h] = (w @ o[s, h, :P]) / (w @ l[s, h, :P])
    return out


# ---------------------------------------------------------------------------
# cache write through the slot mapping
# ---------------------------------------------------------------------------

def oracle_write(k, v, src_dtype, slot_mapping, k_pool, v_pool, pool_dtype,
                 k_scale=1.0, v_scale=1.0):
    """Scatter new K/V rows into copies of the pools; returns ``(k_pool, v_pool)``.

    Token t with slot s goes to block s // bs at in-block offset s % bs, for
    every KV head ([UL] "페이징의 작동 방식": the pool example stores position
    pos at ``[table[pos // bs], pos % bs]``; [VL] "Attention kernelとmemory
    manager": the implementation writes K and V through physical blocks and a
    slot mapping).  Rows are ``[T, Hkv, D]``.

    When the pool dtype equals the source dtype the bits are copied.  For an
    e4m3 pool with a 32/16-bit source, each element is widened to float32,
    multiplied in float32 by ``inv = float32(1) / float32(scale)`` and encoded
    with :func:`e4m3_encode` (round to nearest even, saturating).
    """
    k_pool = k_pool.copy()
    v_pool = v_pool.copy()
    slots = np.asarray(slot_mapping, dtype=np.int64)
    num_blocks, _, block_size, _ = k_pool.shape
    if slots.size and (slots.min() < 0 or slots.max() >= num_blocks * block_size):
        raise ValueError("slot outside the pool")
    if len(np.unique(slots)) != len(slots):
        raise ValueError("slots must be distinct")
    blk, off = slots // block_size, slots % block_size
    if pool_dtype == src_dtype:
        k_pool[blk, :, off, :] = k
        v_pool[blk, :, off, :] = v
    elif pool_dtype == "fp8_e4m3" and src_dtype in ("f32", "f16", "bf16"):
        for rows, pool, sc in ((k, k_pool, k_scale), (v, v_pool, v_scale)):
            inv = np.float32(1.0) / np.float32(sc)
            scaled = _to_float32(rows, src_dtype) * inv          # float32 multiply
            pool[blk, :, off, :] = e4m3_encode(scaled)
    else:
        raise ValueError(f"unsupported write {src_dtype} -> {pool_dtype}")
    return k_pool, v_pool


# ---------------------------------------------------------------------------
# copy-on-write block copy
# ---------------------------------------------------------------------------

def oracle_copy(k_pool, v_pool, src_dst_pairs):
    """Copy whole blocks (every head and slot) for each (src, dst) pair;
    returns new ``(k_pool, v_pool)``.

    [VL] "Copy-on-Writeで共通prefixを共有できる" and [UL] "시퀀스 간 블록 공유":
    before a sequence writes into a block other sequences still reference,
    the block is first copied to a new physical block.  Destinations are
    distinct and never a source, so the pairs commute.
    """
    k_pool = k_pool.copy()
    v_pool = v_pool.copy()
    pairs = np.asarray(src_dst_pairs, dtype=np.int64).reshape(-1, 2)
    if pairs.size:
        if pairs.min() < 0 or pairs.max() >= k_pool.shape[0]:
            raise ValueError("block id outside the pool")
        if len(np.unique(pairs[:, 1])) != len(pairs) or np.intersect1d(pairs[:, 0], pairs[:, 1]).size:
            raise ValueError("destinations must be distinct and never a source")
    for src, dst in pairs:
        k_pool[dst] = k_pool[src]
        v_pool[dst] = v_pool[src]
    return k_pool, v_pool


# ---------------------------------------------------------------------------
# swap between the GPU pool and host memory
# ---------------------------------------------------------------------------

def oracle_swap(src_k, src_v, dst_k, dst_v, src_dst_pairs):
    """Copy whole blocks from one pool pair to another (the GPU pool and a
    host swap area of the same block shape); returns new ``(dst_k, dst_v)``.

    gufacode.com "PagedAttention:KV cache 的页表革命", section "Swap 到
    CPU:兜底溢出": when the pool runs out, every block of a low-priority
    sequence is copied to the CPU swap area and its GPU blocks are freed;
    later the sequence is copied back and continues decoding.
    vasteelab.pages.dev, section "blockが足りなくなったとき": swapping to the
    CPU costs transfer time and CPU memory.  Sources may repeat (a block
    copied to several places); destinations must be distinct.
    """
    if src_k.shape[1:] != dst_k.shape[1:] or src_k.dtype != dst_k.dtype:
        raise ValueError("pools differ in block shape or dtype")
    dst_k = dst_k.copy()
    dst_v = dst_v.copy()
    pairs = np.asarray(src_dst_pairs, dtype=np.int64).reshape(-1, 2)
    if pairs.size:
        if pairs[:, 0].min() < 0 or pairs[:, 0].max() >= src_k.shape[0] or \
                pairs[:, 1].min() < 0 or pairs[:, 1].max() >= dst_k.shape[0]:
            raise ValueError("block id outside its pool")
        if len(np.unique(pairs[:, 1])) != len(pairs):
            raise ValueError("destinations must be distinct")
    for src, dst in pairs:
        dst_k[dst] = src_k[src]
        dst_v[dst] = src_v[src]
    return dst_k, dst_v
