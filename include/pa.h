/*
 * pa.h -- C ABI of libpa.so, the MI355X (gfx950) paged KV-cache hot path.
 *
 * Three operations:
 *
 *   pa_write_kv     scatter new K/V rows into the paged pool through a slot
 *                   mapping (the cache write);
 *   pa_decode       single-token attention for a batch of sequences, reading
 *                   K/V through per-sequence block tables, optionally split
 *                   over the context with a log-sum-exp merge;
 *   pa_copy_blocks  whole-block copies, the copy-on-write step for shared
 *                   prefix blocks.
 *
 * Pages that define the operations (cited by title and section):
 *   - ultralytics.com glossary "PagedAttention", section "페이징의 작동 방식":
 *     a pool of fixed-size blocks shared by all requests, a per-request block
 *     table, position pos stored at [table[pos / bs], pos % bs], and the
 *     attention kernel reading the blocks back in table order;
 *   - vasteelab.pages.dev "PagedAttentionとは？LLMのKV Cacheをblock単位で管理する",
 *     section "PagedAttentionはAttention kernelとmemory managerの組み合わせである":
 *     K and V are written through physical blocks and a slot mapping, and the
 *     model runner hands the mapping to the kernel;
 *   - gufacode.com "PagedAttention:KV cache 的页表革命", section
 *     "PagedAttention CUDA Kernel": per sequence, gather the blocks the table
 *     names and compute softmax(q K^T) V;
 *   - vasteelab.pages.dev, section "Copy-on-Writeで共通prefixを共有できる", and
 *     ultralytics.com, section "시퀀스 간 블록 공유": a block still shared by
 *     other sequences is copied to a fresh block before a sequence writes it.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every array pointer is DEVICE memory owned by the caller (for instance a
 *   torch tensor's data_ptr()), row-major and contiguous.  The pa_kv_pool
 *   descriptor itself is HOST memory and is read during the call only.
 * - The library never allocates, frees or synchronises.  Work is enqueued on
 *   `stream` (a hipStream_t; NULL means the default stream) and the call
 *   returns immediately.  Faults during kernel execution surface at the
 *   caller's next synchronisation on that stream.
 * - Every call returns a pa_status.  Argument errors are found on the host
 *   before anything is enqueued; nothing is enqueued when a call fails.
 *   pa_last_error() then gives a one-line reason (per thread).
 * - Pool layout: K and V are separate arrays, each
 *       [num_blocks][num_kv_heads][block_size][head_dim]
 *   so one (block, head) tile of block_size x head_dim elements is
 *   contiguous.  block_size is a power of two in [2, 256]; head_dim is one of
 *   8, 64, 128, 256.
 * - Element types: PA_F32 (IEEE binary32), PA_F16 (IEEE binary16), PA_BF16
 *   (bfloat16), PA_FP8_E4M3 (OCP 8-bit e4m3 "fn": bias 7, max 448, no
 *   infinities).  An fp8 pool holds code * scale, with one float scale per
 *   tensor (k_scale for K, v_scale for V).
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's hipStream_t (declared here so this header does not need
 * the HIP headers). */
struct ihipStream_t;
typedef struct ihipStream_t *pa_stream_t;

typedef enum {
  PA_F32 = 0,
  PA_F16 = 1,
  PA_BF16 = 2,
  PA_FP8_E4M3 = 3
} pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1, /* null pointer, negative size, shape mismatch */
  PA_ERR_UNSUPPORTED = -2, /* valid but not built: head_dim, dtype combination */
  PA_ERR_WORKSPACE = -3,   /* split-KV workspace missing or too small */
  PA_ERR_HIP = -4          /* the HIP runtime refused the launch */
} pa_status;

/* partition_size value asking pa_decode to balance the work itself (see
 * pa_decode). */
#define PA_PARTITION_AUTO (-1)

/* Describes a caller-owned K/V pool pair. */
typedef struct {
  void *k_pool;          /* device, [num_blocks][num_kv_heads][block_size][head_dim] */
  void *v_pool;          /* device, same shape and dtype as k_pool */
  int64_t num_blocks;    /* N >= 1 */
  int32_t num_kv_heads;  /* Hkv >= 1 */
  int32_t block_size;    /* bs: power of two in [2, 256] */
  int32_t head_dim;      /* D: 8, 64, 128 or 256 */
  int32_t dtype;         /* pa_dtype of the stored elements */
  float k_scale;         /* fp8 pools: K = code * k_scale (> 0, finite); else must be 1 */
  float v_scale;         /* fp8 pools: V = code * v_scale (> 0, finite); else must be 1 */
} pa_kv_pool;

/*
 * pa_write_kv -- the cache write (reshape_and_cache).
 *
 * For every token t < num_tokens with s = slot_mapping[t], and every KV head h:
 *     pool[s / bs][h][s % bs][:] = row[t][h][:]
 * for K (from k) and V (from v).
 *
 *   k, v          device, [num_tokens][num_kv_heads][head_dim] of src_dtype.
 *   src_dtype     equal to pool->dtype (the bits are copied), or PA_F32 /
 *                 PA_F16 / PA_BF16 when pool->dtype is PA_FP8_E4M3: then each
 *                 element is widened to float, multiplied in float by
 *                 (1.0f / scale) and encoded to e4m3 with round-to-nearest-even,
 *                 saturating to +-448 (NaN stays NaN).
 *   slot_mapping  device, int64 [num_tokens]; slots must be distinct and lie
 *                 in [0, num_blocks * bs).  A slot outside that range is
 *                 skipped (its token is not written) rather than faulting.
 *   num_tokens    >= 0; 0 enqueues nothing.
 * Tokens are independent: the call has no ordering between them.
 */
int pa_write_kv(const void *k, const void *v, int32_t src_dtype, int32_t num_tokens,
                const int64_t *slot_mapping, const pa_kv_pool *pool, pa_stream_t stream);

/*
 * pa_decode_workspace_bytes -- device scratch pa_decode needs in split mode:
 * one 64-bit arrival counter per (sequence, group of up to 8 query heads
 * sharing a KV head), padded to 256 bytes, then float32 partial maxima, sums
 * and outputs (head dim 128 with partition_size > 0 stores each partial
 * output normalised by its sum and rounded to the query dtype, in the same
 * space).  With partition_size > 0 there is a partial for every
 * (sequence, query head slot, partition), with
 * ceil(max_blocks_per_seq * block_size / partition_size) partitions per
 * sequence.  With PA_PARTITION_AUTO there are two partials per streaming wave the
 * balanced split may launch, 4 per compute unit of the CURRENT device, so
 * size the workspace with the device that will run the call selected.
 * Returns 0 for partition_size == 0 (single pass) and for invalid arguments.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size,
                                 int32_t partition_size);

/*
 * pa_decode -- paged single-token attention.
 *
 * For every sequence s < num_seqs with n = context_lens[s], and every query
 * head h < num_q_heads, with kv = h / (num_q_heads / num_kv_heads)
 * (contiguous grouping of query heads onto shared KV heads):
 *     K_i = k_pool[block_tables[s][i / bs]][kv][i % bs][:]   for i < n
 *     z_i = scale * <q[s][h], K_i>
 *     out[s][h][:] = sum_i softmax(z)_i * V_i
 * computed with float32 accumulation.  Positions i >= n in the last block
 * never contribute; n == 0 gives a zero row.  The result does not depend on
 * where the blocks physically lie: the accumulation order is a function of
 * the logical positions only, so relabelling the physical blocks gives
 * bit-identical output.
 *
 *   q             device, [num_seqs][num_q_heads][head_dim] of q_dtype.
 *   q_dtype       PA_F32, PA_F16 or PA_BF16.  Built combinations of
 *                 (q_dtype, pool->dtype): (F32,F32), (F16,F16), (BF16,BF16),
 *                 (BF16,FP8_E4M3), (F16,FP8_E4M3).
 *   num_q_heads   a multiple of pool->num_kv_heads.
 *   block_tables  device, int32 [num_seqs][max_blocks_per_seq]; entries
 *                 j < ceil(n / bs) must lie in [0, num_blocks); later entries
 *                 are never read.  A sequence whose table names a block
 *                 outside the pool gets a NaN output row instead of a fault.
 *   context_lens  device, int32 [num_seqs]; 0 <= n <= max_blocks_per_seq * bs
 *                 (a sequence outside that range gets a NaN row).
 *   scale         softmax scale (typically 1/sqrt(head_dim)); finite.
 *   out           device, [num_seqs][num_q_heads][head_dim] of q_dtype,
 *                 rounded to nearest even from float32.  Must not overlap q.
 *   partition_size  PA_PARTITION_AUTO (-1): the library balances the work.
 *                 For head_dim 128 at block size 16 or 32 every launched
 *                 wave gets an equal share of the batch's 16-position tiles
 *                 (a context may be cut anywhere on a tile boundary, and the
 *                 pieces are merged in context order); the cut points depend
 *                 on the batch's lengths and the GPU's size, so results are
 *                 bit-identical across runs and block relabellings on one
 *                 GPU model.  Other shapes run single pass.
 *                 0: single pass, one workgroup walks a whole context.
 *                 > 0: split-KV; a multiple of bs; partition p covers
 *                 positions [p*P, min((p+1)*P, n)); the partial results are
 *                 merged in a fixed order (head dim 128: partitions j, j+g,
 *                 j+2g, ... for each of g lane groups, then the groups in
 *                 order; other shapes: increasing p), so the output does not
 *                 depend on the order in which partitions finish.
 *   workspace     device scratch of at least pa_decode_workspace_bytes(...)
 *                 bytes when partition_size != 0 (else may be NULL).  Its
 *                 leading bytes hold counters, which MUST be zero before the
 *                 first call that uses the workspace: zero-fill the whole
 *                 workspace once when it is allocated.  Every call leaves
 *                 the counters zero again; the rest may hold anything.  One
 *                 workspace, sized for the largest batch, serves calls with
 *                 any number of sequences; it serves one partition mode and
 *                 one head layout (head_dim, query heads per KV head): zero-
 *                 fill it again before switching.  Calls that may run
 *                 concurrently must not share one workspace.  The balanced split relies on
 *                 the dispatcher dealing workgroups to the XCDs in turn; a
 *                 launch that finds otherwise writes NaN rows and marks the
 *                 workspace, and every later call with a marked workspace
 *                 writes NaN rows until it is zero-filled again.
 */
int pa_decode(const void *q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
              const pa_kv_pool *pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
              const int32_t *context_lens, float scale, void *out, int32_t partition_size,
              void *workspace, size_t workspace_bytes, pa_stream_t stream);

/*
 * pa_decode_window -- pa_decode under a sliding attention window (zerocoder.ru
 * "Что такое PagedAttention", section "Где подход не решает задачу": with a
 * limited attention window, blocks that leave it are released;
 * vasteelab.pages.dev, section "hybrid modelではblock設計が複雑になる").
 *
 * As pa_decode, except that sequence s attends only positions
 * lo .. n-1 with lo = max(0, n - window): the current position and the
 * window - 1 before it.  Table entries of blocks wholly before lo
 * (j < lo / block_size) are never read, so they may name released blocks or
 * hold any value.  With partition_size > 0 the partitions are
 * [p*P, (p+1)*P) intersected with [lo, n), merged in pa_decode's fixed order.
 *
 *   window    >= 0; 0 attends the whole context (pa_decode).
 * Every other argument, the workspace contract and the error behaviour are
 * pa_decode's (the workspace is sized with pa_decode_workspace_bytes for the
 * same arguments).
 */
int pa_decode_window(const void *q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                     const pa_kv_pool *pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                     const int32_t *context_lens, int32_t window, float scale, void *out,
                     int32_t partition_size, void *workspace, size_t workspace_bytes, pa_stream_t stream);

/*
 * pa_prefill -- causal multi-query attention over the paged cache: a prompt,
 * or a chunk of one after a cached prefix (chunked prefill).  zerocoder.ru
 * "Что такое PagedAttention", section "Зачем KV cache вообще нужен" (in
 * causal attention each position uses the keys and values of the positions
 * before it); ultralytics.com "PagedAttention", section "관련 기법" (engines run
 * FlashAttention-style kernels that read those from the paged blocks).
 *
 * Sequence s < num_seqs holds n = context_lens[s] positions in its blocks,
 * the new ones already written (pa_write_kv).  Its L = query_start[s+1] -
 * query_start[s] queries are rows query_start[s] .. query_start[s+1]-1 of q
 * and stand for its last L positions: row query_start[s] + i is position
 * p = n - L + i and attends positions lo .. p (lo = 0, or max(0, p + 1 -
 * window) under a sliding window), for every query head h with KV head
 * h / (num_q_heads / num_kv_heads):
 *     out[row][h][:] = sum_{lo <= j <= p} softmax_j(scale * <q[row][h], K_j>) V_j
 * with float32 accumulation; out is rounded to nearest even in q's dtype.
 * The last query of a sequence computes exactly the decode step of
 * pa_decode.  Table entries of blocks holding no position some query of the
 * sequence attends are never read.
 *
 *   q, out        device, [num_tokens][num_q_heads][head_dim] of q_dtype; out
 *                 must not overlap q.  Rows of sequences with invalid
 *                 lengths (n outside [0, max_blocks_per_seq * bs], L > n) are
 *                 NaN.
 *   query_start   device, int32 [num_seqs + 1], nondecreasing, query_start[0]
 *                 = 0 and query_start[num_seqs] = num_tokens.  Entries that
 *                 break these rules never make the call read q or write out
 *                 outside their num_tokens rows; the rows of the sequences
 *                 they spoil hold NaN, keep their old value or hold
 *                 meaningless numbers.
 *   window        >= 0; 0 attends every earlier position.
 * q_dtype / pool dtype combinations, head dims, block sizes, block_tables,
 * context_lens and scale are as for pa_decode.  No workspace is needed.
 * Head dim 128 with a bf16 or f16 cache of block size 16 or 32 and 1, 2, 4
 * or 8 query heads per KV head runs on the matrix cores; other shapes run a
 * vector kernel (one workgroup per query row and head group).
 */
int pa_prefill(const void *q, int32_t q_dtype, int32_t num_tokens, int32_t num_q_heads,
               const pa_kv_pool *pool, int32_t num_seqs, const int32_t *block_tables,
               int32_t max_blocks_per_seq, const int32_t *context_lens, const int32_t *query_start,
               int32_t window, float scale, void *out, pa_stream_t stream);

/*
 * pa_copy_blocks -- copy-on-write block copy.
 *
 * For each pair i < num_pairs, (src, dst) = (src_dst_pairs[2i], src_dst_pairs[2i+1]):
 *     k_pool[dst] = k_pool[src];  v_pool[dst] = v_pool[src]
 * over every head and slot of the block.  Destinations must be distinct and
 * must not also appear as sources (then the pairs commute).  A pair naming a
 * block outside [0, num_blocks), or with src == dst, is skipped.
 *
 *   src_dst_pairs  device, int64 [num_pairs][2].
 *   num_pairs      >= 0; 0 enqueues nothing.
 */
int pa_copy_blocks(const pa_kv_pool *pool, const int64_t *src_dst_pairs, int32_t num_pairs,
                   pa_stream_t stream);

/*
 * pa_decode_status -- health of a workspace the balanced split
 * (PA_PARTITION_AUTO) has used.  Enqueues on `stream` a one-thread kernel
 * that writes the workspace's status word to *status:
 *   PA_WS_CLEAN      (0)  every call so far found its counters in order;
 *   PA_WS_MISPLACED  (1)  a launch found the workgroups dealt to the XCDs
 *                         otherwise than in turn (its rows were written NaN);
 *   PA_WS_TIMED_OUT  (2)  a wait between the waves of one workgroup passed
 *                         its poll bound, which the protocol never needs (a
 *                         fault; the launch wrote NaN rows and every wave
 *                         exited normally).
 * A workspace whose status is not PA_WS_CLEAN makes every later call write
 * NaN rows until it is zero-filled.  The value is ready once `stream` has
 * reached this point (synchronise, or order later work after it).
 *
 *   workspace, workspace_bytes  the workspace given to pa_decode (>= 4096
 *                 bytes when partition_size is PA_PARTITION_AUTO).
 *   partition_size  the mode the workspace serves; any mode other than
 *                 PA_PARTITION_AUTO keeps no status and gives PA_WS_CLEAN.
 *   status        device memory, or host memory from hipHostMalloc, 4 bytes.
 */
#define PA_WS_CLEAN 0
#define PA_WS_MISPLACED 1
#define PA_WS_TIMED_OUT 2
int pa_decode_status(const void *workspace, size_t workspace_bytes, int32_t partition_size,
                     int32_t *status, pa_stream_t stream);

/*
 * pa_set_wait_polls -- test hook.  Sets, for the calling thread's later
 * pa_decode calls, how many polls a wait between the waves of one
 * balanced-split workgroup makes before it gives up (see PA_WS_TIMED_OUT);
 * 0 restores the default (2^20 polls, tens of milliseconds).  A small value
 * lets a test force the give-up path from the host while every wave still
 * exits normally.  Returns PA_ERR_INVALID_ARG for a negative value.
 */
int pa_set_wait_polls(int32_t polls);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, meaning, results and errors as
 * pa_decode, without the workspace: the split-KV scratch is a static device
 * array inside the library, PA_NOALLOC_SCRATCH_BYTES long, that each GPU the
 * library runs on holds from the first call on it until the process ends.
 *
 * - Calls whose split needs more scratch than that (pa_decode_workspace_bytes
 *   above PA_NOALLOC_SCRATCH_BYTES) fail with PA_ERR_WORKSPACE and enqueue
 *   nothing; use pa_decode with a workspace for them.  partition_size 0
 *   needs no scratch.
 * - The call allocates and frees nothing.  It enqueues a fill kernel that
 *   zeroes the scratch's counters ahead of the decode kernels (the scratch
 *   keeps the last call's contents otherwise), so a call never inherits a
 *   marked or half-counted state from an earlier one.
 * - Every call on one GPU shares that GPU's scratch: calls that may overlap
 *   on one GPU (different streams without ordering, several threads) race
 *   and give wrong results.  Order them on one stream.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int pa_decode_noalloc(const void *q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                      const pa_kv_pool *pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                      const int32_t *context_lens, float scale, void *out, int32_t partition_size,
                      pa_stream_t stream);

/*
 * pa_swap_blocks -- whole-block copies from one pool pair to another of the
 * same block shape: the GPU pool and a swap area in pinned host memory, in
 * either direction (gufacode.com "PagedAttention:KV cache 的页表革命", section
 * "Swap 到 CPU:兜底溢出": when the pool runs out, all blocks of a
 * low-priority sequence are copied to CPU memory and freed, and copied back
 * later; vasteelab.pages.dev, section "blockが足りなくなったとき").
 *
 * For each pair i < num_pairs, (s, d) = (src_dst_pairs[2i], src_dst_pairs[2i+1]):
 *     dst->k_pool[d] = src->k_pool[s];  dst->v_pool[d] = src->v_pool[s]
 * over every head and slot of the block, bit for bit.  One kernel moves all
 * pairs; the host side of the copy is read or written over the host link by
 * the kernel itself.
 *
 *   src, dst       descriptors with equal num_kv_heads, block_size, head_dim
 *                  and dtype (num_blocks may differ).  Each pool pointer is
 *                  device memory of the current device or host memory from
 *                  hipHostMalloc (torch: pin_memory=True); anything else
 *                  (pageable host memory) is refused with PA_ERR_INVALID_ARG
 *                  before any launch.
 *   src_dst_pairs  int64 [num_pairs][2], device or pinned host memory.
 *                  Destinations must be distinct (and, within one pool, not
 *                  also sources).  A pair naming a block outside its pool is
 *                  skipped; within one pool so is s == d.
 *   num_pairs      >= 0; 0 enqueues nothing.
 * Host memory written by the kernel is complete once `stream` has reached
 * the end of the call (synchronise before reading it on the host).
 */
int pa_swap_blocks(const pa_kv_pool *src, const pa_kv_pool *dst, const int64_t *src_dst_pairs,
                   int32_t num_pairs, pa_stream_t stream);

/* Static text for a pa_status value. */
const char *pa_status_string(int status);

/* One-line reason for the calling thread's last failed call ("" if none). */
const char *pa_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int pa_version(void);

/*
 * pa_time_next_decode -- benchmark hook.  The calling thread's next
 * pa_decode records start_event as its first kernel begins and stop_event as
 * its last kernel ends (the event pair of hipExtLaunchKernel), so that the
 * pair brackets the decode kernels alone, not the stream's other commands.
 * The pair applies to that one call, whatever its outcome (a call that fails
 * validation or enqueues nothing records neither event).
 *
 *   start_event, stop_event  hipEvent_t handles the caller created with
 *                            timing enabled; both NULL clears a pending pair.
 * Returns PA_OK, or PA_ERR_INVALID_ARG when exactly one of them is NULL.
 */
int pa_time_next_decode(void *start_event, void *stop_event);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
