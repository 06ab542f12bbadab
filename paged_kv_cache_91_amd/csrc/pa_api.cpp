// C ABI of libpa.so: argument validation, kernel selection and launch.
// Declarations, layouts and the error contract are in include/pa.h.
//
// Every check runs on the host before anything is enqueued; a failing call
// enqueues nothing and records a one-line reason for pa_last_error().

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "pa.h"
#include "pa_internal.h"

namespace {

thread_local char g_last_error[256] = "";
// the event pair pa_time_next_decode set for this thread's next pa_decode
thread_local pa_impl::LaunchEvents g_next_events;
// the poll bound of the balanced split's waits for this thread's calls
thread_local int32_t g_wait_polls = pa_impl::kDefaultWaitPolls;

int fail(int status, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return PA_OK;
}

int element_size(int dtype) {
  switch (dtype) {
    case PA_F32: return 4;
    case PA_F16: return 2;
    case PA_BF16: return 2;
    case PA_FP8_E4M3: return 1;
    default: return 0;
  }
}

int log2_exact(int v) {
  if (v <= 0 || (v & (v - 1))) return -1;
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

bool supported_head_dim(int d) { return d == 8 || d == 64 || d == 128 || d == 256; }

int check_pool(const pa_kv_pool *p) {
  if (!p) return fail(PA_ERR_INVALID_ARG, "pool descriptor is NULL");
  if (!p->k_pool || !p->v_pool) return fail(PA_ERR_INVALID_ARG, "pool K or V pointer is NULL");
  if (p->k_pool == p->v_pool) return fail(PA_ERR_INVALID_ARG, "K and V pools alias");
  if (p->num_blocks <= 0) return fail(PA_ERR_INVALID_ARG, "num_blocks must be positive");
  if (p->num_kv_heads <= 0) return fail(PA_ERR_INVALID_ARG, "num_kv_heads must be positive");
  if (p->block_size < 2 || p->block_size > 256 || log2_exact(p->block_size) < 0)
    return fail(PA_ERR_INVALID_ARG, "block_size %d is not a power of two in [2, 256]", p->block_size);
  if (element_size(p->dtype) == 0) return fail(PA_ERR_INVALID_ARG, "unknown pool dtype %d", p->dtype);
  if (!supported_head_dim(p->head_dim))
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d not built (8, 64, 128, 256)", p->head_dim);
  if (p->dtype == PA_FP8_E4M3) {
    if (!(p->k_scale > 0.0f) || !std::isfinite(p->k_scale) || !(p->v_scale > 0.0f) ||
        !std::isfinite(p->v_scale))
      return fail(PA_ERR_INVALID_ARG, "fp8 pool scales must be finite and positive");
  } else if (p->k_scale != 1.0f || p->v_scale != 1.0f) {
    return fail(PA_ERR_INVALID_ARG, "scales must be 1 for a non-fp8 pool");
  }
  // block bytes and slot counts must fit the kernels' 64-bit offsets
  const double bytes = static_cast<double>(p->num_blocks) * p->num_kv_heads * p->block_size *
                       p->head_dim * element_size(p->dtype);
  if (bytes > 9.0e18) return fail(PA_ERR_INVALID_ARG, "pool too large");
  return PA_OK;
}

int hip_fail(hipError_t e) {
  return fail(PA_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(e));
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Query heads per workgroup: the group size rounded up to a power of two, at
// most 8; larger groups are split into head groups of 8.
int heads_per_wg(int group) {
  int h = 1;
  while (h < group && h < 8) h <<= 1;
  return h;
}

// Split-KV scratch.
//  Fixed partitions: one 8-byte counter per (sequence, head group), padded to
//  256 bytes (kept zero; the head-dim-128 split merges in a second launch and
//  does not count arrivals), then float32 partials (m, l and head_dim outputs)
//  for every (sequence, head group, partition, head of the group).
//  Balanced split: 4 KiB of registration and exit counters, one 128-byte
//  counter line per (sequence, head group), then two partial slots per range
//  of every share (one share per XCD, one range per streaming wave).
bool workspace_layout(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size,
                      int32_t partition_size, pa_impl::WorkspaceLayout *w) {
  if ((partition_size <= 0 && partition_size != PA_PARTITION_AUTO) || num_seqs <= 0 ||
      num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads || head_dim <= 0 ||
      max_blocks_per_seq <= 0 || block_size <= 0)
    return false;
  const int group = num_q_heads / num_kv_heads;
  const int hpw = heads_per_wg(group);
  const int64_t hg = ceil_div(group, hpw);
  *w = pa_impl::WorkspaceLayout{};
  w->units = static_cast<int64_t>(num_seqs) * num_kv_heads * hg;
  if (partition_size == PA_PARTITION_AUTO) {
    w->stream_waves = static_cast<int64_t>(pa_impl::device_compute_units()) * pa_impl::kStreamWavesPerCu;
    w->num_xcd = std::min(pa_impl::device_xccs(), 16);   // the control block holds 16 registration counters
    w->share_ranges = pa_impl::kStreamWavesPerCu * ceil_div(w->stream_waves / pa_impl::kStreamWavesPerCu, w->num_xcd);
    w->ctl_bytes = 4096;
    w->counter_bytes = w->units * 128;
    w->partial_floats = w->num_xcd * w->share_ranges * 2 * (hpw * static_cast<int64_t>(head_dim) + pa_impl::kSlotMlFloats);
  } else {
    w->max_parts = ceil_div(static_cast<int64_t>(max_blocks_per_seq) * block_size, partition_size);
    w->counter_bytes = ceil_div(w->units * 8, 256) * 256;
    w->partial_floats = w->units * w->max_parts * hpw * (static_cast<int64_t>(head_dim) + 2);
  }
  return true;
}

}  // namespace

extern "C" {

const char *pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    default: return "PA_ERR_UNKNOWN";
  }
}

const char *pa_last_error(void) { return g_last_error; }

int pa_version(void) { return 100; }

int pa_time_next_decode(void *start_event, void *stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(PA_ERR_INVALID_ARG, "pa_time_next_decode: give both events or neither");
  g_next_events.start = static_cast<hipEvent_t>(start_event);
  g_next_events.stop = static_cast<hipEvent_t>(stop_event);
  return ok();
}

int pa_write_kv(const void *k, const void *v, int32_t src_dtype, int32_t num_tokens,
                const int64_t *slot_mapping, const pa_kv_pool *pool, pa_stream_t stream) {
  if (int st = check_pool(pool)) return st;
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens must be >= 0");
  if (num_tokens == 0) return ok();
  if (!k || !v || !slot_mapping) return fail(PA_ERR_INVALID_ARG, "k, v or slot_mapping is NULL");
  if (element_size(src_dtype) == 0) return fail(PA_ERR_INVALID_ARG, "unknown source dtype %d", src_dtype);
  if (src_dtype != pool->dtype &&
      !(pool->dtype == PA_FP8_E4M3 && src_dtype != PA_FP8_E4M3))
    return fail(PA_ERR_UNSUPPORTED, "write from dtype %d into pool dtype %d not built", src_dtype,
                pool->dtype);
  pa_impl::WriteArgs a{};
  a.k = k;
  a.v = v;
  a.slots = slot_mapping;
  a.k_pool = pool->k_pool;
  a.v_pool = pool->v_pool;
  a.num_slots = pool->num_blocks * pool->block_size;
  a.num_tokens = num_tokens;
  a.num_kv_heads = pool->num_kv_heads;
  a.head_dim = pool->head_dim;
  a.bs_log2 = log2_exact(pool->block_size);
  a.k_inv = 1.0f / pool->k_scale;
  a.v_inv = 1.0f / pool->v_scale;
  const int64_t total_units = static_cast<int64_t>(num_tokens) * pool->num_kv_heads * pool->head_dim;
  if (total_units / 4 / 256 > 0x7fffffffLL) return fail(PA_ERR_INVALID_ARG, "too many tokens");
  bool supported = true;
  hipError_t e = pa_impl::launch_write(src_dtype, pool->dtype, a,
                                       reinterpret_cast<hipStream_t>(stream), &supported);
  if (!supported) return fail(PA_ERR_UNSUPPORTED, "write combination not built");
  if (e != hipSuccess) return hip_fail(e);
  return ok();
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size,
                                 int32_t partition_size) {
  pa_impl::WorkspaceLayout w{};
  if (!workspace_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                        block_size, partition_size, &w))
    return 0;
  return static_cast<size_t>(w.total_bytes());
}

int pa_decode(const void *q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
              const pa_kv_pool *pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
              const int32_t *context_lens, float scale, void *out, int32_t partition_size,
              void *workspace, size_t workspace_bytes, pa_stream_t stream) {
  return pa_impl::decode_entry(q, q_dtype, num_seqs, num_q_heads, pool, block_tables, max_blocks_per_seq,
                               context_lens, 0, scale, out, partition_size, workspace, workspace_bytes,
                               stream, false);
}

int pa_decode_window(const void *q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                     const pa_kv_pool *pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                     const int32_t *context_lens, int32_t window, float scale, void *out,
                     int32_t partition_size, void *workspace, size_t workspace_bytes, pa_stream_t stream) {
  if (window < 0) return fail(PA_ERR_INVALID_ARG, "window must be >= 0");
  return pa_impl::decode_entry(q, q_dtype, num_seqs, num_q_heads, pool, block_tables, max_blocks_per_seq,
                               context_lens, window, scale, out, partition_size, workspace, workspace_bytes,
                               stream, false);
}

}  // extern "C"

namespace pa_impl {

int set_error(int status, const char *msg) { return fail(status, "%s", msg); }

int decode_entry(const void *q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                 const pa_kv_pool *pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                 const int32_t *context_lens, int32_t window, float scale, void *out, int32_t partition_size,
                 void *workspace, size_t workspace_bytes, pa_stream_t stream, bool clear_counters) {
  const pa_impl::LaunchEvents ev = g_next_events;    // the pair applies to this call only
  g_next_events = pa_impl::LaunchEvents{};
  if (int st = check_pool(pool)) return st;
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs must be >= 0");
  if (num_seqs == 0) return ok();
  if (num_seqs > 65535) return fail(PA_ERR_INVALID_ARG, "num_seqs %d above 65535", num_seqs);
  if (!q || !out || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID_ARG, "q, out, block_tables or context_lens is NULL");
  if (q == out) return fail(PA_ERR_INVALID_ARG, "out must not alias q");
  if (num_q_heads <= 0 || num_q_heads % pool->num_kv_heads)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                num_q_heads, pool->num_kv_heads);
  if (max_blocks_per_seq <= 0) return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq must be positive");
  if (static_cast<int64_t>(max_blocks_per_seq) * pool->block_size > 0x7fffffffLL)
    return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq * block_size overflows int32");
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale must be finite");
  if (q_dtype != PA_F32 && q_dtype != PA_F16 && q_dtype != PA_BF16)
    return fail(PA_ERR_INVALID_ARG, "q dtype must be F32, F16 or BF16");
  const bool combo = (q_dtype == pool->dtype) ||
                     (pool->dtype == PA_FP8_E4M3 && (q_dtype == PA_BF16 || q_dtype == PA_F16));
  if (!combo) return fail(PA_ERR_UNSUPPORTED, "q dtype %d with pool dtype %d not built", q_dtype, pool->dtype);
  if (partition_size < 0 && partition_size != PA_PARTITION_AUTO)
    return fail(PA_ERR_INVALID_ARG, "partition_size must be >= 0 or PA_PARTITION_AUTO");
  if (partition_size > 0 && partition_size % pool->block_size)
    return fail(PA_ERR_INVALID_ARG, "partition_size %d is not a multiple of block_size %d",
                partition_size, pool->block_size);

  const int group = num_q_heads / pool->num_kv_heads;
  const int hpw = heads_per_wg(group);
  const int head_groups = static_cast<int>(ceil_div(group, hpw));
  if (static_cast<int64_t>(pool->num_kv_heads) * head_groups > 65535)
    return fail(PA_ERR_INVALID_ARG, "too many heads");

  pa_impl::DecodeArgs a{};
  a.q = q;
  a.k_pool = pool->k_pool;
  a.v_pool = pool->v_pool;
  a.tables = block_tables;
  a.ctx = context_lens;
  a.out = out;
  a.num_blocks = pool->num_blocks;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.group = group;
  a.heads_per_wg = hpw;
  a.head_groups = head_groups;
  a.head_dim = pool->head_dim;
  a.block_size = pool->block_size;
  a.bs_log2 = log2_exact(pool->block_size);
  a.max_blocks = max_blocks_per_seq;
  a.partition_size = partition_size;
  a.max_parts = 1;
  const double log2e = 1.4426950408889634;
  const double ks = pool->dtype == PA_FP8_E4M3 ? static_cast<double>(pool->k_scale) : 1.0;
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * ks * log2e);
  a.v_scale = pool->dtype == PA_FP8_E4M3 ? pool->v_scale : 1.0f;
  a.wait_polls = g_wait_polls;
  a.window = window;

  const bool fast = pa_impl::fast_decode_applies(q_dtype, pool->dtype, a);
  if (partition_size == PA_PARTITION_AUTO && !fast) {
    partition_size = 0;                 // the generic kernel walks each context in one pass
    a.partition_size = 0;
  }
  if (partition_size == PA_PARTITION_AUTO) {
    pa_impl::WorkspaceLayout w{};
    workspace_layout(num_seqs, num_q_heads, pool->num_kv_heads, pool->head_dim, max_blocks_per_seq,
                     pool->block_size, partition_size, &w);
    const size_t need = static_cast<size_t>(w.total_bytes());
    if (!workspace || workspace_bytes < need)
      return fail(PA_ERR_WORKSPACE, "balanced-split workspace needs %zu bytes, got %zu", need,
                  workspace ? workspace_bytes : static_cast<size_t>(0));
    a.partition_size = 0;
    a.stream_waves = static_cast<int32_t>(w.stream_waves);
    a.num_xcd = static_cast<int32_t>(w.num_xcd);
    a.share_ranges = static_cast<int32_t>(w.share_ranges);
    // control words, then the partial slots (their size does not depend on
    // the batch), then a counter line per (sequence, head group): unit u's
    // line sits at the same offset whatever the number of sequences, so one
    // zero-filled workspace serves batches of any size
    char *base = static_cast<char *>(workspace);
    a.ctl = reinterpret_cast<int32_t *>(base);
    float *ws = reinterpret_cast<float *>(base + w.ctl_bytes);
    a.counters = reinterpret_cast<int32_t *>(base + w.ctl_bytes + w.partial_floats * 4);
    const int64_t slots = w.num_xcd * w.share_ranges * 2;
    a.part_o = ws;                                     // [share][range][side][head][D]
    a.part_m = ws + slots * hpw * pool->head_dim;      // [share][range][side][32]: (m, l) per head
  } else if (partition_size > 0) {
    pa_impl::WorkspaceLayout w{};
    workspace_layout(num_seqs, num_q_heads, pool->num_kv_heads, pool->head_dim, max_blocks_per_seq,
                     pool->block_size, partition_size, &w);
    const size_t need = static_cast<size_t>(w.total_bytes());
    if (!workspace || workspace_bytes < need)
      return fail(PA_ERR_WORKSPACE, "split-KV workspace needs %zu bytes, got %zu", need,
                  workspace ? workspace_bytes : static_cast<size_t>(0));
    a.max_parts = static_cast<int32_t>(w.max_parts);
    a.counters = static_cast<int32_t *>(workspace);
    float *ws = reinterpret_cast<float *>(static_cast<char *>(workspace) + w.counter_bytes);
    if (fast) {
      // [unit][part][head][D] outputs, then [unit][part][head][m, l]
      a.part_o = ws;
      a.part_m = ws + w.units * w.max_parts * hpw * pool->head_dim;
      a.part_l = nullptr;
    } else {
      // [S][Hq][part] maxima, [S][Hq][part] sums, [S][Hq][part][D] outputs
      const int64_t rows = static_cast<int64_t>(num_seqs) * num_q_heads * w.max_parts;
      a.part_m = ws;
      a.part_l = ws + rows;
      a.part_o = ws + 2 * rows;
    }
  }
  hipError_t e;
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (clear_counters && partition_size != 0) {
    // the words that must start at zero: the control block and the unit
    // counters of the balanced split, the arrival counters of fixed partitions
    pa_impl::WorkspaceLayout w{};
    workspace_layout(num_seqs, num_q_heads, pool->num_kv_heads, pool->head_dim, max_blocks_per_seq,
                     pool->block_size, partition_size, &w);
    char *base = static_cast<char *>(workspace);
    if (partition_size == PA_PARTITION_AUTO) {
      e = pa_impl::launch_zero(base, w.ctl_bytes, hs);
      if (e == hipSuccess) e = pa_impl::launch_zero(base + w.ctl_bytes + w.partial_floats * 4, w.counter_bytes, hs);
    } else {
      e = pa_impl::launch_zero(base, w.counter_bytes, hs);
    }
    if (e != hipSuccess) return hip_fail(e);
  }
  if (fast) {
    e = pa_impl::launch_decode_fast(q_dtype, pool->dtype, a, hs, ev);
  } else {
    bool supported = true;
    if (ev.start && (e = hipEventRecord(ev.start, hs)) != hipSuccess) return hip_fail(e);
    e = pa_impl::launch_decode(q_dtype, pool->dtype, a, hs, &supported);
    if (!supported) return fail(PA_ERR_UNSUPPORTED, "decode specialisation not built");
    if (e == hipSuccess && ev.stop) e = hipEventRecord(ev.stop, hs);
  }
  if (e != hipSuccess) return hip_fail(e);
  return ok();
}

}  // namespace pa_impl

extern "C" {

int pa_decode_status(const void *workspace, size_t workspace_bytes, int32_t partition_size,
                     int32_t *status, pa_stream_t stream) {
  if (!status) return fail(PA_ERR_INVALID_ARG, "status is NULL");
  if (partition_size < 0 && partition_size != PA_PARTITION_AUTO)
    return fail(PA_ERR_INVALID_ARG, "partition_size must be >= 0 or PA_PARTITION_AUTO");
  const int32_t *word = nullptr;
  if (partition_size == PA_PARTITION_AUTO) {
    if (!workspace || workspace_bytes < 4096)
      return fail(PA_ERR_WORKSPACE, "a balanced-split workspace holds at least 4096 bytes");
    word = reinterpret_cast<const int32_t *>(static_cast<const char *>(workspace) + pa_impl::kWsStatusOffset);
  }
  hipError_t e = pa_impl::launch_status(word, status, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  return ok();
}

int pa_set_wait_polls(int32_t polls) {
  if (polls < 0) return fail(PA_ERR_INVALID_ARG, "polls must be >= 0");
  g_wait_polls = polls == 0 ? pa_impl::kDefaultWaitPolls : polls;
  return ok();
}

int pa_copy_blocks(const pa_kv_pool *pool, const int64_t *src_dst_pairs, int32_t num_pairs,
                   pa_stream_t stream) {
  if (int st = check_pool(pool)) return st;
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARG, "num_pairs must be >= 0");
  if (num_pairs == 0) return ok();
  if (!src_dst_pairs) return fail(PA_ERR_INVALID_ARG, "src_dst_pairs is NULL");
  pa_impl::CopyArgs a{};
  a.src_k = a.dst_k = pool->k_pool;
  a.src_v = a.dst_v = pool->v_pool;
  a.pairs = src_dst_pairs;
  a.src_blocks = a.dst_blocks = pool->num_blocks;
  a.block_bytes = static_cast<int64_t>(pool->num_kv_heads) * pool->block_size * pool->head_dim *
                  element_size(pool->dtype);
  a.num_pairs = num_pairs;
  a.same_pool = 1;
  if (ceil_div(a.block_bytes, 4096) > 65535) return fail(PA_ERR_INVALID_ARG, "block too large");
  hipError_t e = pa_impl::launch_copy(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  return ok();
}

int pa_prefill(const void *q, int32_t q_dtype, int32_t num_tokens, int32_t num_q_heads,
               const pa_kv_pool *pool, int32_t num_seqs, const int32_t *block_tables,
               int32_t max_blocks_per_seq, const int32_t *context_lens, const int32_t *query_start,
               int32_t window, float scale, void *out, pa_stream_t stream) {
  if (int st = check_pool(pool)) return st;
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens must be >= 0");
  if (num_tokens == 0) return ok();
  if (num_seqs <= 0 || num_seqs > 65535) return fail(PA_ERR_INVALID_ARG, "num_seqs must be in [1, 65535]");
  if (!q || !out || !block_tables || !context_lens || !query_start)
    return fail(PA_ERR_INVALID_ARG, "q, out, block_tables, context_lens or query_start is NULL");
  if (q == out) return fail(PA_ERR_INVALID_ARG, "out must not alias q");
  if (num_q_heads <= 0 || num_q_heads % pool->num_kv_heads)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                num_q_heads, pool->num_kv_heads);
  if (max_blocks_per_seq <= 0) return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq must be positive");
  if (static_cast<int64_t>(max_blocks_per_seq) * pool->block_size > 0x7fffffffLL)
    return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq * block_size overflows int32");
  if (window < 0) return fail(PA_ERR_INVALID_ARG, "window must be >= 0");
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale must be finite");
  if (q_dtype != PA_F32 && q_dtype != PA_F16 && q_dtype != PA_BF16)
    return fail(PA_ERR_INVALID_ARG, "q dtype must be F32, F16 or BF16");
  const bool combo = (q_dtype == pool->dtype) ||
                     (pool->dtype == PA_FP8_E4M3 && (q_dtype == PA_BF16 || q_dtype == PA_F16));
  if (!combo) return fail(PA_ERR_UNSUPPORTED, "q dtype %d with pool dtype %d not built", q_dtype, pool->dtype);
  const int group = num_q_heads / pool->num_kv_heads;
  const int hpw = heads_per_wg(group);
  const int head_groups = static_cast<int>(ceil_div(group, hpw));
  if (static_cast<int64_t>(pool->num_kv_heads) * head_groups > 65535)
    return fail(PA_ERR_INVALID_ARG, "too many heads");

  pa_impl::DecodeArgs a{};
  a.q = q;
  a.k_pool = pool->k_pool;
  a.v_pool = pool->v_pool;
  a.tables = block_tables;
  a.ctx = context_lens;
  a.out = out;
  a.num_blocks = pool->num_blocks;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.group = group;
  a.heads_per_wg = hpw;
  a.head_groups = head_groups;
  a.head_dim = pool->head_dim;
  a.block_size = pool->block_size;
  a.bs_log2 = log2_exact(pool->block_size);
  a.max_blocks = max_blocks_per_seq;
  a.partition_size = 0;
  a.max_parts = 1;
  const double ks = pool->dtype == PA_FP8_E4M3 ? static_cast<double>(pool->k_scale) : 1.0;
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * ks * 1.4426950408889634);
  a.v_scale = pool->dtype == PA_FP8_E4M3 ? pool->v_scale : 1.0f;
  a.window = window;
  a.query_start = query_start;
  a.num_tokens = num_tokens;
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (pa_impl::prefill_fast_applies(q_dtype, pool->dtype, a)) {
    e = pa_impl::launch_prefill_fast(q_dtype, a, hs);
  } else {
    bool supported = true;
    e = pa_impl::launch_decode(q_dtype, pool->dtype, a, hs, &supported);
    if (!supported) return fail(PA_ERR_UNSUPPORTED, "prefill specialisation not built");
  }
  if (e != hipSuccess) return hip_fail(e);
  return ok();
}

// Device address a kernel of the current device can use for `p`: device
// memory of the current device as is, pinned host memory through its mapped
// device address; anything else (pageable host memory, another device's
// memory, an unknown pointer) is refused before any launch.
static int kernel_address(const void *p, const char *what, void **out) {
  if (!p) return fail(PA_ERR_INVALID_ARG, "%s is NULL", what);
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();            // leave no error behind for the caller's next call
    return fail(PA_ERR_INVALID_ARG, "%s is not device memory or pinned host memory", what);
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PA_ERR_HIP, "no current device");
  if (at.type == hipMemoryTypeDevice) {
    if (at.device != dev) return fail(PA_ERR_INVALID_ARG, "%s lives on device %d, not the current %d", what, at.device, dev);
    *out = const_cast<void *>(p);
    return PA_OK;
  }
  if (at.type == hipMemoryTypeHost && at.devicePointer) {
    // the mapped address of this exact byte (p may point inside the allocation)
    const char *host_base = static_cast<const char *>(at.hostPointer ? at.hostPointer : p);
    *out = static_cast<char *>(at.devicePointer) + (static_cast<const char *>(p) - host_base);
    return PA_OK;
  }
  return fail(PA_ERR_INVALID_ARG, "%s is not device memory or pinned host memory (hipHostMalloc)", what);
}

int pa_swap_blocks(const pa_kv_pool *src, const pa_kv_pool *dst, const int64_t *src_dst_pairs,
                   int32_t num_pairs, pa_stream_t stream) {
  if (!src || !dst) return fail(PA_ERR_INVALID_ARG, "pool descriptor is NULL");
  // the descriptors' own checks, with the pointer check done below instead
  if (int st = check_pool(src)) return st;
  if (int st = check_pool(dst)) return st;
  if (src->num_kv_heads != dst->num_kv_heads || src->block_size != dst->block_size ||
      src->head_dim != dst->head_dim || src->dtype != dst->dtype)
    return fail(PA_ERR_INVALID_ARG, "source and destination pools differ in block shape or dtype");
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARG, "num_pairs must be >= 0");
  if (num_pairs == 0) return ok();
  pa_impl::CopyArgs a{};
  void *sk, *sv, *dk, *dv, *pairs;
  if (int st = kernel_address(src->k_pool, "source K pool", &sk)) return st;
  if (int st = kernel_address(src->v_pool, "source V pool", &sv)) return st;
  if (int st = kernel_address(dst->k_pool, "destination K pool", &dk)) return st;
  if (int st = kernel_address(dst->v_pool, "destination V pool", &dv)) return st;
  if (int st = kernel_address(src_dst_pairs, "src_dst_pairs", &pairs)) return st;
  a.src_k = sk;
  a.src_v = sv;
  a.dst_k = dk;
  a.dst_v = dv;
  a.pairs = static_cast<const int64_t *>(pairs);
  a.src_blocks = src->num_blocks;
  a.dst_blocks = dst->num_blocks;
  a.block_bytes = static_cast<int64_t>(src->num_kv_heads) * src->block_size * src->head_dim *
                  element_size(src->dtype);
  a.num_pairs = num_pairs;
  a.same_pool = (src->k_pool == dst->k_pool) ? 1 : 0;
  if (ceil_div(a.block_bytes, 4096) > 65535) return fail(PA_ERR_INVALID_ARG, "block too large");
  hipError_t e = pa_impl::launch_copy(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  return ok();
}

}  // extern "C"
