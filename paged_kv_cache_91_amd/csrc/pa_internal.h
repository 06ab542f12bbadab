// Internal interface between the C ABI layer (pa_api.cpp) and the HIP
// kernels (pa_kernels.hip).  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "pa.h"

namespace pa_impl {

// Element storage codes; equal to the public pa_dtype values.
enum Dt : int { kF32 = 0, kF16 = 1, kBF16 = 2, kFP8 = 3 };

struct DecodeArgs {
  const void *q;
  const void *k_pool;
  const void *v_pool;
  const int32_t *tables;   // [S][max_blocks]
  const int32_t *ctx;      // [S]
  void *out;               // [S][Hq][D]
  float *part_m;           // split mode: [S][Hq][max_parts]
  float *part_l;           // split mode: [S][Hq][max_parts]
  float *part_o;           // split mode: [S][Hq][max_parts][D]
  int32_t *counters;       // split mode: per (sequence, head group) counters; zero between calls
  int32_t *ctl;            // balanced split: registration counters and the poison word; zero between calls
  int64_t num_blocks;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;           // Hq / Hkv
  int32_t heads_per_wg;    // power of two <= 8
  int32_t head_groups;     // ceil(group / heads_per_wg)
  int32_t head_dim;
  int32_t block_size;
  int32_t bs_log2;
  int32_t max_blocks;
  int32_t partition_size;  // 0 = single pass
  int32_t stream_waves;    // > 0: balanced (stream-K) split over this many single-wave workgroups
  int32_t max_parts;       // partitions per sequence in the workspace (1 if single pass)
  int32_t num_xcd;         // balanced split: XCDs of the device (one share each)
  int32_t share_ranges;    // balanced split: ranges per share the partial slots are sized for
  float scale_log2;        // scale * k_scale * log2(e)
  float v_scale;           // 1 unless fp8
  int32_t wait_polls;      // balanced split: polls before a wait between waves of a workgroup gives up
  int32_t window;          // sliding window: positions max(0, n - window) .. n-1 (0: the whole context)
  // prefill (causal, several queries per sequence): non-null query_start
  // [S + 1] gives sequence s the q / out rows query_start[s] .. query_start[s+1]-1,
  // which stand for its last positions; num_tokens = query_start[S]
  const int32_t *query_start;
  int32_t num_tokens;
};

// Polls (each about 30-80 ns) before a wait between the waves of one
// workgroup gives up: far beyond any wait the protocol has (a peer wave's
// handling of one mailbox entry, microseconds).
constexpr int32_t kDefaultWaitPolls = 1 << 20;
// Byte offset of the balanced split's status word in its workspace.
constexpr int64_t kWsStatusOffset = 4 * 32 * 17;

struct WriteArgs {
  const void *k;
  const void *v;
  const int64_t *slots;
  void *k_pool;
  void *v_pool;
  int64_t num_slots;       // num_blocks * block_size
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t bs_log2;
  float k_inv;             // 1 / k_scale (fp8 destination)
  float v_inv;
};

struct CopyArgs {
  const void *src_k;       // source pools (device, or pinned host memory's device address)
  const void *src_v;
  void *dst_k;             // destination pools (the source pools for a copy within one pool)
  void *dst_v;
  const int64_t *pairs;    // [num_pairs][2] (src block, dst block)
  int64_t src_blocks;      // blocks in the source pools
  int64_t dst_blocks;      // blocks in the destination pools
  int64_t block_bytes;     // Hkv * bs * D * element size
  int32_t num_pairs;
  int32_t same_pool;       // 1: copy within one pool (pairs with src == dst are skipped)
};

// Each returns hipSuccess or the launch error; `supported` (when given) is
// set false for combinations no kernel was built for.
hipError_t launch_decode(int q_dtype, int kv_dtype, const DecodeArgs &a, hipStream_t s,
                         bool *supported);
hipError_t launch_write(int src_dtype, int dst_dtype, const WriteArgs &a, hipStream_t s,
                        bool *supported);
hipError_t launch_copy(const CopyArgs &a, hipStream_t s);
// *out = word ? *word : 0, one thread, on stream s
hipError_t launch_status(const int32_t *word, int32_t *out, hipStream_t s);
// zero `bytes` bytes at p (a multiple of 16, 16-byte aligned) with a fill kernel
hipError_t launch_zero(void *p, int64_t bytes, hipStream_t s);

// Events the launch records as its first kernel begins and its last kernel
// ends (none when null).
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
// one launcher per (q, cache) dtype pair (each built from pa_decode_fast.hip)
hipError_t launch_fast_bf16_bf16(const DecodeArgs &a, hipStream_t s, const LaunchEvents &ev);
hipError_t launch_fast_f16_f16(const DecodeArgs &a, hipStream_t s, const LaunchEvents &ev);
hipError_t launch_fast_bf16_fp8(const DecodeArgs &a, hipStream_t s, const LaunchEvents &ev);
hipError_t launch_fast_f16_fp8(const DecodeArgs &a, hipStream_t s, const LaunchEvents &ev);
inline bool fast_decode_applies(int q_dtype, int kv_dtype, const DecodeArgs &a) {
  if (a.head_dim != 128 || (a.block_size != 16 && a.block_size != 32)) return false;
  if (q_dtype != kBF16 && q_dtype != kF16) return false;
  return kv_dtype == q_dtype || kv_dtype == kFP8;
}
inline hipError_t launch_decode_fast(int q_dtype, int kv_dtype, const DecodeArgs &a, hipStream_t s,
                                     const LaunchEvents &ev) {
  if (q_dtype == kBF16 && kv_dtype == kBF16) return launch_fast_bf16_bf16(a, s, ev);
  if (q_dtype == kF16 && kv_dtype == kF16) return launch_fast_f16_f16(a, s, ev);
  if (q_dtype == kBF16 && kv_dtype == kFP8) return launch_fast_bf16_fp8(a, s, ev);
  if (q_dtype == kF16 && kv_dtype == kFP8) return launch_fast_f16_fp8(a, s, ev);
  return hipErrorInvalidValue;
}

// Prefill (pa_prefill.hip): the matrix-core kernel for head_dim 128, block
// 16/32, 16-bit caches and groups 1, 2, 4, 8; prefill_fast_applies() says
// whether it covers a call (else the generic kernel's prefill mode runs).
bool prefill_fast_applies(int q_dtype, int kv_dtype, const DecodeArgs &a);
hipError_t launch_prefill_fast(int q_dtype, const DecodeArgs &a, hipStream_t s);

// Compute units of the current device (256 when it cannot be queried, e.g.
// on a machine without a GPU, where only sizes are computed).
inline int device_compute_units() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  return cus;
}

// XCDs of the current device (8, the MI355X count, when it cannot be
// queried).
inline int device_xccs() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 8;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || n <= 0) return 8;
  return n;
}

// Streaming waves per compute unit in the balanced split (one per SIMD, each
// with a helper wave); its workspace holds two partials per streaming wave.
constexpr int kStreamWavesPerCu = 4;
// Balanced split: floats per partial slot's (m, l) block, one 128-byte line
// (pairs for up to 16 heads).  No two slots share a line, so a compute unit
// that loads one slot never caches a line of another slot that is not yet
// published.
constexpr int kSlotMlFloats = 32;

// Record `msg` for pa_last_error() on this thread; returns status.
int set_error(int status, const char *msg);

// The body of pa_decode and pa_decode_window (pa_api.cpp); window 0 is the
// whole context.  With clear_counters, the words of
// the workspace that must start at zero are zero-filled on the stream first
// (after validation, so a failing call still enqueues nothing).
int decode_entry(const void *q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                 const pa_kv_pool *pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                 const int32_t *context_lens, int32_t window, float scale, void *out, int32_t partition_size,
                 void *workspace, size_t workspace_bytes, pa_stream_t stream, bool clear_counters);

// Workspace layout shared by the API layer and the kernels.
struct WorkspaceLayout {
  int64_t units;           // S * Hkv * head_groups
  int64_t max_parts;       // fixed partitions per sequence (0 in the balanced split)
  int64_t stream_waves;    // balanced split: streaming waves the workspace is sized for
  int64_t num_xcd;         // balanced split: shares (one per XCD)
  int64_t share_ranges;    // balanced split: ranges per share
  int64_t ctl_bytes;       // balanced split: registration counters and the poison word, 128-byte lines
  int64_t counter_bytes;   // per unit: 8 bytes (fixed partitions) or a 128-byte line (balanced split)
  int64_t partial_floats;  // partials: heads_per_wg * (head_dim + 2) floats each
  int64_t total_bytes() const { return ctl_bytes + counter_bytes + partial_floats * 4; }
};

}  // namespace pa_impl
