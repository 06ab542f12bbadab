// pa_decode_noalloc: pa_decode whose split-KV scratch is a static device
// array of the library, for callers that cannot allocate device memory
// (code under stream capture, tight serving loops, harnesses that forbid
// allocation).  Declared in include/pa.h.
//
// The array lives in the library's code object: every GPU the library runs
// on holds its own copy from the first call on that GPU until the process
// ends.  Host code never passes the array's name to a kernel (on the host it
// is only a stand-in for the symbol); it passes the device address that
// hipGetSymbolAddress returns, taken once per device with that device
// current.

#include <hip/hip_runtime.h>

#include <mutex>

#include "pa.h"
#include "pa_internal.h"

namespace {

// PA_NOALLOC_SCRATCH_BYTES (32 MiB): the balanced split of every batch shape
// up to ~190,000 (sequence, head group) units, and fixed partitions while
// units x partitions x heads x (head_dim + 2) x 4 bytes fit.
constexpr size_t kScratchBytes = PA_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device, once taken

// The current device's copy of `scratch`; hipGetSymbolAddress the first
// time a device is seen (with that device current).
hipError_t scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int pa_decode_noalloc(const void *q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                      const pa_kv_pool *pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                      const int32_t *context_lens, float scale, void *out, int32_t partition_size,
                      pa_stream_t stream) {
  void *ws = nullptr;
  size_t ws_bytes = 0;
  if (partition_size != 0 && pool && num_seqs > 0) {
    const size_t need = pa_decode_workspace_bytes(num_seqs, num_q_heads, pool->num_kv_heads, pool->head_dim,
                                                  max_blocks_per_seq, pool->block_size, partition_size);
    if (need > kScratchBytes) {
      char msg[200];
      snprintf(msg, sizeof(msg), "split needs %zu bytes of scratch; the static scratch holds %zu "
               "(pass a workspace to pa_decode instead)", need, kScratchBytes);
      return pa_impl::set_error(PA_ERR_WORKSPACE, msg);
    }
    if (need > 0) {
      const hipError_t e = scratch_address(&ws);
      if (e != hipSuccess) {
        char msg[200];
        snprintf(msg, sizeof(msg), "hipGetSymbolAddress of the static scratch failed: %s", hipGetErrorString(e));
        return pa_impl::set_error(PA_ERR_HIP, msg);
      }
      ws_bytes = kScratchBytes;
    }
  }
  // pa_decode's validation and kernels, with the scratch's counters zeroed
  // on the stream ahead of them (the scratch keeps the last call's contents)
  return pa_impl::decode_entry(q, q_dtype, num_seqs, num_q_heads, pool, block_tables, max_blocks_per_seq,
                               context_lens, 0, scale, out, partition_size, ws, ws_bytes, stream, true);
}

}  // extern "C"
