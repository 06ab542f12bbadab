// HIP kernels for the paged KV-cache hot path on gfx950 (CDNA4, wave64).
//
//   write_kv_kernel      cache write through a slot mapping (ultralytics.com
//                        "PagedAttention", section "페이징의 작동 방식": position
//                        pos lives at [table[pos / bs], pos % bs]; vasteelab.pages.dev
//                        "PagedAttentionとは？", section on the attention kernel and
//                        memory manager: K/V are written through a slot mapping).
//   copy_blocks_kernel   copy-on-write block copy (vasteelab.pages.dev, section
//                        "Copy-on-Writeで共通prefixを共有できる").
//   decode_kernel        attention of one query token per sequence over its paged
//                        K/V, walking the block table in logical order and
//                        fusing the gather with the dot products (gufacode.com
//                        "PagedAttention:KV cache 的页表革命", section
//                        "PagedAttention CUDA Kernel").  Softmax is evaluated
//                        online (running max / sum, accumulator rescaled), the
//                        tiling that keeps the score vector out of memory
//                        (ultralytics.com, section "관련 기법", FlashAttention).
//   reduce_kernel        merge of split-KV partials with log-sum-exp weights,
//                        in increasing partition order.
//
// Data layout: pools [num_blocks][Hkv][bs][D]; one (block, head) tile is a
// contiguous bs x D slab, so each lane reads whole 16-byte (8-byte for fp8)
// runs of a K or V row.  K/V bytes are consumed once by exactly one wave, so
// they go straight from global memory to registers; the next tile's loads are
// issued before the current tile is computed.
//
// Softmax statistics are kept in the base-2 domain: scores are multiplied by
// scale * log2(e) once, and exp2 is the hardware v_exp_f32.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "pa_common.h"
#include "pa_internal.h"

namespace pa_impl {
namespace {

// ---------------------------------------------------------------------------
// cross-lane reductions
// ---------------------------------------------------------------------------

template <int FROM, int TO>
__device__ __forceinline__ float xor_sum(float v) {
#pragma unroll
  for (int o = FROM; o < TO; o <<= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
template <int FROM, int TO>
__device__ __forceinline__ float xor_max(float v) {
#pragma unroll
  for (int o = FROM; o < TO; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// ---------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------

constexpr int kDecodeWaves = 4;

// The sequence whose query rows hold packed row t: the last s with
// query_start[s] <= t (query_start is nondecreasing, so those s form a
// prefix), found 64 sequences per wave-wide load.
__device__ __forceinline__ int seq_of_row(const DecodeArgs &a, int t, int lane) {
  int count = 0;
  for (int c0 = 0; c0 < a.num_seqs; c0 += kWave) {
    const int s = c0 + lane;
    const bool le = s < a.num_seqs && a.query_start[s] <= t;
    const int k = __popcll(__ballot(le));
    count += k;
    if (k < kWave) break;
  }
  return count - 1;
}

template <typename QS, typename KS, int D, int GT>
struct DecodeKernel {
  using KV = Kv<KS>;
  using Raw = typename KV::Raw;
  static constexpr int E = (KV::kElems < D) ? KV::kElems : D;   // elements per lane
  static constexpr int LPR = D / E;                              // lanes per K/V row
  static constexpr int RPW = kWave / LPR;                        // rows per wave load
  // positions per wave tile: at least 16, at most 8 loads of K (and of V) per lane
  static constexpr int TP = (RPW >= 16) ? RPW : ((8 * RPW < 16) ? 8 * RPW : 16);
  static constexpr int CH = TP / RPW;                            // loads per tile (K and V each)
  static_assert(E == KV::kElems, "head_dim smaller than one lane load is not built");
  static_assert(LPR >= 1 && LPR <= kWave && (LPR & (LPR - 1)) == 0, "bad lane split");

  struct Tile {
    Raw k[CH];
    Raw v[CH];
  };

  // Issue the K/V loads of the wave tile starting at position `base`.
  // UNIFORM: every chunk of RPW positions lies inside one block (RPW <= bs),
  // so its table entry is wave-uniform.
  // Positions outside [pbeg, pend) are read from the block of pbeg or
  // pend - 1 instead (in bounds, and never a released block before a
  // window) and masked by the caller.
  template <bool UNIFORM>
  static __device__ __forceinline__ void load_tile(
      Tile &t, int base, int pbeg, int pend, int row, int col, const int32_t *__restrict__ trow,
      const uint8_t *__restrict__ kbase, const uint8_t *__restrict__ vbase, int64_t block_bytes,
      int bs_log2, int64_t num_blocks, bool &bad) {
    const int bs_mask = (1 << bs_log2) - 1;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      int j, off;
      if constexpr (UNIFORM) {
        const int c0 = base + c * RPW;
        j = max(min(c0, pend - 1), pbeg) >> bs_log2;
        off = (c0 & bs_mask) + row;
      } else {
        const int p = max(min(base + c * RPW + row, pend - 1), pbeg);
        j = p >> bs_log2;
        off = p & bs_mask;
      }
      int64_t phys = trow[j];
      if (static_cast<uint64_t>(phys) >= static_cast<uint64_t>(num_blocks)) {
        bad = true;
        phys = 0;
      }
      const int64_t o = phys * block_bytes + static_cast<int64_t>((off * D + col * E) * KV::kSize);
      t.k[c] = *reinterpret_cast<const Raw *>(kbase + o);
      t.v[c] = *reinterpret_cast<const Raw *>(vbase + o);
    }
  }

  template <bool UNIFORM>
  static __device__ void run(const DecodeArgs &a) {
    const int kvh = blockIdx.y / a.head_groups;
    const int hg = blockIdx.y - kvh * a.head_groups;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int row = lane / LPR;
    const int col = lane % LPR;
    const int maxn = a.max_blocks * (1 << a.bs_log2);

    // decode: sequence blockIdx.z, partition blockIdx.x, its q / out row;
    // prefill: q / out row blockIdx.x of sequence `seq`, attending its
    // positions 0 .. p (n = p + 1)
    int part, seq, n;
    int64_t qrow;
    bool bad_len;
    if (a.query_start) {
      const int t = blockIdx.x;
      seq = max(seq_of_row(a, t, lane), 0);
      const int ns = a.ctx[seq];
      const int q0 = a.query_start[seq];
      const int L = a.query_start[seq + 1] - q0;
      // a malformed prefix sum (row outside its sequence's range) or length
      // gives NaN rows
      bad_len = ns < 0 || ns > maxn || L > ns || t < q0 || t >= q0 + L;
      n = bad_len ? 0 : ns - L + (t - q0) + 1;
      part = 0;
      qrow = t;
    } else {
      part = blockIdx.x;
      seq = blockIdx.z;
      n = a.ctx[seq];
      bad_len = n < 0 || n > maxn;
      qrow = seq;
    }
    // positions [pstart, pend); with a window, partitions are counted from
    // the one holding the window's first position
    const int lo = bad_len ? 0 : window_lo(n, a.window);
    int pstart = lo, pend = n;
    if (a.partition_size > 0) {
      const int ap = lo / a.partition_size + part;
      pstart = max(lo, ap * a.partition_size);
      pend = min(n, (ap + 1) * a.partition_size);
      if (!bad_len && ap * a.partition_size >= n) return;   // partition past the context: no partial
    }

    // query heads handled here: hq0 .. hq0 + GT - 1, valid while h < hcount
    const int hq0 = kvh * a.group + hg * GT;
    const int hcount = min(GT, a.group - hg * GT);

    __shared__ float s_m[kDecodeWaves][GT];
    __shared__ float s_l[kDecodeWaves][GT];
    __shared__ float s_acc[kDecodeWaves][GT][D];

    if (bad_len || n == 0) {
      // n == 0 (single pass): zero row.  Out-of-range n: NaN row.
      const float fill = bad_len ? __builtin_nanf("") : 0.0f;
      for (int i = threadIdx.x; i < GT * D; i += kDecodeWaves * kWave) {
        const int h = i / D, d = i % D;
        if (h >= hcount) continue;
        const int64_t oi = (qrow * a.num_q_heads + hq0 + h);
        if (a.partition_size > 0) {
          if (d == 0) { a.part_m[oi * a.max_parts + part] = fill; a.part_l[oi * a.max_parts + part] = fill; }
          a.part_o[(oi * a.max_parts + part) * D + d] = fill;
        } else {
          Qv<QS>::put(a.out, oi * D + d, fill);
        }
      }
      return;
    }

    // q for this lane's E dims, GT heads, as float
    float q[GT][E];
#pragma unroll
    for (int h = 0; h < GT; ++h) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        q[h][e] = (h < hcount)
            ? Qv<QS>::get(a.q, (qrow * a.num_q_heads + hq0 + h) * D + col * E + e)
            : 0.0f;
      }
    }

    float m_run[GT], l_run[GT], acc[GT][E];
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      m_run[h] = -INFINITY;
      l_run[h] = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[h][e] = 0.0f;
    }

    const int64_t head_bytes = static_cast<int64_t>(D) * KV::kSize << a.bs_log2;
    const int64_t block_bytes = head_bytes * a.num_kv_heads;
    const uint8_t *kbase = static_cast<const uint8_t *>(a.k_pool) + kvh * head_bytes;
    const uint8_t *vbase = static_cast<const uint8_t *>(a.v_pool) + kvh * head_bytes;
    const int32_t *trow = a.tables + static_cast<int64_t>(seq) * a.max_blocks;
    bool bad = false;

    // tiles start on a multiple of TP (so each load chunk stays inside one
    // block); positions before pstart are masked
    const int tstart = pstart & ~(TP - 1);
    const int ntiles = (pend - tstart + TP - 1) / TP;
    Tile cur, nxt;
    if (wave < ntiles)
      load_tile<UNIFORM>(cur, tstart + wave * TP, pstart, pend, row, col, trow, kbase, vbase, block_bytes,
                         a.bs_log2, a.num_blocks, bad);

    for (int t = wave; t < ntiles; t += kDecodeWaves) {
      const int base = tstart + t * TP;
      if (t + kDecodeWaves < ntiles)
        load_tile<UNIFORM>(nxt, base + kDecodeWaves * TP, pstart, pend, row, col, trow, kbase, vbase,
                           block_bytes, a.bs_log2, a.num_blocks, bad);

      // scores of this tile: sc[c][h] for position base + c*RPW + row
      float sc[CH][GT];
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        float kf[E];
        KV::widen(cur.k[c], kf);
        const int pos = base + c * RPW + row;
        const bool valid = pos >= pstart && pos < pend;
#pragma unroll
        for (int h = 0; h < GT; ++h) {
          float s = 0.0f;
#pragma unroll
          for (int e = 0; e < E; ++e) s = fmaf(q[h][e], kf[e], s);
          s = xor_sum<1, LPR>(s);
          sc[c][h] = valid ? s * a.scale_log2 : -INFINITY;
        }
      }

      // online softmax update
      float p[CH][GT];
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        float tmax = sc[0][h];
#pragma unroll
        for (int c = 1; c < CH; ++c) tmax = fmaxf(tmax, sc[c][h]);
        tmax = xor_max<LPR, kWave>(tmax);                 // over all rows of the wave
        const float m_new = fmaxf(m_run[h], tmax);
        const float alpha = __builtin_amdgcn_exp2f(m_run[h] - m_new);
        m_run[h] = m_new;
        l_run[h] *= alpha;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] *= alpha;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          p[c][h] = __builtin_amdgcn_exp2f(sc[c][h] - m_new);
          l_run[h] += p[c][h];
        }
      }

      // P . V
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        float vf[E];
        KV::widen(cur.v[c], vf);
        const int pos = base + c * RPW + row;
        const bool valid = pos >= pstart && pos < pend;
#pragma unroll
        for (int e = 0; e < E; ++e) vf[e] = valid ? vf[e] : 0.0f;
#pragma unroll
        for (int h = 0; h < GT; ++h) {
#pragma unroll
          for (int e = 0; e < E; ++e) acc[h][e] = fmaf(p[c][h], vf[e], acc[h][e]);
        }
      }
      cur = nxt;
    }

    // sum the per-row partials of l and acc over the wave's rows
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      l_run[h] = xor_sum<LPR, kWave>(l_run[h]);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[h][e] = xor_sum<LPR, kWave>(acc[h][e]);
    }
    if (row == 0) {
#pragma unroll
      for (int h = 0; h < GT; ++h) {
#pragma unroll
        for (int e = 0; e < E; ++e) s_acc[wave][h][col * E + e] = acc[h][e];
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        s_m[wave][h] = m_run[h];
        s_l[wave][h] = l_run[h];
      }
    }
    const bool any_bad = __syncthreads_or(bad);

    // merge the waves in wave order and write
    for (int i = threadIdx.x; i < GT * D; i += kDecodeWaves * kWave) {
      const int h = i / D, d = i % D;
      if (h >= hcount) continue;
      float big_m = s_m[0][h];
#pragma unroll
      for (int w = 1; w < kDecodeWaves; ++w) big_m = fmaxf(big_m, s_m[w][h]);
      float l = 0.0f, o = 0.0f;
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(s_m[w][h] - big_m);
        l = fmaf(s_l[w][h], f, l);
        o = fmaf(s_acc[w][h][d], f, o);
      }
      const int64_t oi = qrow * a.num_q_heads + hq0 + h;
      if (a.partition_size > 0) {
        const float nanv = __builtin_nanf("");
        if (d == 0) {
          a.part_m[oi * a.max_parts + part] = any_bad ? nanv : big_m;
          a.part_l[oi * a.max_parts + part] = any_bad ? nanv : l;
        }
        a.part_o[(oi * a.max_parts + part) * D + d] = any_bad ? nanv : o * a.v_scale;
      } else {
        Qv<QS>::put(a.out, oi * D + d, any_bad ? __builtin_nanf("") : o * a.v_scale / l);
      }
    }
  }
};

template <typename QS, typename KS, int D, int GT>
__global__ __launch_bounds__(kDecodeWaves * kWave) void decode_kernel(DecodeArgs a) {
  using K = DecodeKernel<QS, KS, D, GT>;
  if ((1 << a.bs_log2) >= K::RPW)
    K::template run<true>(a);
  else
    K::template run<false>(a);
}

// Merge split-KV partials: one workgroup per (query head, sequence).
template <typename QS>
__global__ __launch_bounds__(256) void reduce_kernel(DecodeArgs a) {
  const int hq = blockIdx.x;
  const int seq = blockIdx.y;
  const int n = a.ctx[seq];
  const int64_t oi = static_cast<int64_t>(seq) * a.num_q_heads + hq;
  const int D = a.head_dim;
  if (n < 0 || n > a.max_blocks * (1 << a.bs_log2)) {
    for (int d = threadIdx.x; d < D; d += blockDim.x) Qv<QS>::put(a.out, oi * D + d, __builtin_nanf(""));
    return;
  }
  const int parts = (n + a.partition_size - 1) / a.partition_size - window_lo(n, a.window) / a.partition_size;
  const float *pm = a.part_m + oi * a.max_parts;
  const float *pl = a.part_l + oi * a.max_parts;
  float big_m = -INFINITY;
  for (int p = 0; p < parts; ++p) big_m = fmaxf(big_m, pm[p]);
  bool nan_seen = false;
  for (int p = 0; p < parts; ++p) nan_seen |= (pm[p] != pm[p]);
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float l = 0.0f, o = 0.0f;
    for (int p = 0; p < parts; ++p) {
      const float f = __builtin_amdgcn_exp2f(pm[p] - big_m);
      l = fmaf(pl[p], f, l);
      o = fmaf(a.part_o[(oi * a.max_parts + p) * D + d], f, o);
    }
    const float r = parts == 0 ? 0.0f : (nan_seen ? __builtin_nanf("") : o / l);
    Qv<QS>::put(a.out, oi * D + d, r);
  }
}

template <typename QS, typename KS, int D>
hipError_t launch_decode_d(const DecodeArgs &a, hipStream_t s) {
  const dim3 grid(a.query_start ? a.num_tokens : (a.partition_size > 0 ? a.max_parts : 1),
                  a.num_kv_heads * a.head_groups, a.query_start ? 1 : a.num_seqs);
  const dim3 block(kDecodeWaves * kWave);
  switch (a.heads_per_wg) {
    case 1: hipLaunchKernelGGL((decode_kernel<QS, KS, D, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_kernel<QS, KS, D, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_kernel<QS, KS, D, 4>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((decode_kernel<QS, KS, D, 8>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.partition_size == 0) return e;
  hipLaunchKernelGGL((reduce_kernel<QS>), dim3(a.num_q_heads, a.num_seqs), dim3(D < 256 ? D : 256), 0, s, a);
  return hipGetLastError();
}

template <typename QS, typename KS>
hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t s, bool *supported) {
  switch (a.head_dim) {
    case 8: return launch_decode_d<QS, KS, 8>(a, s);
    case 64: return launch_decode_d<QS, KS, 64>(a, s);
    case 128: return launch_decode_d<QS, KS, 128>(a, s);
    case 256: return launch_decode_d<QS, KS, 256>(a, s);
    default: if (supported) *supported = false; return hipSuccess;
  }
}

// ---------------------------------------------------------------------------
// cache write
// ---------------------------------------------------------------------------

// Thread i of a write handles piece i % 2^units_log2 of row i >> units_log2,
// row r = token * num_kv_heads + head.  The source bytes do not depend on
// the slot, so they are loaded before it: one memory round trip, not two.
// (r / heads is done in 32 bits whenever r fits, as in every realistic batch.)
__device__ __forceinline__ int64_t write_token(int64_t r, int heads) {
  return r < (int64_t{1} << 32) ? static_cast<int64_t>(static_cast<uint32_t>(r) / static_cast<uint32_t>(heads))
                                : r / heads;
}

// Same-dtype write: one thread moves UNIT bytes of one (token, head) row.
template <int UNIT>
__global__ __launch_bounds__(256) void write_copy_kernel(WriteArgs a, int units_log2) {
  using U = typename std::conditional<UNIT == 16, uint4, uint2>::type;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t r = i >> units_log2;
  if (r >= static_cast<int64_t>(a.num_tokens) * a.num_kv_heads) return;
  const int64_t row_bytes = static_cast<int64_t>(UNIT) << units_log2;
  const int64_t piece = (i & ((int64_t{1} << units_log2) - 1)) * UNIT;
  const int64_t src = r * row_bytes + piece;
  const U kx = *reinterpret_cast<const U *>(static_cast<const uint8_t *>(a.k) + src);
  const U vx = *reinterpret_cast<const U *>(static_cast<const uint8_t *>(a.v) + src);
  const int64_t t = write_token(r, a.num_kv_heads);
  const int64_t h = r - t * a.num_kv_heads;
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= a.num_slots) return;
  const int64_t blk = slot >> a.bs_log2;
  const int64_t off = slot & ((1 << a.bs_log2) - 1);
  const int64_t dst = (((blk * a.num_kv_heads + h) << a.bs_log2) + off) * row_bytes + piece;
  *reinterpret_cast<U *>(static_cast<uint8_t *>(a.k_pool) + dst) = kx;
  *reinterpret_cast<U *>(static_cast<uint8_t *>(a.v_pool) + dst) = vx;
}

// Quantising write into an e4m3 pool: one thread encodes 8 elements
// (4 for float sources: one 16-byte source load either way).
template <typename SS>
__global__ __launch_bounds__(256) void write_fp8_kernel(WriteArgs a, int units_log2) {
  constexpr int E = std::is_same<SS, F32S>::value ? 4 : 8;
  using KV = Kv<SS>;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t r = i >> units_log2;
  if (r >= static_cast<int64_t>(a.num_tokens) * a.num_kv_heads) return;
  const int64_t elem = (i & ((int64_t{1} << units_log2) - 1)) * E;
  const int64_t src = (r * a.head_dim + elem) * KV::kSize;
  const uint4 raw[2] = {*reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(a.k) + src),
                        *reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(a.v) + src)};
  const int64_t t = write_token(r, a.num_kv_heads);
  const int64_t h = r - t * a.num_kv_heads;
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= a.num_slots) return;
  const int64_t blk = slot >> a.bs_log2;
  const int64_t off = slot & ((1 << a.bs_log2) - 1);
  const int64_t dst = (((blk * a.num_kv_heads + h) << a.bs_log2) + off) * a.head_dim + elem;
  for (int which = 0; which < 2; ++which) {
    const float inv = which ? a.v_inv : a.k_inv;
    float f[8];
    KV::widen(raw[which], f);
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < E; ++e) w[e >> 2] |= f32_to_e4m3(f[e] * inv) << (8 * (e & 3));
    uint8_t *dp = static_cast<uint8_t *>(which ? a.v_pool : a.k_pool) + dst;
    if constexpr (E == 8) {
      *reinterpret_cast<uint2 *>(dp) = make_uint2(w[0], w[1]);
    } else {
      *reinterpret_cast<uint32_t *>(dp) = w[0];
    }
  }
}

// ---------------------------------------------------------------------------
// block copy
// ---------------------------------------------------------------------------

// Whole-block copies: within one pool (copy-on-write) or from one pool to
// another of the same block shape (the swap between the GPU pool and pinned
// host memory, whose loads or stores then cross the host link).
// grid: (num_pairs, 2 [K, V], ceil(block_bytes / 4096)); 256 threads x 16 B.
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyArgs a) {
  const int pair = blockIdx.x;
  const int64_t src = a.pairs[2 * pair];
  const int64_t dst = a.pairs[2 * pair + 1];
  if (src < 0 || dst < 0 || src >= a.src_blocks || dst >= a.dst_blocks || (a.same_pool && src == dst)) return;
  const uint8_t *from = static_cast<const uint8_t *>(blockIdx.y ? a.src_v : a.src_k);
  uint8_t *to = static_cast<uint8_t *>(blockIdx.y ? a.dst_v : a.dst_k);
  const int64_t off = static_cast<int64_t>(blockIdx.z) * 4096 + threadIdx.x * 16;
  if (off >= a.block_bytes) return;
  *reinterpret_cast<uint4 *>(to + dst * a.block_bytes + off) =
      *reinterpret_cast<const uint4 *>(from + src * a.block_bytes + off);
}

// zero fill, 16 bytes a thread (a kernel rather than a memset node, so the
// fill is safe to capture in a graph)
__global__ __launch_bounds__(256) void zero_kernel(uint4 *p, int64_t n16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// the balanced split's workspace status word, copied where the caller asks
__global__ __launch_bounds__(64) void status_kernel(const int32_t *word, int32_t *out) {
  if (threadIdx.x == 0) *out = word ? __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

hipError_t launch_decode(int q_dtype, int kv_dtype, const DecodeArgs &a, hipStream_t s,
                         bool *supported) {
  if (supported) *supported = true;
  if (q_dtype == kF32 && kv_dtype == kF32) return launch_decode_t<F32S, F32S>(a, s, supported);
  if (q_dtype == kF16 && kv_dtype == kF16) return launch_decode_t<F16S, F16S>(a, s, supported);
  if (q_dtype == kBF16 && kv_dtype == kBF16) return launch_decode_t<BF16S, BF16S>(a, s, supported);
  if (q_dtype == kBF16 && kv_dtype == kFP8) return launch_decode_t<BF16S, FP8S>(a, s, supported);
  if (q_dtype == kF16 && kv_dtype == kFP8) return launch_decode_t<F16S, FP8S>(a, s, supported);
  if (supported) *supported = false;
  return hipSuccess;
}

// log2 of a power of two
static int log2_int(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

hipError_t launch_write(int src_dtype, int dst_dtype, const WriteArgs &a, hipStream_t s,
                        bool *supported) {
  if (supported) *supported = true;
  const int threads = 256;
  if (src_dtype == dst_dtype) {
    const int esize = src_dtype == kF32 ? 4 : (src_dtype == kFP8 ? 1 : 2);
    const int row_bytes = a.head_dim * esize;
    const int unit = (row_bytes % 16 == 0) ? 16 : 8;
    const int units_log2 = log2_int(row_bytes / unit);
    const int64_t total = static_cast<int64_t>(a.num_tokens) * a.num_kv_heads * (row_bytes / unit);
    const dim3 grid(static_cast<unsigned>((total + threads - 1) / threads));
    if (unit == 16)
      hipLaunchKernelGGL((write_copy_kernel<16>), grid, dim3(threads), 0, s, a, units_log2);
    else
      hipLaunchKernelGGL((write_copy_kernel<8>), grid, dim3(threads), 0, s, a, units_log2);
    return hipGetLastError();
  }
  if (dst_dtype != kFP8) {
    if (supported) *supported = false;
    return hipSuccess;
  }
  const int e = src_dtype == kF32 ? 4 : 8;
  const int units_log2 = log2_int(a.head_dim / e);
  const int64_t total = static_cast<int64_t>(a.num_tokens) * a.num_kv_heads * (a.head_dim / e);
  const dim3 grid(static_cast<unsigned>((total + threads - 1) / threads));
  switch (src_dtype) {
    case kF32: hipLaunchKernelGGL((write_fp8_kernel<F32S>), grid, dim3(threads), 0, s, a, units_log2); break;
    case kF16: hipLaunchKernelGGL((write_fp8_kernel<F16S>), grid, dim3(threads), 0, s, a, units_log2); break;
    case kBF16: hipLaunchKernelGGL((write_fp8_kernel<BF16S>), grid, dim3(threads), 0, s, a, units_log2); break;
    default: if (supported) *supported = false; return hipSuccess;
  }
  return hipGetLastError();
}

hipError_t launch_copy(const CopyArgs &a, hipStream_t s) {
  const dim3 grid(a.num_pairs, 2, static_cast<unsigned>((a.block_bytes + 4095) / 4096));
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_zero(void *p, int64_t bytes, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  if (n16 <= 0) return hipSuccess;
  const int64_t blocks = (n16 + 255) / 256;
  hipLaunchKernelGGL(zero_kernel, dim3(static_cast<unsigned>(blocks < 1024 ? blocks : 1024)), dim3(256), 0, s,
                     static_cast<uint4 *>(p), n16);
  return hipGetLastError();
}

hipError_t launch_status(const int32_t *word, int32_t *out, hipStream_t s) {
  hipLaunchKernelGGL(status_kernel, dim3(1), dim3(64), 0, s, word, out);
  return hipGetLastError();
}

}  // namespace pa_impl
