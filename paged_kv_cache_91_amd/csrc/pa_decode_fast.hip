// Paged decode for head_dim 128 on gfx950: one wave per (partition, KV head
// group, sequence), q.K^T on the matrix cores, P.V on the vector ALUs, and
// the split-KV log-sum-exp merge done by the last partition to finish.
//
// What is computed is the decode attention of gufacode.com "PagedAttention:KV
// cache 的页表革命", section "PagedAttention CUDA Kernel" (per sequence: the
// blocks its table names, in logical order, then softmax(q K^T) V), with the
// explicit scale and exactly context_len positions; the gather is fused into
// the loads, as that section describes for the production kernel.  Query
// heads that share a KV head (ultralytics.com "PagedAttention", section
// "관련 기법", grouped-query attention) are handled together so every K/V
// byte is read once per head group.
//
// Work split.  A partition of P positions (or the whole context when the
// split is off) is walked in tiles of 16 positions; a tile never straddles a
// block (block size 16 or 32).  The wave keeps the next tile's loads and the
// table entry after that in flight while it computes the current tile.
//
// q.K^T as a 16x16x32 MFMA per 32 head dims: A = K tile (rows = the 16
// positions), B = the group's q vectors (columns = query heads, zero beyond
// the group), C[pos][head] in fp32.  The contraction only needs A and B to
// agree on which head dim sits in which (lane group, element) slot, so each
// lane loads 16 contiguous bytes of a K row.
//
// Online softmax per head in the base-2 domain (scores pre-multiplied by
// scale * log2 e).  Lane l holds the scores of positions 4*(l/16)+r, r < 4,
// for head l%16.
//
// P.V on the VALU: lane l reads the V row of position 4*(l/16)+c (c < 4),
// dims 8*(l%16)..+7, so every load instruction covers 4 whole rows; the
// probability of that position for head h is broadcast inside the 16-lane
// row from lane h (DPP row_newbcast).  The 4 row groups' partial sums are
// added at the end.
//
// Split merge.  Each partition writes m, l and the unnormalised output o for
// its heads, then bumps a per-(sequence, head group) counter; the partition
// that brings it to the partition count merges all partials in increasing
// partition order (M = max m_p, out = sum 2^(m_p-M) o_p / sum 2^(m_p-M) l_p)
// and resets the counter to zero for the next call.  The result does not
// depend on which partition finishes last.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "pa_common.h"
#include "pa_internal.h"

namespace pa_impl {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kHd = 128;      // head_dim handled here
constexpr int kTile = 16;     // positions per MFMA tile

template <typename QS> struct Mma;
template <> struct Mma<BF16S> {
  using V8 = bf16x8_t;
  static __device__ __forceinline__ f32x4_t run(V8 a, V8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // two e4m3 codes (low or high half of w) -> two bf16 values, exact
  template <bool HI>
  static __device__ __forceinline__ uint32_t from_fp8(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  }
};
template <> struct Mma<F16S> {
  using V8 = f16x8_t;
  static __device__ __forceinline__ f32x4_t run(V8 a, V8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  template <bool HI>
  static __device__ __forceinline__ uint32_t from_fp8(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
  }
};

// Broadcast lane H of each 16-lane row to the whole row (DPP row_newbcast).
template <int H>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + H,
                                                            0xf, 0xf, true));
}

// Combine each lane's value with the lane 16 (resp. 32) away, on the VALU
// (v_permlane16_swap / v_permlane32_swap), so no LDS traffic is involved.
// The swaps are written as inline assembly: given the same value twice, the
// compiler's model of the intrinsics treats both results as that value and
// drops the exchange.  The leading s_nop covers the VALU-write -> permlane
// read hazard on the operands.
__device__ __forceinline__ void swap16(uint32_t &a, uint32_t &b) {
  asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap32(uint32_t &a, uint32_t &b) {
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float xor16_max(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap16(a, b);
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float xor32_max(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap32(a, b);
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float xor16_sum(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap16(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}
__device__ __forceinline__ float xor32_sum(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap32(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// Device-coherent (agent scope) 32-bit store / load: written through to, and
// read back from, the level all XCDs share, so partials published by one
// workgroup are seen by another without flushing or invalidating any L2.
__device__ __forceinline__ void coherent_store(float *p, float x) {
  __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename QS, typename KS, int GT, int BS>
struct Fast {
  using M = Mma<QS>;
  using V8 = typename M::V8;
  static constexpr bool kFp8 = std::is_same<KS, FP8S>::value;
  static constexpr int kEsz = kFp8 ? 1 : 2;
  static constexpr int kRow = kHd * kEsz;              // bytes per K/V row
  static_assert(BS % kTile == 0, "block size must be a multiple of 16");

  // first head dim of chunk j's 8-element run for lane group g (A and B agree)
  static __device__ __forceinline__ int dbase(int j, int g) {
    return kFp8 ? 64 * (j >> 1) + 16 * g + 8 * (j & 1) : 32 * j + 8 * g;
  }

  using VRaw = typename std::conditional<kFp8, uint2, uint4>::type;
  struct Tile {
    uint4 k[kFp8 ? 2 : 4];        // MFMA A operand source
    VRaw v[4];
  };

  static __device__ __forceinline__ void issue(Tile &t, const uint8_t *__restrict__ kb,
                                               const uint8_t *__restrict__ vb, int64_t off_blk,
                                               int o0, int r16, int g4) {
    const uint8_t *kp = kb + off_blk + (o0 + r16) * kRow;
    if constexpr (kFp8) {
      t.k[0] = *reinterpret_cast<const uint4 *>(kp + 16 * g4);
      t.k[1] = *reinterpret_cast<const uint4 *>(kp + 64 + 16 * g4);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) t.k[j] = *reinterpret_cast<const uint4 *>(kp + (32 * j + 8 * g4) * 2);
    }
    const uint8_t *vp = vb + off_blk + (o0 + 4 * g4) * kRow + 8 * r16 * kEsz;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      t.v[c] = *reinterpret_cast<const VRaw *>(vp + c * kRow);
  }

  static __device__ __forceinline__ V8 a_operand(const Tile &t, int j) {
    if constexpr (kFp8) {
      const uint4 w = t.k[j >> 1];
      const uint32_t lo = (j & 1) ? w.z : w.x;
      const uint32_t hi = (j & 1) ? w.w : w.y;
      uint4 r;
      r.x = M::template from_fp8<false>(lo);
      r.y = M::template from_fp8<true>(lo);
      r.z = M::template from_fp8<false>(hi);
      r.w = M::template from_fp8<true>(hi);
      return __builtin_bit_cast(V8, r);
    } else {
      return __builtin_bit_cast(V8, t.k[j]);
    }
  }

  static __device__ __forceinline__ void widen_v(const Tile &t, int c, float *f) {
    if constexpr (kFp8) {
      Kv<FP8S>::widen(t.v[c], f);
    } else {
      Kv<KS>::widen(t.v[c], f);
    }
  }

  template <bool MASKED>
  static __device__ __forceinline__ void compute(const Tile &t, const V8 (&qb)[4], int tpos,
                                                 int pend, int r16, int g4, float scale_log2,
                                                 float &m_run, float &l_run, float (&acc)[GT][8]) {
    f32x4_t s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) s = M::run(a_operand(t, j), qb[j], s);
    const int p0 = tpos + 4 * g4;
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sc[r] = s[r] * scale_log2;
      if constexpr (MASKED) sc[r] = (p0 + r < pend) ? sc[r] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = xor32_max(xor16_max(mx));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(sc[r] - m_new);
    l_run = fmaf(l_run, alpha, (p[0] + p[1]) + (p[2] + p[3]));
    m_run = m_new;
    // rescale the accumulators only when some head's maximum moved
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        const float ah = bcast_head(alpha, h);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= ah;
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float vf[8];
      widen_v(t, c, vf);
      if constexpr (MASKED) {
        const bool ok = p0 + c < pend;
#pragma unroll
        for (int e = 0; e < 8; ++e) vf[e] = ok ? vf[e] : 0.0f;
      }
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        const float ph = bcast_head(p[c], h);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(ph, vf[e], acc[h][e]);
      }
    }
  }

  static __device__ __forceinline__ float bcast_head(float x, int h) {
    switch (h) {
      case 0: return row_bcast<0>(x);
      case 1: return row_bcast<1>(x);
      case 2: return row_bcast<2>(x);
      case 3: return row_bcast<3>(x);
      case 4: return row_bcast<4>(x);
      case 5: return row_bcast<5>(x);
      case 6: return row_bcast<6>(x);
      default: return row_bcast<7>(x);
    }
  }

  static __device__ __forceinline__ void store_row(const DecodeArgs &a, int64_t row, int r16,
                                                   const float (&o)[8], float mul) {
    if constexpr (std::is_same<QS, BF16S>::value) {
      uint4 w;
      w.x = f32_to_bf16(o[0] * mul) | (static_cast<uint32_t>(f32_to_bf16(o[1] * mul)) << 16);
      w.y = f32_to_bf16(o[2] * mul) | (static_cast<uint32_t>(f32_to_bf16(o[3] * mul)) << 16);
      w.z = f32_to_bf16(o[4] * mul) | (static_cast<uint32_t>(f32_to_bf16(o[5] * mul)) << 16);
      w.w = f32_to_bf16(o[6] * mul) | (static_cast<uint32_t>(f32_to_bf16(o[7] * mul)) << 16);
      *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(a.out) + row * kHd + 8 * r16) = w;
    } else {
      uint4 w;
      w.x = f32_to_f16(o[0] * mul) | (static_cast<uint32_t>(f32_to_f16(o[1] * mul)) << 16);
      w.y = f32_to_f16(o[2] * mul) | (static_cast<uint32_t>(f32_to_f16(o[3] * mul)) << 16);
      w.z = f32_to_f16(o[4] * mul) | (static_cast<uint32_t>(f32_to_f16(o[5] * mul)) << 16);
      w.w = f32_to_f16(o[6] * mul) | (static_cast<uint32_t>(f32_to_f16(o[7] * mul)) << 16);
      *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(a.out) + row * kHd + 8 * r16) = w;
    }
  }

  static __device__ void run(const DecodeArgs &a) {
    const int part = blockIdx.x;
    const int kvh = blockIdx.y / a.head_groups;
    const int hg = blockIdx.y - kvh * a.head_groups;
    const int seq = blockIdx.z;
    const int lane = threadIdx.x;
    const int r16 = lane & 15;
    const int g4 = lane >> 4;
    const int n = a.ctx[seq];
    const int hq0 = kvh * a.group + hg * GT;
    const int hcount = min(GT, a.group - hg * GT);
    const bool bad_len = n < 0 || n > a.max_blocks * BS;

    if (bad_len || n == 0) {           // NaN rows for a bad length, zero rows for an empty one
      if (part != 0) return;
      const float fill = bad_len ? __builtin_nanf("") : 0.0f;
      const float z[8] = {fill, fill, fill, fill, fill, fill, fill, fill};
      for (int h = g4; h < hcount; h += 4)
        store_row(a, static_cast<int64_t>(seq) * a.num_q_heads + hq0 + h, r16, z, 1.0f);
      return;
    }
    const int P = a.partition_size > 0 ? a.partition_size : n;
    const int nparts = (n + P - 1) / P;
    const int pstart = part * P;
    if (pstart >= n) return;
    const int pend = min(n, pstart + P);
    const int ntiles = (pend - pstart + kTile - 1) / kTile;

    // q of this head group as the MFMA B operand (zero columns beyond the group)
    V8 qb[4];
    {
      const uint16_t *qrow = static_cast<const uint16_t *>(a.q) +
                             (static_cast<int64_t>(seq) * a.num_q_heads + hq0 + r16) * kHd;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint4 w = make_uint4(0u, 0u, 0u, 0u);
        if (r16 < hcount) w = *reinterpret_cast<const uint4 *>(qrow + dbase(j, g4));
        qb[j] = __builtin_bit_cast(V8, w);
      }
    }

    const int64_t head_bytes = static_cast<int64_t>(BS) * kRow;
    const int64_t blk_bytes = head_bytes * a.num_kv_heads;
    const uint8_t *kb = static_cast<const uint8_t *>(a.k_pool) + kvh * head_bytes;
    const uint8_t *vb = static_cast<const uint8_t *>(a.v_pool) + kvh * head_bytes;
    const int32_t *trow = a.tables + static_cast<int64_t>(seq) * a.max_blocks;
    const int jmax = (pend - 1) / BS;
    bool bad = false;
    auto lookup = [&](int t) -> int64_t {
      const int j = min((pstart + t * kTile) / BS, jmax);
      int64_t ph = trow[j];
      if (static_cast<uint64_t>(ph) >= static_cast<uint64_t>(a.num_blocks)) {
        bad = true;
        ph = 0;
      }
      return ph * blk_bytes;
    };
    auto in_block = [&](int t) { return (pstart + t * kTile) % BS; };

    float m_run = -INFINITY, l_run = 0.0f;
    float acc[GT][8];
#pragma unroll
    for (int h = 0; h < GT; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;

    auto full = [&](const Tile &t, int ti) {
      compute<false>(t, qb, pstart + ti * kTile, pend, r16, g4, a.scale_log2, m_run, l_run, acc);
    };
    auto last_tile = [&](const Tile &t, int ti) {
      const int tpos = pstart + ti * kTile;
      if (tpos + kTile <= pend)
        compute<false>(t, qb, tpos, pend, r16, g4, a.scale_log2, m_run, l_run, acc);
      else
        compute<true>(t, qb, tpos, pend, r16, g4, a.scale_log2, m_run, l_run, acc);
    };

    // Two tile buffers: while one is computed the other's loads are in
    // flight; the table entry of the tile after that is fetched a tile ahead.
    // Every prefetch in the loop body is unconditional (the last one or two
    // tiles are peeled), so the wait counts stay exact.
    Tile A, B;
    int64_t offA = lookup(0);
    int64_t offB = lookup(1);
    issue(A, kb, vb, offA, in_block(0), r16, g4);
    int t = 0;
    for (; t + 2 < ntiles; t += 2) {
      issue(B, kb, vb, offB, in_block(t + 1), r16, g4);
      offA = lookup(t + 2);
      full(A, t);
      issue(A, kb, vb, offA, in_block(t + 2), r16, g4);
      offB = lookup(t + 3);
      full(B, t + 1);
    }
    if (t + 1 < ntiles) {
      issue(B, kb, vb, offB, in_block(t + 1), r16, g4);
      full(A, t);
      last_tile(B, t + 1);
    } else {
      last_tile(A, t);
    }

    // add the four row groups' partial sums
    l_run = xor32_sum(xor16_sum(l_run));
#pragma unroll
    for (int h = 0; h < GT; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = xor32_sum(xor16_sum(acc[h][e]));
    const bool any_bad = __builtin_amdgcn_ballot_w64(bad) != 0;
    const float nanv = __builtin_nanf("");

    if (nparts == 1) {
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        // l of head h sits in lane h (every row holds the same sums now)
        const float lh = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l_run), h));
        if (h < hcount && g4 == (h & 3))
          store_row(a, static_cast<int64_t>(seq) * a.num_q_heads + hq0 + h, r16, acc[h],
                    any_bad ? nanv : a.v_scale / lh);
      }
      return;
    }

    // split: publish this partition's partial with device-coherent stores,
    // wait until they are complete, then count the arrival
    const int64_t unit = static_cast<int64_t>(seq) * (a.num_kv_heads * a.head_groups) + blockIdx.y;
    float *po = a.part_o + (unit * a.max_parts + part) * (GT * kHd);
    float *pml = a.part_m + (unit * a.max_parts + part) * (GT * 2);
    const float mul = any_bad ? nanv : 1.0f;
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      if (g4 == (h & 3)) {
#pragma unroll
        for (int e = 0; e < 8; ++e) coherent_store(po + h * kHd + 8 * r16 + e, acc[h][e] * mul);
      }
    }
    if (g4 == 0 && r16 < GT) {
      coherent_store(pml + 2 * r16, any_bad ? nanv : m_run);
      coherent_store(pml + 2 * r16 + 1, any_bad ? nanv : l_run);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);          // vmcnt(0): the stores above have landed
    int last = 0;
    if (lane == 0)
      last = __hip_atomic_fetch_add(a.counters + unit, 1, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) == nparts - 1;
    last = __builtin_amdgcn_readlane(last, 0);
    if (!last) return;

    // merge every partition of this (sequence, head group) in partition order
    const float *bo = a.part_o + unit * a.max_parts * (GT * kHd);
    const float *bml = a.part_m + unit * a.max_parts * (GT * 2);
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      if (h >= hcount || g4 != (h & 3)) continue;
      float big_m = -INFINITY;
      for (int p = 0; p < nparts; ++p) big_m = fmaxf(big_m, coherent_load(bml + p * GT * 2 + 2 * h));
      float l = 0.0f, o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      bool nan_seen = false;
      for (int p = 0; p < nparts; ++p) {
        const float mp = coherent_load(bml + p * GT * 2 + 2 * h);
        nan_seen |= (mp != mp);
        const float f = __builtin_amdgcn_exp2f(mp - big_m);
        l = fmaf(coherent_load(bml + p * GT * 2 + 2 * h + 1), f, l);
        const float *src = bo + p * GT * kHd + h * kHd + 8 * r16;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = fmaf(coherent_load(src + e), f, o[e]);
      }
      store_row(a, static_cast<int64_t>(seq) * a.num_q_heads + hq0 + h, r16, o,
                nan_seen ? nanv : a.v_scale / l);
    }
    if (lane == 0) __hip_atomic_store(a.counters + unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
};

template <typename QS, typename KS, int GT, int BS>
__global__ __launch_bounds__(64) void decode_fast_kernel(DecodeArgs a) {
  Fast<QS, KS, GT, BS>::run(a);
}

template <typename QS, typename KS, int BS>
hipError_t launch_fast_bs(const DecodeArgs &a, hipStream_t s) {
  const dim3 grid(a.partition_size > 0 ? a.max_parts : 1, a.num_kv_heads * a.head_groups, a.num_seqs);
  switch (a.heads_per_wg) {
    case 1: hipLaunchKernelGGL((decode_fast_kernel<QS, KS, 1, BS>), grid, dim3(64), 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_fast_kernel<QS, KS, 2, BS>), grid, dim3(64), 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_fast_kernel<QS, KS, 4, BS>), grid, dim3(64), 0, s, a); break;
    case 8: hipLaunchKernelGGL((decode_fast_kernel<QS, KS, 8, BS>), grid, dim3(64), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename QS, typename KS>
hipError_t launch_fast_t(const DecodeArgs &a, hipStream_t s) {
  return a.block_size == 16 ? launch_fast_bs<QS, KS, 16>(a, s) : launch_fast_bs<QS, KS, 32>(a, s);
}

}  // namespace

bool fast_decode_applies(int q_dtype, int kv_dtype, const DecodeArgs &a) {
  if (a.head_dim != kHd || (a.block_size != 16 && a.block_size != 32)) return false;
  if (q_dtype != kBF16 && q_dtype != kF16) return false;
  return kv_dtype == q_dtype || kv_dtype == kFP8;
}

hipError_t launch_decode_fast(int q_dtype, int kv_dtype, const DecodeArgs &a, hipStream_t s) {
  if (q_dtype == kBF16 && kv_dtype == kBF16) return launch_fast_t<BF16S, BF16S>(a, s);
  if (q_dtype == kF16 && kv_dtype == kF16) return launch_fast_t<F16S, F16S>(a, s);
  if (q_dtype == kBF16 && kv_dtype == kFP8) return launch_fast_t<BF16S, FP8S>(a, s);
  if (q_dtype == kF16 && kv_dtype == kFP8) return launch_fast_t<F16S, FP8S>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace pa_impl
