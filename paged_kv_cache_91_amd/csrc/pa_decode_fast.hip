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
typedef float f32x2_t __attribute__((ext_vector_type(2)));

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

// Device-coherent (agent scope) stores and loads: written through to, and
// read back from, the level all XCDs share, so the partials one workgroup
// publishes are seen by another without flushing or invalidating any L2.
// The vector forms are inline assembly with the sc1 scope bit (what the
// compiler emits for agent-scope atomic accesses, which it only offers per
// 32-bit word and never batches).  Loads issued here are not tracked by the
// compiler's wait counting, so each batch ends with coherent_wait(), whose
// operands tie the loaded registers to the wait.
__device__ __forceinline__ void coherent_store(float *p, float x) {
  __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coherent_store4(float *p, f32x4_t v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ f32x4_t coherent_load4(const float *p) {
  f32x4_t r;
  asm volatile("global_load_dwordx4 %0, %1, off sc1" : "=&v"(r) : "v"(p) : "memory");
  return r;
}
__device__ __forceinline__ f32x2_t coherent_load2(const float *p) {
  f32x2_t r;
  asm volatile("global_load_dwordx2 %0, %1, off sc1" : "=&v"(r) : "v"(p) : "memory");
  return r;
}
template <typename T>
__device__ __forceinline__ void coherent_wait(T &x) {
  asm volatile("s_waitcnt vmcnt(0)" : "+v"(x) : : "memory");
}

// One segment's partial for one head: running max m, sum l, and this lane's
// 8 unnormalised output dims.
struct Partial {
  f32x2_t ml;
  f32x4_t o0, o1;
};

// Fold partials into (M, L, O) in order: the online form of
// M = max m_p, L = sum 2^(m_p - M) l_p, O = sum 2^(m_p - M) o_p.
__device__ __forceinline__ void fold(const Partial &x, float &big_m, float &l, float (&o)[8],
                                     bool &nan_seen) {
  const float m = x.ml[0];
  nan_seen |= (m != m);
  const float nm = fmaxf(big_m, m);
  const float c_old = __builtin_amdgcn_exp2f(big_m - nm);
  const float c_new = __builtin_amdgcn_exp2f(m - nm);
  l = l * c_old + x.ml[1] * c_new;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[e] = o[e] * c_old + x.o0[e] * c_new;
    o[4 + e] = o[4 + e] * c_old + x.o1[e] * c_new;
  }
  big_m = nm;
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// K/V bytes are read exactly once: non-temporal loads keep them from
// displacing reusable lines (tables, q, partials) in the caches.
__device__ __forceinline__ uint4 load_stream(const uint8_t *p, uint4) {
  const u32x4_t r = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(r[0], r[1], r[2], r[3]);
}
__device__ __forceinline__ uint2 load_stream(const uint8_t *p, uint2) {
  const u32x2_t r = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
  return make_uint2(r[0], r[1]);
}

// NW waves share one partition: wave w takes tiles w, w+NW, w+2NW, ...; the
// waves' softmax states are merged through LDS, so a partition costs one
// partial write and one arrival however many waves stream it.
template <typename QS, typename KS, int GT, int BS, int NW>
struct Fast {
  using M = Mma<QS>;
  using V8 = typename M::V8;
  static constexpr bool kFp8 = std::is_same<KS, FP8S>::value;
  static constexpr int kEsz = kFp8 ? 1 : 2;
  static constexpr int kRow = kHd * kEsz;              // bytes per K/V row
  static constexpr int kThreads = NW * 64;
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
      t.k[0] = load_stream(kp + 16 * g4, uint4{});
      t.k[1] = load_stream(kp + 64 + 16 * g4, uint4{});
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) t.k[j] = load_stream(kp + (32 * j + 8 * g4) * 2, uint4{});
    }
    const uint8_t *vp = vb + off_blk + (o0 + 4 * g4) * kRow + 8 * r16 * kEsz;
#pragma unroll
    for (int c = 0; c < 4; ++c) t.v[c] = load_stream(vp + c * kRow, VRaw{});
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

  // Accumulate `count` tiles of one (sequence, head group) into this wave's
  // online-softmax state: tile t_first + stride * i for i < count, each 16
  // positions starting at 16 * tile; positions >= pend are masked.
  static __device__ __forceinline__ void accumulate(
      const DecodeArgs &a, const V8 (&qb)[4], const uint8_t *__restrict__ kb,
      const uint8_t *__restrict__ vb, const int32_t *__restrict__ trow, int pend, int t_first,
      int count, int stride, int r16, int g4, float &m_run, float &l_run, float (&acc)[GT][8],
      bool &bad) {
    const int64_t blk_bytes = static_cast<int64_t>(BS) * kRow * a.num_kv_heads;
    const int jmax = (pend - 1) / BS;
    auto tpos = [&](int i) { return (t_first + stride * i) * kTile; };
    auto lookup = [&](int i) -> int64_t {
      const int j = min(tpos(i) / BS, jmax);
      int64_t ph = trow[j];
      if (static_cast<uint64_t>(ph) >= static_cast<uint64_t>(a.num_blocks)) {
        bad = true;
        ph = 0;
      }
      return ph * blk_bytes;
    };
    auto in_block = [&](int i) { return min(tpos(i), pend - 1) % BS / kTile * kTile; };

    m_run = -INFINITY;
    l_run = 0.0f;
#pragma unroll
    for (int h = 0; h < GT; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;
    if (count <= 0) return;

    auto full = [&](const Tile &t, int i) {
      compute<false>(t, qb, tpos(i), pend, r16, g4, a.scale_log2, m_run, l_run, acc);
    };
    auto last_tile = [&](const Tile &t, int i) {
      if (tpos(i) + kTile <= pend)
        compute<false>(t, qb, tpos(i), pend, r16, g4, a.scale_log2, m_run, l_run, acc);
      else
        compute<true>(t, qb, tpos(i), pend, r16, g4, a.scale_log2, m_run, l_run, acc);
    };

    // Two tile buffers: while one is computed the other's loads are in
    // flight, and the table entry after that is fetched one tile ahead.
    // Every prefetch in the loop body is unconditional (the last one or two
    // tiles are peeled), so the wait counts stay exact.
    Tile A, B;
    int64_t offA = lookup(0);
    int64_t offB = lookup(1);
    issue(A, kb, vb, offA, in_block(0), r16, g4);
    int i = 0;
    for (; i + 2 < count; i += 2) {
      issue(B, kb, vb, offB, in_block(i + 1), r16, g4);
      offA = lookup(i + 2);
      full(A, i);
      issue(A, kb, vb, offA, in_block(i + 2), r16, g4);
      offB = lookup(i + 3);
      full(B, i + 1);
    }
    if (i + 1 < count) {
      issue(B, kb, vb, offB, in_block(i + 1), r16, g4);
      last_tile(A, i);
      last_tile(B, i + 1);
    } else {
      last_tile(A, i);
    }
  }

  // q of one head group as the MFMA B operand (zero columns beyond the group)
  static __device__ __forceinline__ void load_q(const DecodeArgs &a, int64_t row0, int hcount,
                                                int r16, int g4, V8 (&qb)[4]) {
    const uint16_t *qrow = static_cast<const uint16_t *>(a.q) + (row0 + r16) * kHd;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (r16 < hcount) w = *reinterpret_cast<const uint4 *>(qrow + dbase(j, g4));
      qb[j] = __builtin_bit_cast(V8, w);
    }
  }

  // four consecutive outputs, rounded to the q dtype
  static __device__ __forceinline__ void store4(const DecodeArgs &a, int64_t idx, float4 o, float mul) {
    uint2 w;
    if constexpr (std::is_same<QS, BF16S>::value) {
      w.x = f32_to_bf16(o.x * mul) | (static_cast<uint32_t>(f32_to_bf16(o.y * mul)) << 16);
      w.y = f32_to_bf16(o.z * mul) | (static_cast<uint32_t>(f32_to_bf16(o.w * mul)) << 16);
    } else {
      w.x = f32_to_f16(o.x * mul) | (static_cast<uint32_t>(f32_to_f16(o.y * mul)) << 16);
      w.y = f32_to_f16(o.z * mul) | (static_cast<uint32_t>(f32_to_f16(o.w * mul)) << 16);
    }
    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + idx) = w;
  }

  static __device__ __forceinline__ float4 fma4(float4 x, float f, float4 acc) {
    return make_float4(fmaf(x.x, f, acc.x), fmaf(x.y, f, acc.y), fmaf(x.z, f, acc.z), fmaf(x.w, f, acc.w));
  }


  // -------------------------------------------------------------------------
  // Balanced (stream-K) decode.  The work of the whole batch is the list of
  // 16-position tiles of every (sequence, head group) unit, units ordered by
  // sequence then head group.  A grid of W single-wave workgroups, sized to
  // what the GPU holds at once, gives wave w the contiguous tile range
  // [floor(w T / W), floor((w+1) T / W)).  A unit inside one wave's range is
  // finished by that wave; a unit cut by range boundaries gets one partial
  // per wave that touches it (a wave writes at most two: its first and its
  // last unit), and the wave that brings the unit's arrival count to its
  // segment count merges the partials in wave order.
  // -------------------------------------------------------------------------

  static __device__ __forceinline__ int64_t range_lo(int64_t T, int64_t W, int64_t w) {
    return T * w / W;
  }
  // wave whose tile range holds global tile g
  static __device__ __forceinline__ int64_t wave_of(int64_t T, int64_t W, int64_t g) {
    int64_t w = g * W / T;
    while (w + 1 < W && range_lo(T, W, w + 1) <= g) ++w;
    while (w > 0 && range_lo(T, W, w) > g) --w;
    return w;
  }

  static __device__ void run_stream(const DecodeArgs &a) {
    const int64_t W = gridDim.x;
    const int64_t w = blockIdx.x;
    const int lane = threadIdx.x;
    const int r16 = lane & 15;
    const int g4 = lane >> 4;
    const int S = a.num_seqs;
    const int KVG = a.num_kv_heads * a.head_groups;
    const int maxn = a.max_blocks * BS;
    const float nanv = __builtin_nanf("");
    auto tiles_of = [&](int n) { return (n > 0 && n <= maxn) ? (n + kTile - 1) / kTile : 0; };

    // rows of empty (zero) and out-of-range (NaN) sequences
    for (int s = static_cast<int>(w); s < S; s += static_cast<int>(W)) {
      const int n = a.ctx[s];
      if (n > 0 && n <= maxn) continue;
      const float fill = n == 0 ? 0.0f : nanv;
      for (int i = lane; i < a.num_q_heads * (kHd / 4); i += 64)
        store4(a, (static_cast<int64_t>(s) * a.num_q_heads + (i >> 5)) * kHd + 4 * (i & 31),
               make_float4(fill, fill, fill, fill), 1.0f);
    }

    // total tiles, then the sequence holding this wave's first tile
    int64_t T = 0;
    for (int c0 = 0; c0 < S; c0 += 64) {
      int64_t cnt = (c0 + lane < S) ? tiles_of(a.ctx[c0 + lane]) : 0;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) cnt += __shfl_xor(cnt, o, 64);
      T += cnt;
    }
    T *= KVG;
    const int64_t lo = range_lo(T, W, w);
    const int64_t hi = range_lo(T, W, w + 1);
    if (lo >= hi) return;
    int s = 0;
    int64_t G = 0;                     // first global tile of sequence s
    {
      int64_t base = 0;
      for (int c0 = 0; c0 < S; c0 += 64) {
        const int64_t cnt = ((c0 + lane < S) ? tiles_of(a.ctx[c0 + lane]) : 0) * static_cast<int64_t>(KVG);
        int64_t incl = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int64_t up = __shfl_up(incl, o, 64);
          if (lane >= o) incl += up;
        }
        const int64_t total = __shfl(incl, 63, 64);
        if (base + total > lo) {
          const int first = __builtin_ctzll(__builtin_amdgcn_ballot_w64(base + incl > lo));
          s = c0 + first;
          G = base + __shfl(incl, first, 64) - __shfl(cnt, first, 64);
          break;
        }
        base += total;
      }
    }
    int nts = tiles_of(a.ctx[s]);
    int gidx = static_cast<int>((lo - G) / nts);
    int t = static_cast<int>((lo - G) % nts);

    for (int64_t g = lo; g < hi;) {
      const int seg = static_cast<int>(min(hi - g, static_cast<int64_t>(nts - t)));
      const int kvh = gidx / a.head_groups;
      const int hg = gidx - kvh * a.head_groups;
      const int hq0 = kvh * a.group + hg * GT;
      const int hcount = min(GT, a.group - hg * GT);
      const int64_t row0 = static_cast<int64_t>(s) * a.num_q_heads + hq0;
      const int n = a.ctx[s];

      V8 qb[4];
      load_q(a, row0, hcount, r16, g4, qb);
      const int64_t head_bytes = static_cast<int64_t>(BS) * kRow;
      const uint8_t *kb = static_cast<const uint8_t *>(a.k_pool) + kvh * head_bytes;
      const uint8_t *vb = static_cast<const uint8_t *>(a.v_pool) + kvh * head_bytes;
      const int32_t *trow = a.tables + static_cast<int64_t>(s) * a.max_blocks;
      bool bad = false;
      float m_run, l_run, acc[GT][8];
      accumulate(a, qb, kb, vb, trow, n, t, seg, 1, r16, g4, m_run, l_run, acc, bad);

      l_run = xor32_sum(xor16_sum(l_run));
#pragma unroll
      for (int h = 0; h < GT; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = xor32_sum(xor16_sum(acc[h][e]));
      const bool any_bad = __builtin_amdgcn_ballot_w64(bad) != 0;

      if (t == 0 && seg == nts) {
        // the whole unit is this wave's: write the output rows
#pragma unroll
        for (int h = 0; h < GT; ++h) {
          const float lh = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l_run), h));
          if (h < hcount && g4 == (h & 3)) {
            const float mul = any_bad ? nanv : a.v_scale / lh;
            const int64_t base_idx = (row0 + h) * kHd + 8 * r16;
            store4(a, base_idx, make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]), mul);
            store4(a, base_idx + 4, make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]), mul);
          }
        }
      } else {
        // a segment of a unit shared with neighbouring waves: publish a partial
        const int slot = g == lo ? 0 : 1;
        float *po = a.part_o + (w * 2 + slot) * (GT * kHd);
        float *pml = a.part_m + (w * 2 + slot) * (GT * 2);
        const float mul = any_bad ? nanv : 1.0f;
#pragma unroll
        for (int h = 0; h < GT; ++h) {
          if (g4 == (h & 3)) {
            float *dst = po + h * kHd + 8 * r16;
            coherent_store4(dst, f32x4_t{acc[h][0] * mul, acc[h][1] * mul, acc[h][2] * mul, acc[h][3] * mul});
            coherent_store4(dst + 4, f32x4_t{acc[h][4] * mul, acc[h][5] * mul, acc[h][6] * mul, acc[h][7] * mul});
          }
        }
        if (g4 == 0 && r16 < GT) {
          coherent_store(pml + 2 * r16, any_bad ? nanv : m_run);
          coherent_store(pml + 2 * r16 + 1, any_bad ? nanv : l_run);
        }
        __builtin_amdgcn_s_waitcnt(0x0f70);      // vmcnt(0): the stores above have landed
        const int64_t unit = static_cast<int64_t>(s) * KVG + gidx;
        const int64_t gu = G + static_cast<int64_t>(gidx) * nts;          // unit's first tile
        const int64_t wf = wave_of(T, W, gu);
        const int64_t wl = wave_of(T, W, gu + nts - 1);
        int last = 0;
        if (lane == 0)
          last = __hip_atomic_fetch_add(a.counters + unit, 1, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == static_cast<int>(wl - wf);
        last = __builtin_amdgcn_readlane(last, 0);
        if (last) {
          // merge the unit's segments in wave order; row g4 merges heads
          // g4, g4 + 4, ..., four segments' loads in flight at a time.
          // A segment's partial sits in the first slot of its wave unless
          // the wave's range began inside this unit's predecessor.
          const int64_t wsplit = wave_of(T, W, gu) + (range_lo(T, W, wave_of(T, W, gu)) < gu ? 1 : 0);
          for (int h = g4; h < hcount; h += 4) {
            float big_m = -INFINITY, l = 0.0f, o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            bool nan_seen = false;
            for (int64_t v0 = wf; v0 <= wl; v0 += 4) {
              Partial x[4];
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                const int64_t v = min(v0 + k, wl);
                const int64_t sl = v < wsplit ? 1 : 0;
                x[k].ml = coherent_load2(a.part_m + (v * 2 + sl) * (GT * 2) + 2 * h);
                const float *src = a.part_o + (v * 2 + sl) * (GT * kHd) + h * kHd + 8 * r16;
                x[k].o0 = coherent_load4(src);
                x[k].o1 = coherent_load4(src + 4);
              }
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                coherent_wait(x[k].ml);
                coherent_wait(x[k].o0);
                coherent_wait(x[k].o1);
              }
#pragma unroll
              for (int k = 0; k < 4; ++k)
                if (v0 + k <= wl) fold(x[k], big_m, l, o, nan_seen);
            }
            const float mul2 = nan_seen ? nanv : a.v_scale / l;
            const int64_t base_idx = (row0 + h) * kHd + 8 * r16;
            store4(a, base_idx, make_float4(o[0], o[1], o[2], o[3]), mul2);
            store4(a, base_idx + 4, make_float4(o[4], o[5], o[6], o[7]), mul2);
          }
          if (lane == 0)
            __hip_atomic_store(a.counters + unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }

      // next unit
      g += seg;
      t = 0;
      if (++gidx == KVG) {
        gidx = 0;
        G += static_cast<int64_t>(nts) * KVG;
        if (g < hi) {
          do {
            ++s;
            nts = tiles_of(a.ctx[s]);
          } while (nts == 0);
        }
      }
    }
  }

  static __device__ void run(const DecodeArgs &a) {
    __shared__ float s_ml[NW][GT][2];
    __shared__ float4 s_acc[NW][GT][kHd / 4];
    __shared__ int s_last;

    const int part = blockIdx.x;
    const int kvh = blockIdx.y / a.head_groups;
    const int hg = blockIdx.y - kvh * a.head_groups;
    const int seq = blockIdx.z;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);    // uniform: keeps tile math scalar
    const int lane = tid & 63;
    const int r16 = lane & 15;
    const int g4 = lane >> 4;
    const int n = a.ctx[seq];
    const int hq0 = kvh * a.group + hg * GT;
    const int hcount = min(GT, a.group - hg * GT);
    const int64_t row0 = static_cast<int64_t>(seq) * a.num_q_heads + hq0;
    const bool bad_len = n < 0 || n > a.max_blocks * BS;

    if (bad_len || n == 0) {           // NaN rows for a bad length, zero rows for an empty one
      if (part != 0) return;
      const float fill = bad_len ? __builtin_nanf("") : 0.0f;
      for (int i = tid; i < hcount * (kHd / 4); i += kThreads)
        store4(a, (row0 + (i >> 5)) * kHd + 4 * (i & 31), make_float4(fill, fill, fill, fill), 1.0f);
      return;
    }
    const int P = a.partition_size > 0 ? a.partition_size : n;
    const int nparts = (n + P - 1) / P;
    const int pstart = part * P;
    if (pstart >= n) return;
    const int pend = min(n, pstart + P);
    const int ntiles = (pend - pstart + kTile - 1) / kTile;
    const int nloc = ntiles > wave ? (ntiles - wave + NW - 1) / NW : 0;   // this wave's tiles

    V8 qb[4];
    load_q(a, row0, hcount, r16, g4, qb);

    const int64_t head_bytes = static_cast<int64_t>(BS) * kRow;
    const uint8_t *kb = static_cast<const uint8_t *>(a.k_pool) + kvh * head_bytes;
    const uint8_t *vb = static_cast<const uint8_t *>(a.v_pool) + kvh * head_bytes;
    const int32_t *trow = a.tables + static_cast<int64_t>(seq) * a.max_blocks;
    bool bad = false;
    float m_run, l_run, acc[GT][8];
    accumulate(a, qb, kb, vb, trow, pend, pstart / kTile + wave, nloc, NW, r16, g4, m_run, l_run, acc,
               bad);

    // add the four row groups' partial sums, then hand the wave's state to LDS
    l_run = xor32_sum(xor16_sum(l_run));
#pragma unroll
    for (int h = 0; h < GT; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = xor32_sum(xor16_sum(acc[h][e]));
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      if (g4 == (h & 3)) {
        s_acc[wave][h][2 * r16] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
        s_acc[wave][h][2 * r16 + 1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
      }
    }
    if (g4 == 0 && r16 < GT) {
      s_ml[wave][r16][0] = m_run;
      s_ml[wave][r16][1] = l_run;
    }
    const bool any_bad = __syncthreads_or(bad);
    const float nanv = __builtin_nanf("");

    // merge the waves (fixed wave order): M, L and the unnormalised output
    auto wave_merge = [&](int h, int d4, float &big_m, float &l, float4 &o) {
      big_m = s_ml[0][h][0];
#pragma unroll
      for (int w = 1; w < NW; ++w) big_m = fmaxf(big_m, s_ml[w][h][0]);
      l = 0.0f;
      o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = __builtin_amdgcn_exp2f(s_ml[w][h][0] - big_m);
        l = fmaf(s_ml[w][h][1], f, l);
        o = fma4(s_acc[w][h][d4], f, o);
      }
    };

    if (nparts == 1) {
      for (int i = tid; i < hcount * (kHd / 4); i += kThreads) {
        const int h = i >> 5, d4 = i & 31;
        float big_m, l;
        float4 o;
        wave_merge(h, d4, big_m, l, o);
        store4(a, (row0 + h) * kHd + 4 * d4, o, any_bad ? nanv : a.v_scale / l);
      }
      return;
    }

    // split: publish this partition's partial with device-coherent stores,
    // wait until they are complete, then count the arrival
    const int64_t unit = static_cast<int64_t>(seq) * (a.num_kv_heads * a.head_groups) + blockIdx.y;
    float *po = a.part_o + (unit * a.max_parts + part) * (GT * kHd);
    float *pml = a.part_m + (unit * a.max_parts + part) * (GT * 2);
    for (int i = tid; i < GT * (kHd / 4); i += kThreads) {
      const int h = i >> 5, d4 = i & 31;
      float big_m, l;
      float4 o;
      wave_merge(h, d4, big_m, l, o);
      const float mul = any_bad ? nanv : 1.0f;
      coherent_store4(po + h * kHd + 4 * d4, f32x4_t{o.x * mul, o.y * mul, o.z * mul, o.w * mul});
      if (d4 == 0) {
        coherent_store(pml + 2 * h, any_bad ? nanv : big_m);
        coherent_store(pml + 2 * h + 1, any_bad ? nanv : l);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);          // vmcnt(0): this thread's stores have landed
    __syncthreads();                             // ... and every other thread's
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(a.counters + unit, 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) == nparts - 1;
    __syncthreads();
    if (!s_last) return;

    // merge every partition of this (sequence, head group) in partition
    // order, four partitions' loads in flight at a time
    const float *bo = a.part_o + unit * a.max_parts * (GT * kHd);
    const float *bml = a.part_m + unit * a.max_parts * (GT * 2);
    for (int i = tid; i < hcount * (kHd / 4); i += kThreads) {
      const int h = i >> 5, d4 = i & 31;
      float big_m = -INFINITY, l = 0.0f, o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      bool nan_seen = false;
      for (int p0 = 0; p0 < nparts; p0 += 4) {
        Partial x[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int pp = min(p0 + k, nparts - 1);
          x[k].ml = coherent_load2(bml + pp * GT * 2 + 2 * h);
          x[k].o0 = coherent_load4(bo + pp * GT * kHd + h * kHd + 4 * d4);
          x[k].o1 = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          coherent_wait(x[k].ml);
          coherent_wait(x[k].o0);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (p0 + k < nparts) fold(x[k], big_m, l, o, nan_seen);
      }
      store4(a, (row0 + h) * kHd + 4 * d4, make_float4(o[0], o[1], o[2], o[3]),
             nan_seen ? nanv : a.v_scale / l);
    }
    if (tid == 0) __hip_atomic_store(a.counters + unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
};

constexpr int kFastWaves = 4;

template <typename QS, typename KS, int GT, int BS>
__global__ __launch_bounds__(kFastWaves * 64) void decode_fast_kernel(DecodeArgs a) {
  Fast<QS, KS, GT, BS, kFastWaves>::run(a);
}

template <typename QS, typename KS, int GT, int BS>
__global__ __launch_bounds__(64) void decode_stream_kernel(DecodeArgs a) {
  Fast<QS, KS, GT, BS, 1>::run_stream(a);
}

// Grid of the balanced split: as many single-wave workgroups as the GPU
// keeps resident (occupancy of this kernel x compute units), capped by the
// workspace capacity the caller sized for.
template <typename QS, typename KS, int GT, int BS>
hipError_t launch_stream_gt(const DecodeArgs &a, hipStream_t s) {
  static const int per_cu = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_stream_kernel<QS, KS, GT, BS>, 64, 0) !=
            hipSuccess || n <= 0)
      n = 8;
    return n;
  }();
  const int waves = min(a.stream_waves, device_compute_units() * per_cu);
  hipLaunchKernelGGL((decode_stream_kernel<QS, KS, GT, BS>), dim3(waves), dim3(64), 0, s, a);
  return hipGetLastError();
}

template <typename QS, typename KS, int BS>
hipError_t launch_fast_bs(const DecodeArgs &a, hipStream_t s) {
  if (a.stream_waves > 0) {
    switch (a.heads_per_wg) {
      case 1: return launch_stream_gt<QS, KS, 1, BS>(a, s);
      case 2: return launch_stream_gt<QS, KS, 2, BS>(a, s);
      case 4: return launch_stream_gt<QS, KS, 4, BS>(a, s);
      case 8: return launch_stream_gt<QS, KS, 8, BS>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
  const dim3 grid(a.partition_size > 0 ? a.max_parts : 1, a.num_kv_heads * a.head_groups, a.num_seqs);
  const dim3 block(kFastWaves * 64);
  switch (a.heads_per_wg) {
    case 1: hipLaunchKernelGGL((decode_fast_kernel<QS, KS, 1, BS>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_fast_kernel<QS, KS, 2, BS>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_fast_kernel<QS, KS, 4, BS>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((decode_fast_kernel<QS, KS, 8, BS>), grid, block, 0, s, a); break;
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
