// Paged decode for head_dim 128 on gfx950: q.K^T and P.V on the matrix
// cores, the online softmax on the vector ALUs, and the split-KV log-sum-exp
// merge done by the last piece of a context to finish.
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
// P.V as eight 16x16x16 MFMAs per tile, one per e < 8: A = V restricted to
// the dims 8*i+e (rows i < 16) over the tile's 16 positions, B = P (positions
// x query heads), C[i][head] accumulating O[head][8*i+e] in fp32.  Lane l
// reads the V rows of positions 4*(l/16)+c (c < 4), dims 8*(l%16)..+7, so
// every load instruction covers 4 whole rows and the lane already holds its
// A slots (4 positions of one dim) up to a 16-bit shuffle (v_perm); its B
// slots (4 positions of head l%16) are exactly the probabilities the q.K^T
// MFMA left in it, rounded to the MFMA's input type.  C lands with head l%16
// and dims 32*(l/16)..+31 in lane l, so each lane's rescale factor is its own
// head's and the outputs need no cross-lane sum.
//
// Split merge.  Each partition writes m, l and the unnormalised output o for
// its heads, then bumps a per-(sequence, head group) counter; the partition
// that brings it to the partition count merges all partials in increasing
// partition order (M = max m_p, out = sum 2^(m_p-M) o_p / sum 2^(m_p-M) l_p)
// and resets the counter to zero for the next call.  The result does not
// depend on which partition finishes last.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "pa_common.h"
#include "pa_internal.h"
#include "pa_mfma.h"

namespace pa_impl {
namespace {

constexpr int kHd = 128;      // head_dim handled here
constexpr int kTile = 16;     // positions per MFMA tile

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
// the same 8-byte store at a uniform base (SGPRs) plus a per-lane byte
// offset: one offset register per lane instead of a 64-bit address
__device__ __forceinline__ void coherent_store2_at(const void *base, uint32_t off, uint2 v) {
  asm volatile("global_store_dwordx2 %0, %1, %2 sc1" : : "v"(off), "v"(v), "s"(base) : "memory");
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

// The same device-coherent accesses as buffer instructions with the sc1
// cache-policy bit, which the compiler sees and counts, so it places the
// waits itself.  `r` is a resource over a whole float array, `off` a byte
// offset into it (accesses past the array read zeros and write nothing).
constexpr int kSc1 = 16;                 // cache policy bits: device-coherent scope
__device__ __forceinline__ __amdgpu_buffer_rsrc_t float_rsrc(const float *base, int64_t count) {
  const int64_t bytes = count * 4;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), 0,
                                           static_cast<int>(bytes < 0x7fffffff ? bytes : 0x7fffffff),
                                           0x00020000);
}
__device__ __forceinline__ void rsrc_store4(__amdgpu_buffer_rsrc_t r, int off, f32x4_t v) {
  typedef uint32_t w4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(w4, v), r, off, 0, kSc1);
}
__device__ __forceinline__ void rsrc_store2(__amdgpu_buffer_rsrc_t r, int off, f32x2_t v) {
  typedef uint32_t w2 __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(w2, v), r, off, 0, kSc1);
}
__device__ __forceinline__ f32x4_t rsrc_load4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSc1));
}
__device__ __forceinline__ f32x2_t rsrc_load2(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kSc1));
}

// Mailbox flags shared by the waves of a workgroup: volatile LDS accesses
// (the explicit address space keeps them ds_read / ds_write; a generic
// volatile access would be a flat access, counted with the K/V loads).
typedef __attribute__((address_space(3))) volatile int lds_vint_t;
__device__ __forceinline__ int lds_get(int *p) { return *(lds_vint_t *)(p); }
__device__ __forceinline__ void lds_put(int *p, int v) { *(lds_vint_t *)(p) = v; }

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
// fold() for four dims
__device__ __forceinline__ void fold4(f32x2_t ml, f32x4_t x, float &big_m, float &l, float (&o)[4],
                                      bool &nan_seen) {
  const float m = ml[0];
  nan_seen |= (m != m);
  const float nm = fmaxf(big_m, m);
  const float c_old = __builtin_amdgcn_exp2f(big_m - nm);
  const float c_new = __builtin_amdgcn_exp2f(m - nm);
  l = l * c_old + ml[1] * c_new;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = o[e] * c_old + x[e] * c_new;
  big_m = nm;
}
// lane groups of 32 in the split's merge (up to 8 per workgroup)
constexpr int kMergeGroups = 8;



// K/V tiles are read with buffer loads: a tile is one (block, KV head)
// range of 16 rows given as a buffer resource, so a load can be switched off
// by giving the resource zero size (the instruction still issues and counts,
// it reads nothing and returns zeros).  That keeps every step of the
// prefetch ring unconditional, which the compiler's wait counting needs to
// keep loads in flight across steps.  The loads are non-temporal: K/V bytes
// are read exactly once and should not displace reusable lines.
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit elements (gfx9 family)
constexpr int kLoadNt = 2;               // cache policy bits: non-temporal

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), 0, bytes, kRsrcWord3);
}
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t r, int off, uint4 &x) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kLoadNt);
  x = make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t r, int off, uint2 &x) {
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kLoadNt);
  x = make_uint2(v[0], v[1]);
}

// Block-table entries and context lengths are read through the constant
// address space: they are not written while the kernel runs, and such loads
// become scalar loads, whose completion is counted apart from the K/V loads
// (a vector load of a table entry would wait behind the tile loads issued
// before it).
typedef const __attribute__((address_space(4))) int32_t cint32_t;
__device__ __forceinline__ int load_const(const int32_t *p, int64_t i) {
  return ((cint32_t *)p)[i];
}

// NW waves share one partition: wave w takes tiles w, w+NW, w+2NW, ...; the
// waves' softmax states are merged through LDS, so a partition costs one
// partial write however many waves stream it.
// WIN: the balanced split with a sliding window (per-sequence first tile);
// without it the window fields fold to zero.
template <typename QS, typename KS, int GT, int BS, int NW, bool WIN = false>
struct Fast {
  using M = Mma<QS>;
  using V8 = typename M::V8;
  static constexpr bool kFp8 = std::is_same<KS, FP8S>::value;
  static constexpr int kEsz = kFp8 ? 1 : 2;
  static constexpr int kRow = kHd * kEsz;              // bytes per K/V row
  static constexpr int kThreads = NW * 64;
  static_assert(BS % kTile == 0, "block size must be a multiple of 16");
  // K/V tiles in flight per wave (an fp8 tile carries half the bytes)
  static constexpr int kRing = kFp8 ? 4 : 2;
  // the ring of accumulate(): the split's one-wave workgroups run three
  // waves per SIMD, so each keeps one fp8 tile less in flight (the 16
  // registers it frees make room for the third wave)
  static constexpr int kAccRing = (NW == 1 && kFp8) ? 3 : kRing;
  static constexpr int kKxBytes = kFp8 ? kTile * kRow : 16;     // LDS of k_relayout per wave
  // how far (log2 units) a tile's maximum may pass the running maximum
  // before the accumulators are rescaled
  static constexpr float kLazy = 8.0f;

  // first head dim of chunk j's 8-element run for lane group g (A and B agree)
  static __device__ __forceinline__ int dbase(int j, int g) {
    return kFp8 ? 64 * (j >> 1) + 16 * g + 8 * (j & 1) : 32 * j + 8 * g;
  }

  using VRaw = typename std::conditional<kFp8, uint2, uint4>::type;
  struct Tile {
    uint4 k[kFp8 ? 2 : 4];        // MFMA A operand source
    VRaw v[4];
  };

  // Issue the loads of the tile whose 16 rows start at byte `off` of the K
  // and V pools (uniform), or loads that read nothing when !on.  ko / vo are
  // this lane's byte offsets inside a tile (lane_offsets()).
  template <bool KW>
  static __device__ __forceinline__ void issue(Tile &t, const uint8_t *__restrict__ kb,
                                               const uint8_t *__restrict__ vb, int64_t off, bool on,
                                               int ko, int vo) {
    const int bytes = on ? kTile * kRow : 0;
    const auto rk = tile_rsrc(kb + off, bytes);
    const auto rv = tile_rsrc(vb + off, bytes);
#pragma unroll
    for (int j = 0; j < (kFp8 ? 2 : 4); ++j) load_tile(rk, ko + (KW ? 1024 : 64) * j, t.k[j]);
#pragma unroll
    for (int c = 0; c < 4; ++c) load_tile(rv, vo + c * kRow, t.v[c]);
  }
  // K: lane (r16, g4) reads row r16, 16 bytes at 16*g4 of every 64-byte
  // chunk (the MFMA A slots, matching dbase).  An fp8 row is one 128-byte
  // line, which that layout fetches in two halves; with KW (whole rows, fp8
  // only) lane l reads bytes 16 l of each kilobyte instead (load j: rows
  // 8j .. 8j + 7 whole) and k_relayout moves the chunks into the A slots.
  // V: rows 4*g4 .. 4*g4+3, the 8 elements from 8*r16.
  template <bool KW>
  static __device__ __forceinline__ int k_lane_offset(int r16, int g4) {
    static_assert(!KW || kFp8, "whole-row K loads are for fp8 rows");
    return KW ? 16 * (r16 + 16 * g4) : r16 * kRow + 16 * g4;
  }

  // fp8 K from whole-row loads to the MFMA layout, through the wave's own
  // 2 KiB of LDS (`kx`): lane (r16, g4) gets the 16-byte chunks g4 and g4 + 4
  // of row r16 (dims 16 g4 .. + 15 and 64 + 16 g4 .. + 15, as dbase reads
  // them).  Chunk c of row r sits at chunk c ^ ((r >> 1) & 7) of the row's
  // 128 bytes, so the 16 rows read by one quarter of the wave fall on
  // distinct banks.  A wave's LDS operations complete in order, so the slot
  // is reused by the next tile without a wait.
  static __device__ __forceinline__ void k_relayout(const Tile &t, uint8_t *kx, int lane, uint4 (&kk)[2]) {
    auto at = [&](int row, int c) { return reinterpret_cast<uint4 *>(kx + row * 128 + 16 * (c ^ ((row >> 1) & 7))); };
#pragma unroll
    for (int j = 0; j < 2; ++j) *at(8 * j + (lane >> 3), lane & 7) = t.k[j];
    const int r16 = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) kk[h] = *at(r16, g4 + 4 * h);
  }
  static __device__ __forceinline__ int v_lane_offset(int r16, int g4) {
    return 4 * g4 * kRow + 8 * r16 * kEsz;
  }

  static __device__ __forceinline__ V8 a_operand(const uint4 (&kk)[kFp8 ? 2 : 4], int j) {
    if constexpr (kFp8) {
      const uint4 w = kk[j >> 1];
      const uint32_t lo = (j & 1) ? w.z : w.x;
      const uint32_t hi = (j & 1) ? w.w : w.y;
      uint4 r;
      r.x = M::template from_fp8<false>(lo);
      r.y = M::template from_fp8<true>(lo);
      r.z = M::template from_fp8<false>(hi);
      r.w = M::template from_fp8<true>(hi);
      return __builtin_bit_cast(V8, r);
    } else {
      return __builtin_bit_cast(V8, kk[j]);
    }
  }

  // P.V for one tile: acc[e] += V(dims 8*i+e) x P, e < 8 (see the layout
  // notes at the top).  v_perm builds the A operand from the lane's rows:
  // selector 0x05040100 takes the low 16 bits of two dwords, 0x07060302 the
  // high 16 bits.  fp8 rows are first transposed bytewise (four rows' codes
  // of one dim into one dword) and then widened exactly to the MFMA type.
  static __device__ __forceinline__ void pv(const Tile &t, const uint32_t pb_lo, const uint32_t pb_hi,
                                            f32x4_t (&acc)[8]) {
    using V4 = typename M::V4;
    const V4 pb = __builtin_bit_cast(V4, make_uint2(pb_lo, pb_hi));
    auto mma = [&](int e, uint32_t a01, uint32_t a23) {
      acc[e] = M::run16(__builtin_bit_cast(V4, make_uint2(a01, a23)), pb, acc[e]);
    };
    if constexpr (kFp8) {
      uint32_t x[4][2];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        x[c][0] = t.v[c].x;
        x[c][1] = t.v[c].y;
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t t01l = __builtin_amdgcn_perm(x[1][k], x[0][k], 0x05010400u);
        const uint32_t t01h = __builtin_amdgcn_perm(x[1][k], x[0][k], 0x07030602u);
        const uint32_t t23l = __builtin_amdgcn_perm(x[3][k], x[2][k], 0x05010400u);
        const uint32_t t23h = __builtin_amdgcn_perm(x[3][k], x[2][k], 0x07030602u);
        const uint32_t y[4] = {__builtin_amdgcn_perm(t23l, t01l, 0x05040100u),
                               __builtin_amdgcn_perm(t23l, t01l, 0x07060302u),
                               __builtin_amdgcn_perm(t23h, t01h, 0x05040100u),
                               __builtin_amdgcn_perm(t23h, t01h, 0x07060302u)};
#pragma unroll
        for (int b = 0; b < 4; ++b)
          mma(4 * k + b, M::template from_fp8<false>(y[b]), M::template from_fp8<true>(y[b]));
      }
    } else {
      uint32_t x[4][4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        x[c][0] = t.v[c].x;
        x[c][1] = t.v[c].y;
        x[c][2] = t.v[c].z;
        x[c][3] = t.v[c].w;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        mma(2 * k, __builtin_amdgcn_perm(x[1][k], x[0][k], 0x05040100u),
            __builtin_amdgcn_perm(x[3][k], x[2][k], 0x05040100u));
        mma(2 * k + 1, __builtin_amdgcn_perm(x[1][k], x[0][k], 0x07060302u),
            __builtin_amdgcn_perm(x[3][k], x[2][k], 0x07060302u));
      }
    }
  }

  // One tile: q.K^T, the online softmax, P.V.  `masked` (uniform): some of
  // the tile's rows lie outside [pbeg, pend) (past the context end, or
  // before a sliding window's first position); their scores become -inf and
  // their V rows, whose bytes may hold NaN or Inf, are zeroed in place
  // before the product.  Only inputs change under the branch, so the
  // accumulators keep one set of registers (a masked and an unmasked copy
  // of the whole tile made the compiler move them between two sets on
  // every tile).
  template <bool KW>
  static __device__ __forceinline__ void compute(Tile &t, const V8 (&qb)[4], int tpos, int pbeg, int pend,
                                                 bool masked, int g4, float scale_log2,
                                                 float &m_run, float &l_run, f32x4_t (&acc)[8],
                                                 uint8_t *kx, int lane) {
    const int p0 = tpos + 4 * g4;
    auto keep = [&](int c) { return p0 + c < pend && p0 + c >= pbeg; };
    if (masked) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bool k = keep(c);
        t.v[c].x = k ? t.v[c].x : 0u;
        t.v[c].y = k ? t.v[c].y : 0u;
        if constexpr (!kFp8) {
          t.v[c].z = k ? t.v[c].z : 0u;
          t.v[c].w = k ? t.v[c].w : 0u;
        }
      }
    }
    uint4 kk[kFp8 ? 2 : 4];
    if constexpr (KW) {
      k_relayout(t, kx, lane, kk);
    } else {
#pragma unroll
      for (int j = 0; j < (kFp8 ? 2 : 4); ++j) kk[j] = t.k[j];
    }
    f32x4_t s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) s = M::run(a_operand(kk, j), qb[j], s);
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = s[r] * scale_log2;
    if (masked) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[r] = keep(r) ? sc[r] : -INFINITY;
    }
    float mx = max2(max2(sc[0], sc[1]), max2(sc[2], sc[3]));
    mx = xor32_max(xor16_max(mx));
    // Lazy running maximum: the exponentials are taken against m_run, which
    // moves (rescaling l and the accumulators of this lane's head) only when
    // some head's tile maximum passes it by more than kLazy.  Any reference
    // value gives the same softmax (the shift cancels between O and l); one
    // that trails the true maximum by at most kLazy keeps p <= 2^kLazy.
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazy) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= alpha;
      m_run = m_new;
    }
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(sc[r] - m_run);
    l_run += (p[0] + p[1]) + (p[2] + p[3]);
    pv(t, M::pack2(p[0], p[1]), M::pack2(p[2], p[3]), acc);
  }

  // Accumulate `count` tiles of one (sequence, head group) into this wave's
  // online-softmax state: tile t_first + stride * i for i < count, each 16
  // positions starting at 16 * tile; positions outside [pbeg, pend) are
  // masked.
  //
  // The tiles stream through a ring of kAccRing buffers: the loads of tile
  // i + kAccRing are issued as soon as tile i has been computed, so kAccRing
  // tiles are in flight while one is computed.  Every step issues loads
  // (switched off past the last tile), and a scheduling barrier keeps each
  // buffer's new loads after the compute that frees it, so the buffers stay
  // in place and the waits stay exact.  Table entries are fetched one step
  // ahead with scalar loads.
  static __device__ __forceinline__ void accumulate(
      const DecodeArgs &a, const V8 (&qb)[4], const uint8_t *__restrict__ kb,
      const uint8_t *__restrict__ vb, const int32_t *__restrict__ trow, int pbeg, int pend, int t_first,
      int count, int stride, int r16, int g4, float &m_run, float &l_run, f32x4_t (&acc)[8],
      bool &bad, uint8_t *kx) {
    const int lane = r16 + 16 * g4;
    const int64_t blk_bytes = static_cast<int64_t>(BS) * kRow * a.num_kv_heads;
    const int jmax = (pend - 1) / BS;
    // fp8: whole-row K loads (measured faster here; the balanced split's
    // stream keeps the half-row layout, which measured faster there)
    constexpr bool KW = kFp8;
    const int ko = k_lane_offset<KW>(r16, g4), vo = v_lane_offset(r16, g4);
    auto tpos = [&](int i) { return (t_first + stride * i) * kTile; };
    // raw table entry for tile i (clamped to the last block, so always readable)
    auto entry = [&](int i) { return load_const(trow, min(tpos(i) / BS, jmax)); };
    // issue tile i from table entry e (nothing when i >= count or e is bad)
    auto issue_tile = [&](Tile &t, int i, int e) {
      const bool valid = static_cast<uint32_t>(e) < static_cast<uint32_t>(a.num_blocks);
      const bool live = i < count;
      bad |= live && !valid;
      const int64_t off = (valid ? static_cast<int64_t>(e) * blk_bytes : 0) + tpos(i) % BS * kRow;
      issue<KW>(t, kb, vb, off, live && valid, ko, vo);
    };

    m_run = -INFINITY;
    l_run = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    if (count <= 0) return;

    Tile ring[kAccRing];
#pragma unroll
    for (int k = 0; k < kAccRing; ++k) issue_tile(ring[k], k, entry(k));
    int e_next = entry(kAccRing);
    for (int i0 = 0; i0 < count; i0 += kAccRing) {
#pragma unroll
      for (int k = 0; k < kAccRing; ++k) {
        const int i = i0 + k;
        if (i < count) {
          const bool masked = !(tpos(i) + kTile <= pend && tpos(i) >= pbeg);
          compute<KW>(ring[k], qb, tpos(i), pbeg, pend, masked, g4, a.scale_log2, m_run, l_run, acc, kx, lane);
        }
        __builtin_amdgcn_sched_barrier(0);
        const int e = e_next;
        e_next = entry(i + kAccRing + 1);
        issue_tile(ring[k], i + kAccRing, e);
        __builtin_amdgcn_sched_barrier(0);
      }
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

  // four outputs rounded to the q dtype, packed in two dwords
  static __device__ __forceinline__ uint2 pack4(float4 o) {
    uint2 w;
    if constexpr (std::is_same<QS, BF16S>::value) {
      w.x = f32_to_bf16(o.x) | (static_cast<uint32_t>(f32_to_bf16(o.y)) << 16);
      w.y = f32_to_bf16(o.z) | (static_cast<uint32_t>(f32_to_bf16(o.w)) << 16);
    } else {
      w.x = f32_to_f16(o.x) | (static_cast<uint32_t>(f32_to_f16(o.y)) << 16);
      w.y = f32_to_f16(o.z) | (static_cast<uint32_t>(f32_to_f16(o.w)) << 16);
    }
    return w;
  }
  // pack4's inverse: four values of the q dtype (two dwords) as floats
  static __device__ __forceinline__ f32x4_t unpack4(uint2 w) {
    if constexpr (std::is_same<QS, BF16S>::value) {
      return f32x4_t{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                     __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
    } else {
      const auto h = [](uint32_t b) { return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b))); };
      return f32x4_t{h(w.x & 0xffffu), h(w.x >> 16), h(w.y & 0xffffu), h(w.y >> 16)};
    }
  }
  // four consecutive outputs, scaled by mul and rounded to the q dtype
  static __device__ __forceinline__ void store4(const DecodeArgs &a, int64_t idx, float4 o, float mul) {
    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + idx) =
        pack4(make_float4(o.x * mul, o.y * mul, o.z * mul, o.w * mul));
  }

  // this lane's 32 output dims (32*g4 .. +31 of head r16), scaled by mul:
  // dims 32*g4 + 8*r + e sit in acc[e][r]
  static __device__ __forceinline__ void store_lane(const DecodeArgs &a, int64_t idx,
                                                    const f32x4_t (&acc)[8], float mul) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      store4(a, idx + 8 * r, make_float4(acc[0][r], acc[1][r], acc[2][r], acc[3][r]), mul);
      store4(a, idx + 8 * r + 4, make_float4(acc[4][r], acc[5][r], acc[6][r], acc[7][r]), mul);
    }
  }

  // store_lane's values into an LDS row (dims 32*g4 .. +31 at dst)
  static __device__ __forceinline__ void stage_lane(uint16_t *dst, const f32x4_t (&acc)[8], float mul) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float4 lo4 = make_float4(acc[0][r] * mul, acc[1][r] * mul, acc[2][r] * mul, acc[3][r] * mul);
      const float4 hi4 = make_float4(acc[4][r] * mul, acc[5][r] * mul, acc[6][r] * mul, acc[7][r] * mul);
      *reinterpret_cast<uint2 *>(dst + 8 * r) = pack4(lo4);
      *reinterpret_cast<uint2 *>(dst + 8 * r + 4) = pack4(hi4);
    }
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

  // Position in the batch's tile list: sequence s (n positions, nts tiles
  // per unit, first global tile G), unit u (KV head * head groups + head
  // group) and tile t of the unit.  With a sliding window the unit's tiles
  // start at tile t0 of the sequence (lo, the window's first position, lies
  // in it); otherwise t0 = lo = 0.
  struct Cursor {
    int s, n, nts, u, t, t0, lo;
    int64_t G;
  };
  static __device__ __forceinline__ int tiles_of(int n, int maxn, int window) {
    if constexpr (!WIN) return (n > 0 && n <= maxn) ? (n + kTile - 1) / kTile : 0;
    return (n > 0 && n <= maxn) ? (n + kTile - 1) / kTile - window_lo(n, window) / kTile : 0;
  }
  static __device__ __forceinline__ void set_seq(Cursor &c, int n, int maxn, int window) {
    c.n = n;
    c.nts = tiles_of(n, maxn, window);
    if constexpr (WIN) {
      c.lo = (n > 0 && n <= maxn) ? window_lo(n, window) : 0;
      c.t0 = c.lo / kTile;
    } else {
      c.lo = 0;
      c.t0 = 0;
    }
  }
  // next tile in list order (past the last one the cursor parks on s = S);
  // n_lane holds the first 64 sequences' lengths, one per lane
  static __device__ __forceinline__ void advance(const DecodeArgs &a, Cursor &c, int KVG, int maxn,
                                                 int n_lane) {
    if (++c.t < c.nts) return;
    c.t = 0;
    if (++c.u < KVG) return;
    c.u = 0;
    c.G += static_cast<int64_t>(c.nts) * KVG;
    for (;;) {
      if (++c.s >= a.num_seqs) {
        c.n = 0;
        c.nts = 1;
        c.t0 = c.lo = 0;
        return;
      }
      set_seq(c, c.s < 64 ? __builtin_amdgcn_readlane(n_lane, c.s) : load_const(a.ctx, c.s), maxn, a.window);
      if (c.nts > 0) return;
    }
  }

  // q staging: 16-byte pieces, piece p = chunk p%16 of head p/16 of the unit
  static constexpr int kQSlots = 4;
  static constexpr int kQPieces = (GT * 16 + 63) / 64;
  static __device__ __forceinline__ uint4 q_piece(const DecodeArgs &a, int s, int u, int p) {
    const int kvh = u / a.head_groups;
    const int hg = u - kvh * a.head_groups;
    const int h = p >> 4;
    if (p >= GT * 16 || h >= min(GT, a.group - hg * GT)) return make_uint4(0u, 0u, 0u, 0u);
    const int64_t row = static_cast<int64_t>(s) * a.num_q_heads + kvh * a.group + hg * GT + h;
    return *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) + row * kHd + (p & 15) * 8);
  }
  // the staged q as the MFMA B operand (zero columns beyond the group)
  static __device__ __forceinline__ void q_from_lds(const uint4 *slot, int hcount, int r16, int g4,
                                                    V8 (&qb)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (r16 < hcount) w = slot[r16 * 16 + dbase(j, g4) / 8];
      qb[j] = __builtin_bit_cast(V8, w);
    }
  }

  // floor(a / b) for 0 <= a < 2^53 and 0 < b < 2^31.  Operands below 2^32
  // take the 32-bit integer division; larger ones the double quotient, which
  // is within one of the exact one, corrected by one integer check on each
  // side (a 64-bit integer division is a long instruction sequence here)
  static __device__ __forceinline__ int64_t floor_div(int64_t a, int64_t b) {
    if (((static_cast<uint64_t>(a) | static_cast<uint64_t>(b)) >> 32) == 0)
      return static_cast<uint32_t>(a) / static_cast<uint32_t>(b);
    int64_t q = static_cast<int64_t>(static_cast<double>(a) / static_cast<double>(b));
    if (q * b > a)
      --q;
    else if ((q + 1) * b <= a)
      ++q;
    return q;
  }
  // first tile of part x when T tiles are cut into W near-equal parts
  // (T * W < 2^53, i.e. fewer than 2^40 tiles)
  static __device__ __forceinline__ int64_t range_lo(int64_t T, int64_t W, int64_t x) {
    return floor_div(T * x, W);
  }
  // the part holding tile g (0 <= g < T): the last x with range_lo(x) <= g,
  // i.e. floor(((g+1) W - 1) / T); parts may be empty when T < W
  static __device__ __forceinline__ int64_t part_of(int64_t T, int64_t W, int64_t g) {
    g = min(max(g, static_cast<int64_t>(0)), T - 1);
    return min(floor_div((g + 1) * W - 1, T), W - 1);
  }

  // -------------------------------------------------------------------------
  // Balanced split: XCD shares, static ranges, paired waves.
  //
  // Work.  The batch's work is the list of 16-position tiles of every
  // (sequence, head group) unit, units ordered by sequence then head group,
  // T tiles in all.  It is cut into one contiguous share per XCD, and share x
  // into 4 * n(x) near-equal ranges, one per streaming wave, where n(x) is
  // the number of workgroups the dispatcher places on XCD x (it deals
  // workgroups to the XCDs in turn, so n(x) = ceil((grid - x) / XCDs)).  A
  // workgroup reads its XCD from the hardware and takes the next index on
  // that XCD's registration counter; its four streamers take the ranges
  // 4 * index .. 4 * index + 3 of the share.  Range boundaries depend on T
  // and the grid only, so a split unit's partials and their merge order do
  // not depend on timing: the output is bit-identical from run to run.
  //
  // Waves.  A workgroup of 8 waves holds 4 streaming waves (0..3, one per
  // SIMD) and 4 helper waves (helper i + 4 shares streamer i's SIMD and
  // serves it).  A streamer issues only K/V, q and table loads: a global
  // store issued between the K/V loads would hold up the counting of every
  // load issued after it until it is acknowledged.  Each finished segment (a
  // whole unit's outputs, or a range's partial for a unit split between
  // ranges) goes to the helper through an LDS mailbox; the helper writes the
  // rows, publishes the partials, counts them in and merges the split units
  // while its streamer keeps streaming.  The range's last segment is taken
  // by whichever of the pair gets to it first (a compare-and-swap on the
  // entry): usually the streamer, once its stream is over, since the helper
  // may still be merging the segment before.
  //
  // Exchange.  The partials of a unit inside one share are written and
  // merged by waves of one XCD, so they go through that XCD's L2 with
  // ordinary stores and loads (a device-coherent store is written through
  // to memory and slows every wave's K/V loads down; a device-scope acquire
  // would drop the XCD's L2 lines the merge is about to read).  The loads
  // may hit the merging compute unit's L1, which is safe because a slot's
  // lines are loaded only after the slot is counted in, once per launch,
  // and no two slots share a line.  A unit that crosses a share boundary
  // (at most one per boundary) uses device-coherent stores and loads.  The
  // counters are device-scope atomics either way.
  //
  // Check.  If the dispatcher placed the workgroups otherwise, some XCD
  // gets more than n(x) of them, and a workgroup that draws an index >= n(x)
  // knows it at once: it marks the workspace (a poison word) and writes NaN
  // into every output row, so rows of ranges nobody streamed are NaN rather
  // than stale.  A marked workspace makes every later call write NaN rows
  // (its counters can no longer be trusted) until it is zero-filled again.
  // When every XCD's last index n(x) - 1 has been drawn, the registrations
  // are complete and exact; the last of those workgroups resets the
  // registration counters, early in the launch and off its critical path.
  // -------------------------------------------------------------------------

  // workgroups the dispatcher places on XCD x, and share x's tiles and ranges
  static __device__ __forceinline__ int64_t wgs_on(int64_t x, int NX) {
    return (gridDim.x - static_cast<uint32_t>(x) + static_cast<uint32_t>(NX) - 1) / static_cast<uint32_t>(NX);
  }
  struct Share {
    int64_t X0, X1, nr;   // tiles [X0, X1) in nr ranges
  };
  static __device__ __forceinline__ Share share_geom(int64_t T, int NX, int64_t x) {
    return Share{range_lo(T, NX, x), range_lo(T, NX, x + 1), 4 * wgs_on(x, NX)};
  }
  static __device__ __forceinline__ void range_of(const Share &sh, int64_t i, int64_t &lo, int64_t &hi) {
    const int64_t L = sh.X1 - sh.X0;
    lo = sh.X0 + range_lo(L, sh.nr, i);
    hi = sh.X0 + range_lo(L, sh.nr, i + 1);
  }

  // One finished segment in the mailbox: unnormalised outputs o (head h,
  // dims 4*d4 .. +3 at o[h * 32 + d4]), per head (m, l), and where it belongs.
  static constexpr int kMail = 4;
  struct Mail {
    f32x4_t o[GT * (kHd / 4)];
    f32x2_t ml[GT];
    int64_t unit, gu, row0;
    int nts, hcount, split, side;
    int taken;                     // claimed for handling (by the helper, or by the streamer for its last entry)
  };
  struct Box {
    Mail m[kMail];
    int head, tail, done, pad;     // posted (streamer), taken (helper); streamer finished
  };

  // The unit a range ends inside, when the range cuts it, worked out while
  // the range streams: its holder count and partial slots (tile order), so
  // that the merge at the range's end, the one on the kernel's critical
  // path, needs no table walk and issues all its loads at once.
  static constexpr int kPre = 8;
  struct Pre {
    bool on, cross;
    int64_t unit, count;
    int64_t slot[kPre];
  };

  // total tiles T of the batch; n_lane / cnt0 / incl0: the first 64
  // sequences' lengths, tile counts and inclusive running sums, one per lane
  // context lengths below which 64 sequences' tile counts fit 32 bits
  static constexpr int kScan32 = 1 << 28;
  static __device__ __forceinline__ int64_t count_tiles(const DecodeArgs &a, int lane, int &n_lane,
                                                        int64_t &cnt0, int64_t &incl0) {
    const int S = a.num_seqs;
    const int KVG = a.num_kv_heads * a.head_groups;
    const int maxn = a.max_blocks * BS;
    n_lane = lane < S ? a.ctx[lane] : 0;
    cnt0 = tiles_of(n_lane, maxn, a.window);
    int64_t T;
    if (maxn < kScan32) {
      // 64 sequences' tiles fit 32 bits: a DPP scan
      incl0 = wave_incl_sum(static_cast<uint32_t>(cnt0));
      T = lane_value(incl0, 63);
      for (int c0 = 64; c0 < S; c0 += 64) {
        const uint32_t cnt = (c0 + lane < S) ? static_cast<uint32_t>(tiles_of(a.ctx[c0 + lane], maxn, a.window)) : 0u;
        T += __builtin_amdgcn_readlane(wave_incl_sum(cnt), 63);
      }
    } else {
      incl0 = cnt0;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int64_t up = __shfl_up(incl0, o, 64);
        if (lane >= o) incl0 += up;
      }
      T = lane_value(incl0, 63);
      for (int c0 = 64; c0 < S; c0 += 64) {
        int64_t cnt = (c0 + lane < S) ? tiles_of(a.ctx[c0 + lane], maxn, a.window) : 0;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) cnt += __shfl_xor(cnt, o, 64);
        T += cnt;
      }
    }
    return uniform(T * KVG);
  }

  // the list position of global tile g (0 <= g < T)
  static __device__ Cursor locate(const DecodeArgs &a, int64_t g, int lane, int n_lane, int64_t cnt0,
                                  int64_t incl0) {
    const int S = a.num_seqs;
    const int KVG = a.num_kv_heads * a.head_groups;
    const int maxn = a.max_blocks * BS;
    int s = 0, n0 = 0;
    int64_t G = 0;                     // first global tile of sequence s
    const int64_t total0 = lane_value(incl0, 63) * KVG;
    if (total0 > g) {
      const int first = uniform(static_cast<int>(__builtin_ctzll(__builtin_amdgcn_ballot_w64(incl0 * KVG > g))));
      s = first;
      G = (lane_value(incl0, first) - lane_value(cnt0, first)) * KVG;
      n0 = __builtin_amdgcn_readlane(n_lane, first);
    } else {
      int64_t base = total0;
      for (int c0 = 64; c0 < S; c0 += 64) {
        const int64_t t = (c0 + lane < S) ? tiles_of(a.ctx[c0 + lane], maxn, a.window) : 0;
        int64_t incl;
        if (maxn < kScan32) {
          incl = wave_incl_sum(static_cast<uint32_t>(t));
        } else {
          incl = t;
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const int64_t up = __shfl_up(incl, o, 64);
            if (lane >= o) incl += up;
          }
        }
        const int64_t cnt = t * KVG;
        incl *= KVG;
        const int64_t total = lane_value(incl, 63);
        if (base + total > g) {
          const int first = uniform(static_cast<int>(__builtin_ctzll(__builtin_amdgcn_ballot_w64(base + incl > g))));
          s = c0 + first;
          G = base + lane_value(incl, first) - lane_value(cnt, first);
          n0 = load_const(a.ctx, s);
          break;
        }
        base += total;
      }
    }
    Cursor c;
    c.s = s;
    set_seq(c, n0, maxn, a.window);
    c.u = static_cast<int>(floor_div(g - G, c.nts));
    c.t = static_cast<int>(g - G - static_cast<int64_t>(c.u) * c.nts);
    c.G = G;
    return c;
  }

  // Workspace control words, one 128-byte line each: the count of XCDs
  // whose registrations are complete at ctl[0], XCD x's registration count
  // at ctl[32 * (1 + x)] (x < 16), the poison word at ctl[32 * 17]; the unit
  // counters at a.counters + 32 * unit (one 128-byte line each, 64-bit).
  static __device__ __forceinline__ int *reg_ctr(const DecodeArgs &a, int64_t x) { return a.ctl + 32 * (x + 1); }
  static __device__ __forceinline__ int *poison_word(const DecodeArgs &a) { return a.ctl + 32 * 17; }
  // values of the poison word (the status pa_decode_status reads back)
  static constexpr int kWsMisplaced = 1;   // the grid was not dealt to the XCDs in turn
  static constexpr int kWsTimedOut = 2;    // a wait between waves of a workgroup ran out

  // NaN into output rows first, first + step, ... of the batch
  static __device__ void nan_rows(const DecodeArgs &a, int64_t first, int64_t step, int lane) {
    const float nanv = __builtin_nanf("");
    const int64_t rows = static_cast<int64_t>(a.num_seqs) * a.num_q_heads;
    for (int64_t r = first; r < rows; r += step)
      for (int i = lane; i < kHd / 4; i += 64) store4(a, r * kHd + 4 * i, make_float4(nanv, nanv, nanv, nanv), 1.0f);
  }
  static __device__ __forceinline__ uint64_t *unit_ctr(const DecodeArgs &a, int64_t unit) {
    return reinterpret_cast<uint64_t *>(a.counters) + 16 * unit;
  }

  // Waits between the waves of one workgroup (all resident together, so
  // each wait ends as soon as the other wave gets there) are bounded all the
  // same: after a.wait_polls polls without the condition, the wave gives up.
  // `ready` reads LDS words other waves write; the result is made uniform.
  template <typename F>
  static __device__ __forceinline__ bool wait_lds(F ready, int polls) {
    for (int i = 0;; ++i) {
      if (uniform(static_cast<int>(ready())) != 0) return true;
      if (i >= polls) return false;
      __builtin_amdgcn_s_sleep(1);
    }
  }
  // A wave whose wait ran out (a protocol fault): it marks the workspace
  // (read back through pa_decode_status; later calls write NaN rows until the
  // workspace is zero-filled, since its counters can no longer be trusted)
  // and writes NaN into every output row, so that no row this launch owed is
  // left stale; then it exits like every other wave.
  static __device__ void abandon(const DecodeArgs &a, int lane) {
    if (lane == 0) __hip_atomic_store(poison_word(a), kWsTimedOut, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    nan_rows(a, 0, 1, lane);
  }

  static __device__ void run_pair(const DecodeArgs &a) {
    __shared__ Box box[4];
    __shared__ uint4 s_q[4][kQSlots][GT * 16];
    __shared__ int s_reg, s_poison, s_tbl, s_preok;
    __shared__ Pre s_pre[4];
    // dynamic LDS: the table of range starts (the helpers' lookups)
    extern __shared__ int64_t pa_dyn_lds[];
    const int wave = uniform(static_cast<int>(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    const int slot = wave & 3;
    const bool helper = wave >= 4;
    Box &bx = box[slot];
    // this workgroup's XCD selects its share (the exchange of a share's
    // partials relies on all its waves sharing one L2)
    const int NX = a.num_xcd;
    const int64_t x = static_cast<int64_t>(__builtin_amdgcn_s_getreg((3 << 11) | 20) & 15) % NX;
    // the first helper registers and reads the poison word while every wave
    // loads the lengths (the two waits overlap)
    int reg_got = 0, poison_got = 0;
    if (threadIdx.x == 256) {
      reg_got = __hip_atomic_fetch_add(reg_ctr(a, x), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      poison_got = __hip_atomic_load(poison_word(a), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    int n_lane;
    int64_t cnt0, incl0;
    const int64_t T = count_tiles(a, lane, n_lane, cnt0, incl0);
    if (threadIdx.x == 256) {
      s_reg = reg_got;
      s_poison = poison_got;
      s_tbl = 0;
      s_preok = 0;
    }
    if (lane == 0) {
      if (helper) {
        bx.tail = 0;
      } else {
        bx.head = 0;
        bx.done = 0;
      }
    }
    __syncthreads();
    // values read back from LDS are per-lane to the compiler: everything the
    // tile loop's addresses and trip counts derive from is made uniform, so
    // that the cursor stays in scalar registers and table entries and lengths
    // remain scalar loads (a vector load there would wait for every tile
    // load in flight)
    const int64_t reg = uniform(static_cast<int64_t>(s_reg));
    const int64_t n_x = wgs_on(x, NX);
    if (reg >= n_x || uniform(s_poison) != 0) {
      // a misplaced grid (this workgroup is surplus on its XCD) or a marked
      // workspace: NaN rows (all of them from the surplus workgroup, a
      // strided share from each workgroup of a marked one), nothing else
      if (helper) {
        if (reg >= n_x && wave == 4 && lane == 0)
          __hip_atomic_store(poison_word(a), kWsMisplaced, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (reg >= n_x)
          nan_rows(a, wave - 4, 4, lane);
        else
          nan_rows(a, (wave - 4) * static_cast<int64_t>(gridDim.x) + blockIdx.x, 4 * static_cast<int64_t>(gridDim.x),
                   lane);
      }
      return;
    }
    if (wave == 4 && reg == n_x - 1) {
      // the last registration on this XCD; the last XCD to complete resets
      // the counters (every workgroup of the grid has registered by then)
      const int xcds = min(NX, static_cast<int>(gridDim.x));
      int done = 0;
      if (lane == 0) done = __hip_atomic_fetch_add(a.ctl, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (uniform(done) == xcds - 1) {
        if (lane < NX) __hip_atomic_store(reg_ctr(a, lane), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (lane == 0) __hip_atomic_store(a.ctl, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    const Share sh = share_geom(T, NX, x);
    const int64_t NR = 4 * static_cast<int64_t>(gridDim.x);
    int64_t *rs = pa_dyn_lds;
    int *rc = reinterpret_cast<int *>(pa_dyn_lds + NR + 1);
    if (!helper) {
      int64_t lo, hi;
      range_of(sh, 4 * reg + slot, lo, hi);
      const bool streamed = lo >= hi || stream(a, bx, s_q[slot], lo, hi, lane, n_lane, cnt0, incl0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      if (lane == 0) lds_put(&bx.done, 1);
      if (!streamed) {
        abandon(a, lane);
        return;
      }
      // the range's last segment, unless the helper already took it: the
      // helper may still be merging the segment before, and this is the
      // merge on the launch's critical path
      const int last = lds_get(&bx.head) - 1;
      if (last >= 0) {
        int won = 0;
        if (lane == 0) {
          int expect = 0;
          won = __hip_atomic_compare_exchange_strong(&bx.m[last % kMail].taken, &expect, 1, __ATOMIC_RELAXED,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        if (uniform(won) != 0) {
          if (!wait_lds([&] { return lds_get(&s_tbl) >= 4 && lds_get(&s_preok) >= 4; }, a.wait_polls)) {
            abandon(a, lane);
            return;
          }
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          Pre pre = s_pre[slot];
          handle(a, T, x * (a.share_ranges) + 4 * reg + slot, bx.m[last % kMail], lane, rs, rc, pre, true);
        }
      }
      return;
    }
    // The helpers fill the table of range starts: rs[r] for the batch's
    // ranges in tile order (r < NR, share by share), rs[NR] = T, and for
    // each range its share y and index i in the share, as (y << 20) | i.
    {
      const int64_t q = static_cast<int64_t>(gridDim.x) / NX, rr = static_cast<int64_t>(gridDim.x) - q * NX;
      for (int64_t r = (wave - 4) * 64 + lane; r <= NR; r += 256) {
        if (r == NR) {
          rs[r] = T;
          continue;
        }
        int64_t y = 0, cum = 0;
        while (cum + 4 * (q + (y < rr ? 1 : 0)) <= r) cum += 4 * (q + (y++ < rr ? 1 : 0));
        const int64_t i = r - cum;
        const Share sy = share_geom(T, NX, y);
        int64_t lo, hi;
        range_of(sy, i, lo, hi);
        rs[r] = lo;
        rc[r] = static_cast<int>((y << 20) | i);
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      if (lane == 0) __hip_atomic_fetch_add(&s_tbl, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      // the four helpers have filled it
      if (!wait_lds([&] { return lds_get(&s_tbl) >= 4; }, a.wait_polls)) {
        abandon(a, lane);
        return;
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
    int64_t lo, hi;
    range_of(sh, 4 * reg + slot, lo, hi);
    helper_main(a, bx, T, x * (a.share_ranges) + 4 * reg + slot, lo, hi, lane, n_lane, cnt0, incl0, rs, rc,
                s_pre[slot], s_preok);
  }

  // The streamer's tile range [lo, hi) of the T-tile list.  Finished
  // segments go to the mailbox `bx`; `sq` stages q of the range's first
  // kQSlots units.  False if the wait for a free mailbox entry ran out.
  static __device__ bool stream(const DecodeArgs &a, Box &bx, uint4 (*sq)[GT * 16], int64_t lo, int64_t hi,
                                int lane, int n_lane, int64_t cnt0, int64_t incl0) {
    const int r16 = lane & 15;
    const int g4 = lane >> 4;
    const int KVG = a.num_kv_heads * a.head_groups;
    const int maxn = a.max_blocks * BS;
    const float nanv = __builtin_nanf("");
    lo = uniform(lo);
    hi = uniform(hi);
    const Cursor c0 = locate(a, lo, lane, n_lane, cnt0, incl0);

    // Set-up order: the first table entry, the q loads, then the first
    // kRing tiles' loads, and only then the q stores to LDS (whose wait for
    // the q loads leaves the tile loads in flight).
    const int ko = k_lane_offset<false>(r16, g4), vo = v_lane_offset(r16, g4);
    const int64_t head_bytes = static_cast<int64_t>(BS) * kRow;
    const int64_t blk_bytes = head_bytes * a.num_kv_heads;
    const uint8_t *kpool = static_cast<const uint8_t *>(a.k_pool);
    const uint8_t *vpool = static_cast<const uint8_t *>(a.v_pool);
    auto entry_at = [&](const Cursor &c) {
      return load_const(a.tables + static_cast<int64_t>(c.s) * a.max_blocks, (c.t0 + c.t) * kTile / BS);
    };
    Cursor ci = c0;                    // issue cursor
    int64_t gi = lo;
    int e_next = entry_at(ci);         // table entry of the tile at ci, fetched one issue ahead
    uint32_t slot_bad = 0;             // bit k: ring slot k's table entry was out of range

    // q of the range's first kQSlots units, staged in LDS, so that starting
    // a unit mid-stream never waits on a global load (that wait would also
    // wait for every K/V load issued before it)
    uint4 qv[kQSlots][kQPieces];
    int nq = 0;
    {
      Cursor cu = c0;
      int64_t gq = lo;
#pragma unroll
      for (int k = 0; k < kQSlots; ++k) {
        if (gq < hi) {
          nq = k + 1;
#pragma unroll
          for (int i = 0; i < kQPieces; ++i) qv[k][i] = q_piece(a, cu.s, cu.u, lane + 64 * i);
          gq += cu.nts - cu.t;
          cu.t = cu.nts - 1;
          advance(a, cu, KVG, maxn, n_lane);
        }
      }
    }

    // One pipeline over the whole range: the issue cursor runs kRing tiles
    // ahead of the compute cursor and crosses unit boundaries freely, so
    // the K/V stream never drains between units.
    auto issue_next = [&](Tile &tile, int k) {
      int64_t off = 0;
      bool on = false;
      if (gi < hi) {
        const int e = e_next;
        const bool valid = static_cast<uint32_t>(e) < static_cast<uint32_t>(a.num_blocks);
        slot_bad = valid ? (slot_bad & ~(1u << k)) : (slot_bad | (1u << k));
        off = static_cast<int64_t>(valid ? e : 0) * blk_bytes + (ci.u / a.head_groups) * head_bytes +
              ((ci.t0 + ci.t) * kTile) % BS * kRow;
        on = valid;
        advance(a, ci, KVG, maxn, n_lane);
        if (gi + 1 < hi) e_next = entry_at(ci);
      }
      ++gi;
      issue<false>(tile, kpool, vpool, off, on, ko, vo);
    };

    Tile ring[kRing];
#pragma unroll
    for (int k = 0; k < kRing; ++k) issue_next(ring[k], k);

#pragma unroll
    for (int k = 0; k < kQSlots; ++k)
      if (k < nq)
#pragma unroll
        for (int i = 0; i < kQPieces; ++i)
          if (lane + 64 * i < GT * 16) sq[k][lane + 64 * i] = qv[k][i];

    Cursor cc = c0;                    // compute cursor
    int64_t gc = lo;
    int nseg = 0;                      // segments started (q slot index)
    int64_t seg_g0 = lo;
    int hcount = 0;
    int64_t row0 = 0;
    float m_run = -INFINITY, l_run = 0.0f;
    f32x4_t acc[8];
    V8 qb[4];
    bool bad = false;
    int head = 0, tail_seen = 0;       // mailbox entries posted / known to be free
    bool gave_up = false;              // the wait for a free entry ran out: post nothing more

    for (int64_t g0 = lo; g0 < hi; g0 += kRing) {
#pragma unroll
      for (int k = 0; k < kRing; ++k) {
        if (gc < hi) {
          if (gc == lo || cc.t == 0) {
            // a segment (the part of a unit inside the range) starts
            seg_g0 = gc;
            const int kvh = cc.u / a.head_groups;
            const int hg = cc.u - kvh * a.head_groups;
            hcount = min(GT, a.group - hg * GT);
            row0 = static_cast<int64_t>(cc.s) * a.num_q_heads + kvh * a.group + hg * GT;
            if (nseg < kQSlots) {
              q_from_lds(sq[nseg], hcount, r16, g4, qb);
            } else {
              // past the staged units (very short contexts): a direct load,
              // waited for here so no pending load leaks into the stream
              load_q(a, row0, hcount, r16, g4, qb);
              __builtin_amdgcn_s_waitcnt(0x0f70);    // vmcnt(0)
            }
            ++nseg;
            m_run = -INFINITY;
            l_run = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            bad = false;
          }
          const int tp = (cc.t0 + cc.t) * kTile;
          const bool masked = !(tp + kTile <= cc.n && tp >= cc.lo);
          compute<false>(ring[k], qb, tp, cc.lo, cc.n, masked, g4, a.scale_log2, m_run, l_run, acc, nullptr, lane);
          bad |= ((slot_bad >> k) & 1u) != 0;

          if (gc == hi - 1 || cc.t == cc.nts - 1) {
            // the segment ends: a whole unit's outputs or this range's
            // partial for a split unit, handed to the helper
            const float l = xor32_sum(xor16_sum(l_run));
            if (head - tail_seen >= kMail && !gave_up) {
              for (int polls = 0;; ++polls) {
                tail_seen = uniform(lds_get(&bx.tail));
                if (head - tail_seen < kMail) break;
                if (polls >= a.wait_polls) {
                  gave_up = true;
                  break;
                }
                __builtin_amdgcn_s_sleep(1);
              }
              __atomic_signal_fence(__ATOMIC_SEQ_CST);
            }
            if (!gave_up) {
            Mail &e = bx.m[head % kMail];
            const float mul = bad ? nanv : 1.0f;
            if (r16 < GT) {
              f32x4_t *dst = &e.o[r16 * (kHd / 4) + 8 * g4];
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                dst[2 * r] = f32x4_t{acc[0][r], acc[1][r], acc[2][r], acc[3][r]} * mul;
                dst[2 * r + 1] = f32x4_t{acc[4][r], acc[5][r], acc[6][r], acc[7][r]} * mul;
              }
              if (g4 == 0) e.ml[r16] = f32x2_t{bad ? nanv : m_run, bad ? nanv : l};
            }
            if (lane == 0) {
              const int64_t gu = cc.G + static_cast<int64_t>(cc.u) * cc.nts;
              e.split = !(seg_g0 == gu && cc.t == cc.nts - 1);
              e.side = seg_g0 == lo ? 0 : 1;
              e.unit = static_cast<int64_t>(cc.s) * KVG + cc.u;
              e.gu = gu;
              e.nts = cc.nts;
              e.hcount = hcount;
              e.row0 = row0;
              e.taken = 0;
            }
            ++head;
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if (lane == 0) lds_put(&bx.head, head);
            }
          }
          advance(a, cc, KVG, maxn, n_lane);
          ++gc;
        }
        __builtin_amdgcn_sched_barrier(0);
        issue_next(ring[k], k);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    return !gave_up;
  }

  // The helper of the streamer with range index `rid` (share * share_ranges
  // + range): first the rows of empty (zero) and out-of-range (NaN)
  // sequences, then the mailbox until the streamer is done.
  static __device__ void helper_main(const DecodeArgs &a, Box &bx, int64_t T, int64_t rid, int64_t lo, int64_t hi,
                                     int lane, int n_lane, int64_t cnt0, int64_t incl0, const int64_t *rs,
                                     const int *rc, Pre &s_pre_own, int &s_preok) {
    const int64_t nh = 4 * static_cast<int64_t>(gridDim.x);
    const int maxn = a.max_blocks * BS;
    const int hid = static_cast<int>(threadIdx.x >> 6) - 4;
    for (int s = hid * static_cast<int>(gridDim.x) + static_cast<int>(blockIdx.x); s < a.num_seqs;
         s += static_cast<int>(nh)) {
      const int n = load_const(a.ctx, s);
      if (n > 0 && n <= maxn) continue;
      const float fill = n == 0 ? 0.0f : __builtin_nanf("");
      for (int i = lane; i < a.num_q_heads * (kHd / 4); i += 64)
        store4(a, (static_cast<int64_t>(s) * a.num_q_heads + (i >> 5)) * kHd + 4 * (i & 31),
               make_float4(fill, fill, fill, fill), 1.0f);
    }

    Pre pre;
    pre.on = false;
    if (lo < hi) {
      const Cursor c = locate(a, hi - 1, lane, n_lane, cnt0, incl0);
      const int64_t gu = c.G + static_cast<int64_t>(c.u) * c.nts, glast = gu + c.nts - 1;
      if (gu < lo || glast >= hi) {
        int64_t r1, count, rl;
        holders(T, gu, glast, rs, rc, r1, count, rl);
        if (count <= kPre) {
          pre.on = true;
          pre.unit = static_cast<int64_t>(c.s) * (a.num_kv_heads * a.head_groups) + c.u;
          pre.count = count;
          pre.cross = (rc[r1] >> 20) != (rc[rl] >> 20);
          int64_t jr = r1;
#pragma unroll
          for (int j = 0; j < kPre; ++j) {
            pre.slot[j] = -1;
            if (j < count) {
              while (rs[jr + 1] == rs[jr]) ++jr;
              pre.slot[j] = ((rc[jr] >> 20) * a.share_ranges + (rc[jr] & 0xfffff)) * 2 + (rs[jr] < gu ? 1 : 0);
              ++jr;
            }
          }
        }
      }
    }

    // the streamer handles its last entry itself when it gets there first
    if (lane == 0) s_pre_own = pre;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (lane == 0) __hip_atomic_fetch_add(&s_preok, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);

    int tail = 0, idle = 0;
    for (;;) {
      const int done = uniform(lds_get(&bx.done));
      const int head = uniform(lds_get(&bx.head));
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      if (tail < head) {
        idle = 0;
        int won = 0;
        if (lane == 0) {
          int expect = 0;
          won = __hip_atomic_compare_exchange_strong(&bx.m[tail % kMail].taken, &expect, 1, __ATOMIC_RELAXED,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        if (uniform(won) != 0) handle(a, T, rid, bx.m[tail % kMail], lane, rs, rc, pre);
        ++tail;
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (lane == 0) lds_put(&bx.tail, tail);
        continue;
      }
      if (done) break;
      if (++idle > a.wait_polls) {     // the streamer neither posts nor finishes
        abandon(a, lane);
        return;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }

  // The ranges holding the unit's tiles [gu, glast]: the first (r1) and
  // last (rl) of them and how many are non-empty (count).  The range holding
  // gu is found from a proportional guess (ranges are near-equal, so it is a
  // step or two away).
  static __device__ __forceinline__ void holders(int64_t T, int64_t gu, int64_t glast, const int64_t *rs,
                                                 const int *rc, int64_t &r1, int64_t &count, int64_t &rl) {
    const int64_t NR = 4 * static_cast<int64_t>(gridDim.x);
    r1 = min(NR - 1, static_cast<int64_t>(static_cast<float>(gu) * static_cast<float>(NR) / static_cast<float>(T)));
    while (rs[r1] > gu) --r1;
    while (rs[r1 + 1] <= gu) ++r1;
    count = 1;
    rl = r1;
    for (int64_t j = r1 + 1; j < NR && rs[j] <= glast; ++j)
      if (rs[j + 1] > rs[j]) {
        ++count;
        rl = j;
      }
  }


  // The helper's work for one mailbox entry of the streamer with range index
  // `rid`.  A whole unit: its output rows.  A split unit: the range's partial
  // is published (partial slot (range index, side); side 1 when the range
  // began before the unit), then counted in on the unit's counter; the count
  // that reaches the number of ranges holding the unit merges their partials
  // in tile order (this one straight from LDS), writes the rows and resets
  // the counter to zero.
  static __device__ void handle(const DecodeArgs &a, int64_t T, int64_t rid, const Mail &e, int lane,
                                const int64_t *rs, const int *rc, Pre &pre, bool probe = false) {
    const int NX = a.num_xcd;
    const int hc = e.hcount;
    const int64_t row0 = e.row0;
    if (!e.split) {
      for (int i = lane; i < hc * (kHd / 4); i += 64) {
        const int h = i >> 5;
        const f32x4_t o = e.o[i];
        store4(a, (row0 + h) * kHd + 4 * (i & 31), make_float4(o[0], o[1], o[2], o[3]), a.v_scale / e.ml[h][1]);
      }
      return;
    }
    const int64_t gu = e.gu, glast = e.gu + e.nts - 1;
    const int64_t sr = a.share_ranges;
    const bool known = pre.on && e.unit == pre.unit;   // the range's last unit, worked out ahead
    int64_t r1 = 0, count, rl = 0;
    bool cross;
    if (known) {
      count = pre.count;
      cross = pre.cross;
    } else {
      holders(T, gu, glast, rs, rc, r1, count, rl);
      cross = (rc[r1] >> 20) != (rc[rl] >> 20);
    }
    // partial slot of range j for this unit
    auto slot_of = [&](int64_t j) {
      return ((rc[j] >> 20) * sr + (rc[j] & 0xfffff)) * 2 + (rs[j] < gu ? 1 : 0);
    };
    const auto ro = float_rsrc(a.part_o, NX * sr * 2 * GT * kHd);
    const auto rm = float_rsrc(a.part_m, NX * sr * 2 * kSlotMlFloats);
    const int own = static_cast<int>(rid * 2 + e.side);
    uint64_t *ctr = unit_ctr(a, e.unit);
    // `probe` (the range's last segment, taken by the streamer): when every
    // other holder is counted in already, this one is the last for sure, so
    // it merges at once and publishes and counts nothing
    bool last_for_sure = false;
    if (probe && known) {
      uint64_t c = 0;
      if (lane == 0) c = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_for_sure = static_cast<uint64_t>(uniform(static_cast<int64_t>(c))) == static_cast<uint64_t>(count - 1);
    }
    if (last_for_sure) {
    } else if (cross) {
      for (int i = lane; i < GT * (kHd / 4); i += 64) rsrc_store4(ro, (own * (GT * kHd) + 4 * i) * 4, e.o[i]);
      if (lane < GT) rsrc_store2(rm, (own * kSlotMlFloats + 2 * lane) * 4, e.ml[lane]);
    } else {
      typedef uint32_t w4 __attribute__((ext_vector_type(4)));
      typedef uint32_t w2 __attribute__((ext_vector_type(2)));
      for (int i = lane; i < GT * (kHd / 4); i += 64)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(w4, e.o[i]), ro, (own * (GT * kHd) + 4 * i) * 4, 0, 0);
      if (lane < GT)
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(w2, e.ml[lane]), rm, (own * kSlotMlFloats + 2 * lane) * 4, 0, 0);
    }
    if (!last_for_sure) {
      // Ordering of publish -> count -> merge.  The memory model offers no
      // scope between a workgroup and the whole device, and an agent-scope
      // release/acquire pair would write back / invalidate the L2 (measured:
      // the acquire alone re-reads the partials from HBM, +1.3 us).  The
      // order is kept by the hardware and pinned for the compiler instead:
      //  * publish: every partial store has completed (vmcnt(0)) before the
      //    count-in atomic is issued, so a counter value that includes this
      //    holder implies its partial sits in the L2 the readers use (the
      //    share's own L2, or memory for the sc1 stores of a unit that
      //    crosses a share boundary);
      //  * merge: the partial loads are issued only after the atomic has
      //    returned the completing count (they depend on its value through
      //    the branch below), and a compiler fence keeps the compiler from
      //    moving any memory access across that point;
      //  * the merging compute unit's L1 holds no stale copy: no line of a
      //    slot is loaded before the slot is counted in, once per launch, and
      //    no two slots share a line (sc1 loads bypass it anyway).
      __builtin_amdgcn_s_waitcnt(0x0f70);      // vmcnt(0): published before counted
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      uint64_t old = 0;
      if (lane == 0) old = __hip_atomic_fetch_add(ctr, uint64_t{1}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (uniform(static_cast<int64_t>(old)) != count - 1) return;
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }

    // the last count: fold the unit's partials in tile order, eight loads in
    // flight at a time
    const float nanv = __builtin_nanf("");
    const int r16 = lane & 15, g4 = lane >> 4;
    for (int h = g4; h < hc; h += 4) {
      float big_m = -INFINITY, l = 0.0f;
      float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      bool nan_seen = false;
      int64_t jr = r1;                 // next range to fold
      for (int64_t done = 0; done < count;) {
        Partial p[8];
        bool live[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          live[j] = done < count;
          int64_t sl = own;
          if (live[j]) {
            if (known) {
              sl = pre.slot[j];              // count <= kPre == 8: one batch
            } else {
              while (rs[jr + 1] == rs[jr]) ++jr;   // empty ranges hold no partial
              sl = slot_of(jr++);
            }
            ++done;
          }
          if (sl == own) {
            p[j].ml = e.ml[h];
            p[j].o0 = e.o[h * (kHd / 4) + 2 * r16];
            p[j].o1 = e.o[h * (kHd / 4) + 2 * r16 + 1];
          } else {
            const int ob = (static_cast<int>(sl) * (GT * kHd) + h * kHd + 8 * r16) * 4;
            const int mb = (static_cast<int>(sl) * kSlotMlFloats + 2 * h) * 4;
            if (cross) {
              p[j].ml = rsrc_load2(rm, mb);
              p[j].o0 = rsrc_load4(ro, ob);
              p[j].o1 = rsrc_load4(ro, ob + 16);
            } else {
              // from the XCD's L2: no line of a slot is loaded before the
              // slot is counted in, and no two slots share a line, so this
              // compute unit's L1 holds no stale copy
              p[j].ml = __builtin_bit_cast(f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rm, mb, 0, 1));
              p[j].o0 = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ro, ob, 0, 1));
              p[j].o1 = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ro, ob + 16, 0, 1));
            }
          }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (live[j]) fold(p[j], big_m, l, o, nan_seen);
      }
      const float mul = nan_seen ? nanv : a.v_scale / l;
      const int64_t base_idx = (row0 + h) * kHd + 8 * r16;
      store4(a, base_idx, make_float4(o[0], o[1], o[2], o[3]), mul);
      store4(a, base_idx + 4, make_float4(o[4], o[5], o[6], o[7]), mul);
    }
    if (lane == 0) __hip_atomic_store(ctr, uint64_t{0}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // Partitions the workgroups of the split take in turn: for each sequence
  // (in order), each of its units, each of its partitions; a sequence with
  // no positions or a bad length has one (that writes its rows).
  static __device__ __forceinline__ int64_t seq_parts(int n, int maxn, int P, int window) {
    return (n <= 0 || n > maxn) ? 1 : (n + P - 1) / P - window_lo(n, window) / P;
  }

  // The split with fixed partitions: gridDim.x workgroups take the batch's
  // partitions i = blockIdx.x, blockIdx.x + gridDim.x, ... so that the grid
  // holds no workgroup for a partition past a context's end.
  static __device__ void run_split(const DecodeArgs &a) {
    const int lane = threadIdx.x & 63;
    const int S = a.num_seqs;
    const int KVG = a.num_kv_heads * a.head_groups;
    const int maxn = a.max_blocks * BS;
    const int P = a.partition_size;
    int64_t base = 0;                  // items before sequence chunk c0
    int c0 = 0;
    int64_t incl = 0, cnt = 0;         // this lane's sequence c0 + lane: items up to and including it, its items
    auto scan = [&]() {
      const int s = c0 + lane;
      cnt = s < S ? seq_parts(load_const(a.ctx, s), maxn, P, a.window) * KVG : 0;
      incl = cnt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int64_t up = __shfl_up(incl, o, 64);
        if (lane >= o) incl += up;
      }
    };
    scan();
    for (int64_t i = blockIdx.x;; i += gridDim.x) {
      // advance to the chunk of 64 sequences holding item i (items only grow)
      while (c0 < S && base + lane_value(incl, 63) <= i) {
        base += lane_value(incl, 63);
        c0 += 64;
        if (c0 < S) scan();
      }
      if (c0 >= S) break;
      const int first = uniform(static_cast<int>(__builtin_ctzll(__builtin_amdgcn_ballot_w64(base + incl > i))));
      const int seq = c0 + first;
      const int64_t r = i - (base + lane_value(incl, first) - lane_value(cnt, first));
      const int64_t np = lane_value(cnt, first) / KVG;
      const int y = static_cast<int>(r / np);
      run_item(a, static_cast<int>(r - y * np), y, seq);
    }
  }

  static __device__ void run(const DecodeArgs &a) { run_item(a, 0, blockIdx.y, blockIdx.z); }

  // Partition `part` of unit `y` (KV head * head_groups + head group) of
  // sequence `seq`.
  static __device__ void run_item(const DecodeArgs &a, int part, int y, int seq) {
    __shared__ float s_ml[NW][GT][2];
    __shared__ float4 s_acc[NW][GT][kHd / 4];
    __shared__ __align__(16) uint8_t s_kx[NW][kKxBytes];       // fp8 K relayout, one slot per wave

    const int kvh = y / a.head_groups;
    const int hg = y - kvh * a.head_groups;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);    // uniform: keeps tile math scalar
    const int lane = tid & 63;
    const int r16 = lane & 15;
    const int g4 = lane >> 4;
    const int n = load_const(a.ctx, seq);
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
    // positions [pstart, pend) of partition `part`, counted from the one
    // holding the first position of a sliding window; tiles start on
    // multiples of 16, positions before pstart are masked
    const int lo = window_lo(n, a.window);
    const int P = a.partition_size > 0 ? a.partition_size : n;
    const int nparts = (n + P - 1) / P - lo / P;
    const int ap = lo / P + part;
    if (ap * P >= n) return;
    const int pstart = max(lo, ap * P);
    const int pend = min(n, (ap + 1) * P);
    const int tfirst = pstart / kTile;
    const int ntiles = (pend + kTile - 1) / kTile - tfirst;
    const int nloc = ntiles > wave ? (ntiles - wave + NW - 1) / NW : 0;   // this wave's tiles

    V8 qb[4];
    load_q(a, row0, hcount, r16, g4, qb);

    const int64_t head_bytes = static_cast<int64_t>(BS) * kRow;
    const uint8_t *kb = static_cast<const uint8_t *>(a.k_pool) + kvh * head_bytes;
    const uint8_t *vb = static_cast<const uint8_t *>(a.v_pool) + kvh * head_bytes;
    const int32_t *trow = a.tables + static_cast<int64_t>(seq) * a.max_blocks;
    bool bad = false;
    float m_run, l_run;
    f32x4_t acc[8];
    accumulate(a, qb, kb, vb, trow, pstart, pend, tfirst + wave, nloc, NW, r16, g4, m_run, l_run, acc,
               bad, s_kx[wave]);

    // add the four row groups' sums of exponentials, then hand the wave's
    // state to LDS (lane (h, g4) holds dims 32*g4 .. +31 of head h)
    l_run = xor32_sum(xor16_sum(l_run));
    if (r16 < GT) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s_acc[wave][r16][8 * g4 + 2 * r] = make_float4(acc[0][r], acc[1][r], acc[2][r], acc[3][r]);
        s_acc[wave][r16][8 * g4 + 2 * r + 1] = make_float4(acc[4][r], acc[5][r], acc[6][r], acc[7][r]);
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

    // split: publish this partition's partial; the merge is a launch of its
    // own (run_merge), which sees it once this launch has ended.  The
    // partial output is stored normalised (o / l, a weighted mean of V rows,
    // so within the range of the cache's values) and rounded to the q dtype,
    // half the bytes of float32; m and l stay float32.  The stores write
    // through to the device-coherent level, so that the launch does not end
    // with the partials as dirty lines in every L2 to write back.
    const int64_t unit = static_cast<int64_t>(seq) * (a.num_kv_heads * a.head_groups) + y;
    uint16_t *po = reinterpret_cast<uint16_t *>(a.part_o) + (unit * a.max_parts + part) * (GT * kHd);
    float *pml = a.part_m + (unit * a.max_parts + part) * (GT * 2);
    for (int i = tid; i < GT * (kHd / 4); i += kThreads) {
      const int h = i >> 5, d4 = i & 31;
      float big_m, l;
      float4 o;
      wave_merge(h, d4, big_m, l, o);
      const float mul = any_bad ? nanv : 1.0f / l;     // l >= 1: the running max's own term
      coherent_store2_at(po, (h * kHd + 4 * d4) * 2, pack4(make_float4(o.x * mul, o.y * mul, o.z * mul, o.w * mul)));
      if (d4 == 0)
        coherent_store2_at(pml, h * 8, __builtin_bit_cast(uint2, make_float2(any_bad ? nanv : big_m, any_bad ? nanv : l)));
    }
  }

  // The split's merge: workgroup (unit, h) folds the partials of query head
  // h of that (sequence, head group).  Its lanes form ng groups of 32 (four
  // dims a lane); group j folds partitions j, j + ng, j + 2 ng, ... in
  // increasing order, all of a round's loads (up to 8 partitions) in flight,
  // and group 0 then folds the groups' states in group order.  The round
  // count, not the bytes, sets the time: one round per 8 * ng partitions
  // instead of one per 8.  Sequences held by one partition were written out
  // by the partition itself.
  static __device__ void run_merge(const DecodeArgs &a, int ng) {
    __shared__ f32x4_t s_o[kMergeGroups][32];
    __shared__ f32x2_t s_ml[kMergeGroups];
    const int unit = static_cast<int>(blockIdx.x);
    const int h = static_cast<int>(blockIdx.y);
    const int g = static_cast<int>(threadIdx.x >> 5);
    const int d4 = threadIdx.x & 31;
    const uint16_t *bo = reinterpret_cast<const uint16_t *>(a.part_o) +
                         static_cast<int64_t>(unit) * a.max_parts * (GT * kHd) + h * kHd + 4 * d4;
    const float *bml = a.part_m + static_cast<int64_t>(unit) * a.max_parts * (GT * 2) + 2 * h;
    f32x2_t ml[8];
    uint2 ov[8];
    auto load_round = [&](int p0, int last) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int pp = min(p0 + k * ng, last);
        ml[k] = *reinterpret_cast<const f32x2_t *>(bml + pp * GT * 2);
        ov[k] = *reinterpret_cast<const uint2 *>(bo + pp * GT * kHd);
      }
    };
    // The first round's loads go out before the sequence's length arrives:
    // every slot below max_parts lies inside the workspace, and slots past
    // the sequence's partitions are loaded but never folded.
    load_round(g, a.max_parts - 1);
    asm volatile("" ::: "memory");     // keep those loads ahead of the length's
    const int KVG = a.num_kv_heads * a.head_groups;
    const int seq = unit / KVG;
    const int y = unit - seq * KVG;
    const int kvh = y / a.head_groups;
    const int hg = y - kvh * a.head_groups;
    const int n = load_const(a.ctx, seq);
    if (n <= 0 || n > a.max_blocks * BS) return;
    const int P = a.partition_size;
    const int nparts = (n + P - 1) / P - window_lo(n, a.window) / P;
    if (nparts <= 1) return;
    const int hcount = min(GT, a.group - hg * GT);
    if (h >= hcount) return;
    const int64_t row0 = static_cast<int64_t>(seq) * a.num_q_heads + kvh * a.group + hg * GT;
    float big_m = -INFINITY, l = 0.0f, o[4] = {0, 0, 0, 0};
    bool nan_seen = false;
    for (int p0 = g; p0 < nparts; p0 += 8 * ng) {
      if (p0 != g) load_round(p0, nparts - 1);
      // a partial's unnormalised output is its stored mean times its l
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (p0 + k * ng < nparts) fold4(ml[k], unpack4(ov[k]) * ml[k][1], big_m, l, o, nan_seen);
    }
    // groups 0 .. min(ng, nparts) - 1 hold at least one partition each
    s_o[g][d4] = f32x4_t{o[0], o[1], o[2], o[3]};
    if (d4 == 0) s_ml[g] = f32x2_t{nan_seen ? __builtin_nanf("") : big_m, l};
    __syncthreads();
    if (g != 0) return;
    const int used = min(ng, nparts);
    big_m = -INFINITY;
    l = 0.0f;
    o[0] = o[1] = o[2] = o[3] = 0.0f;
    nan_seen = false;
    for (int j = 0; j < used; ++j) fold4(s_ml[j], s_o[j][d4], big_m, l, o, nan_seen);
    store4(a, (row0 + h) * kHd + 4 * d4, make_float4(o[0], o[1], o[2], o[3]),
           nan_seen ? __builtin_nanf("") : a.v_scale / l);
  }
};

// Waves per workgroup of the fixed-partition kernel: four share a whole
// context (single pass); one takes a whole partition (split), so that the
// per-workgroup set-up and publish are spread over all of its tiles.
constexpr int kFastWaves = 4;
constexpr int kSplitWaves = 1;

template <typename QS, typename KS, int GT, int BS, int NW>
__global__ __launch_bounds__(NW * 64) void decode_fast_kernel(DecodeArgs a) {
  Fast<QS, KS, GT, BS, NW>::run(a);
}

// Waves per SIMD the split is built for: three, except for the group-2
// 16-bit instances, which need a few more registers than three allow
template <typename KS, int GT>
constexpr int split_waves_per_eu() {
  return (GT == 2 && !std::is_same<KS, FP8S>::value) ? 2 : 3;
}
template <typename QS, typename KS, int GT, int BS>
__global__ __launch_bounds__(kSplitWaves * 64) __attribute__((amdgpu_waves_per_eu(split_waves_per_eu<KS, GT>(), split_waves_per_eu<KS, GT>()))) void decode_split_kernel(DecodeArgs a) {
  Fast<QS, KS, GT, BS, kSplitWaves>::run_split(a);
}

// The fields the merge's first loads depend on come as separate scalar
// arguments ahead of the struct, so that they arrive preloaded in SGPRs
// instead of through dependent loads of the argument block.
template <typename QS, typename KS, int GT, int BS>
__global__ __launch_bounds__(kMergeGroups * 32) void merge_parts_kernel(
    const int32_t *ctx, const float *part_o, const float *part_m, int32_t ng, int32_t max_parts,
    int32_t partition_size, int32_t window, int32_t num_kv_heads, int32_t head_groups, int32_t group,
    int32_t max_blocks, DecodeArgs a) {
  a.ctx = ctx;
  a.part_o = const_cast<float *>(part_o);
  a.part_m = const_cast<float *>(part_m);
  a.max_parts = max_parts;
  a.partition_size = partition_size;
  a.window = window;
  a.num_kv_heads = num_kv_heads;
  a.head_groups = head_groups;
  a.group = group;
  a.max_blocks = max_blocks;
  Fast<QS, KS, GT, BS, kSplitWaves>::run_merge(a, ng);     // ng lane groups: blockDim.x / 32
}

// Most workgroups of the fixed-partition split per compute unit (one wave
// each; the grid is also capped by the workspace's partitions per sequence).
// Every workgroup finds its items by scanning the lengths from the batch's
// start, 64 sequences per step, so the scan grows with the batch: up to 256
// sequences 128 per compute unit beat 32 and 64 (fewer items per workgroup,
// so the dispatcher balances the tail) and 256 (a grid mostly past the
// batch's items); for larger batches 32 beat 128 (fewer workgroups
// repeating long scans).
constexpr int kSplitWgsPerCu = 128;
constexpr int kSplitWgsPerCuLarge = 32;
constexpr int kSplitLargeBatch = 256;      // sequences

template <typename QS, typename KS, int GT, int BS, bool WIN>
// The fields the launch's first loads depend on come as separate scalar
// arguments ahead of the struct, so that they can arrive preloaded in SGPRs
// (kernel-argument preloading) instead of through a load of the argument
// block.
__global__ __launch_bounds__(512) void decode_pair_kernel(const int32_t *ctx, int32_t *ctl, int32_t num_seqs,
                                                          int32_t max_blocks, int32_t num_kv_heads,
                                                          int32_t head_groups, int32_t num_xcd, DecodeArgs a) {
  a.ctx = ctx;
  a.ctl = ctl;
  a.num_seqs = num_seqs;
  a.max_blocks = max_blocks;
  a.num_kv_heads = num_kv_heads;
  a.head_groups = head_groups;
  a.num_xcd = num_xcd;
  Fast<QS, KS, GT, BS, 1, WIN>::run_pair(a);
}

// Grid of the balanced split: one 8-wave workgroup (4 streaming waves, one
// per SIMD, and their 4 helpers) per compute unit.  Dynamic LDS that the
// kernel does not touch brings a workgroup's LDS above half of the 160 KiB a
// compute unit has, which keeps a second workgroup off the same unit.
constexpr int kPairLdsBytes = 84 * 1024;
template <typename QS, typename KS, int GT, int BS, bool WIN>
hipError_t launch_stream_win(const DecodeArgs &a, hipStream_t s, const LaunchEvents &ev) {
  static const int fixed = [] {
    hipFuncAttributes at{};
    if (hipFuncGetAttributes(&at, reinterpret_cast<const void *>(&decode_pair_kernel<QS, KS, GT, BS, WIN>)) !=
        hipSuccess)
      return 0;
    return static_cast<int>(at.sharedSizeBytes);
  }();
  const int wgs = min(a.stream_waves / kStreamWavesPerCu, device_compute_units());
  if (wgs < a.num_xcd) return hipErrorInvalidValue;   // every XCD needs a workgroup
  // dynamic LDS: the table of range starts (8 bytes per range, plus T) and
  // range codes (4 bytes per range), at least up to kPairLdsBytes in all
  const int table = (4 * wgs + 1) * 8 + 4 * wgs * 4;
  const int dyn = max(table, kPairLdsBytes - fixed);
  hipExtLaunchKernelGGL((decode_pair_kernel<QS, KS, GT, BS, WIN>), dim3(wgs), dim3(512), dyn, s, ev.start, ev.stop,
                        0, a.ctx, a.ctl, a.num_seqs, a.max_blocks, a.num_kv_heads, a.head_groups, a.num_xcd, a);
  return hipGetLastError();
}

template <typename QS, typename KS, int GT, int BS>
hipError_t launch_stream_gt(const DecodeArgs &a, hipStream_t s, const LaunchEvents &ev) {
  return a.window > 0 ? launch_stream_win<QS, KS, GT, BS, true>(a, s, ev)
                      : launch_stream_win<QS, KS, GT, BS, false>(a, s, ev);
}

template <typename QS, typename KS, int BS>
hipError_t launch_fast_bs(const DecodeArgs &a, hipStream_t s, const LaunchEvents &ev) {
  if (a.stream_waves > 0) {
    switch (a.heads_per_wg) {
      case 1: return launch_stream_gt<QS, KS, 1, BS>(a, s, ev);
      case 2: return launch_stream_gt<QS, KS, 2, BS>(a, s, ev);
      case 4: return launch_stream_gt<QS, KS, 4, BS>(a, s, ev);
      case 8: return launch_stream_gt<QS, KS, 8, BS>(a, s, ev);
      default: return hipErrorInvalidValue;
    }
  }
  const dim3 grid(a.partition_size > 0 ? a.max_parts : 1, a.num_kv_heads * a.head_groups, a.num_seqs);
  if (a.partition_size > 0) {
    const int64_t units = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads * a.head_groups;
    const dim3 block(kSplitWaves * 64);
    // a window of W positions spans at most (W - 1) / P + 2 partitions, far
    // fewer than the table's width allows; workgroups past the batch's
    // items only scan the lengths and leave
    int64_t parts = a.max_parts;
    if (a.window > 0) parts = min(parts, static_cast<int64_t>((a.window - 1) / a.partition_size + 2));
    const int64_t most = units * parts;
    const int per_cu = a.num_seqs <= kSplitLargeBatch ? kSplitWgsPerCu : kSplitWgsPerCuLarge;
    const dim3 sgrid(static_cast<unsigned>(min(most, static_cast<int64_t>(device_compute_units()) * per_cu)));
    const dim3 mgrid(static_cast<unsigned>(units), static_cast<unsigned>(a.heads_per_wg));
    // lane groups per merge workgroup: enough for one round of loads (8
    // partitions a group) at the workspace's most partitions, at least 2
    int ng = 2;
    while (ng < kMergeGroups && 8 * ng < a.max_parts) ng *= 2;
    const dim3 mblock(32 * ng);
    switch (a.heads_per_wg) {
#define PA_SPLIT(G) \
      case G: \
        hipExtLaunchKernelGGL((decode_split_kernel<QS, KS, G, BS>), sgrid, block, 0, s, ev.start, nullptr, 0, a); \
        hipExtLaunchKernelGGL((merge_parts_kernel<QS, KS, G, BS>), mgrid, mblock, 0, s, nullptr, ev.stop, 0, a.ctx, \
                              a.part_o, a.part_m, ng, a.max_parts, a.partition_size, a.window, a.num_kv_heads, \
                              a.head_groups, a.group, a.max_blocks, a); \
        break;
      PA_SPLIT(1) PA_SPLIT(2) PA_SPLIT(4) PA_SPLIT(8)
#undef PA_SPLIT
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const dim3 block(kFastWaves * 64);
  switch (a.heads_per_wg) {
#define PA_SINGLE(G) \
    case G: hipExtLaunchKernelGGL((decode_fast_kernel<QS, KS, G, BS, kFastWaves>), grid, block, 0, s, ev.start, ev.stop, 0, a); break;
    PA_SINGLE(1) PA_SINGLE(2) PA_SINGLE(4) PA_SINGLE(8)
#undef PA_SINGLE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename QS, typename KS>
hipError_t launch_fast_t(const DecodeArgs &a, hipStream_t s, const LaunchEvents &ev) {
  return a.block_size == 16 ? launch_fast_bs<QS, KS, 16>(a, s, ev) : launch_fast_bs<QS, KS, 32>(a, s, ev);
}

}  // namespace

// This file is compiled once per (q, cache) dtype pair, PA_FAST_COMBO naming
// the pair, so that the four sets of kernels build in parallel.
#if PA_FAST_COMBO == 0
hipError_t launch_fast_bf16_bf16(const DecodeArgs &a, hipStream_t s, const LaunchEvents &ev) {
  return launch_fast_t<BF16S, BF16S>(a, s, ev);
}
#elif PA_FAST_COMBO == 1
hipError_t launch_fast_f16_f16(const DecodeArgs &a, hipStream_t s, const LaunchEvents &ev) {
  return launch_fast_t<F16S, F16S>(a, s, ev);
}
#elif PA_FAST_COMBO == 2
hipError_t launch_fast_bf16_fp8(const DecodeArgs &a, hipStream_t s, const LaunchEvents &ev) {
  return launch_fast_t<BF16S, FP8S>(a, s, ev);
}
#elif PA_FAST_COMBO == 3
hipError_t launch_fast_f16_fp8(const DecodeArgs &a, hipStream_t s, const LaunchEvents &ev) {
  return launch_fast_t<F16S, FP8S>(a, s, ev);
}
#else
#error "PA_FAST_COMBO must name a dtype pair (0..3)"
#endif

}  // namespace pa_impl
