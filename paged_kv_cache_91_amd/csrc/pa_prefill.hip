// Paged prefill for head_dim 128 on gfx950: causal multi-query attention of
// a prompt (or a chunk of one after a cached prefix) over K/V read through
// the block table, with both products on the matrix cores.
//
// What is computed is the causal attention of zerocoder.ru "Что такое
// PagedAttention", section "Зачем KV cache вообще нужен" (each position
// attends the keys and values of the positions before it), read from the
// paged blocks as ultralytics.com "PagedAttention", section "관련 기법",
// describes for FlashAttention-style kernels: K/V tiles are streamed through
// on-chip memory and the softmax is evaluated online, so the score matrix
// never reaches HBM.
//
// Work.  A workgroup of 4 waves owns one (sequence, KV head) and a block of
// kQb consecutive query positions; its columns are the (position, query
// head) pairs of the group (16 per column group, head fastest), 2 column
// groups per wave.  Keys are walked from the first one any column sees to
// the block's last position in tiles of 32, each staged once in LDS for all
// four waves (padded rows; double-buffered, the next tile's global loads in
// flight during the current tile's compute).
//
// Per 32-key tile and column group (the decode kernel's layout with query
// columns in place of heads):
//   S^T = K . Q^T   per 16-key half, four v_mfma_f32_16x16x32 (A = 16 key
//                   rows from LDS, B = the column group's q); lane l holds
//                   keys 4*(l/16)+r of each half for column l%16;
//   online softmax per column in the base-2 domain over the 32 keys, causal
//   (and window) mask only on tiles that reach past a column's position;
//   O^T += V^T . P  eight v_mfma_f32_16x16x32 over all 32 keys (A = V read
//                   from the row-major tile by transposing LDS reads in the
//                   probabilities' key order, B = the probabilities in place).
// Blocks are ordered so that all blocks of one (sequence, KV head) land on
// one XCD (their K/V is re-read from that XCD's L2), last block first.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "pa_common.h"
#include "pa_internal.h"
#include "pa_mfma.h"

namespace pa_impl {
namespace {

constexpr int kHd = 128;
constexpr int kKeys = 32;                  // keys per staged tile
// LDS row stride of the staged K and V tiles: 32 bytes of padding (rows
// start 8 banks apart), which measured free of bank conflicts for all three
// access patterns (the staging writes, the K reads of one column of 16 rows,
// the transposing V reads of 32 bytes from each of 8 rows); 16 bytes left a
// third of the LDS cycles in conflicts.
constexpr int kRowBytes = kHd * 2 + 32;
constexpr int kWaves = 4;
constexpr int kCg = 2;                     // column groups (16 columns each) per wave
constexpr int kRsrcWord3 = 0x00020000;     // buffer resource: raw buffer, 32-bit elements
constexpr int kMfmaPrio = 1;              // wave priority during the matrix-core bursts (measured: 2 gains nothing)
constexpr float kLazy = 8.0f;              // base-2 headroom before the running max moves

// max2 (pa_mfma.h): IEEE maximum, v_maximum3_f32 for two of them in a row
__device__ __forceinline__ float max3(float a, float b, float c) { return max2(max2(a, b), c); }
__device__ __forceinline__ float lanes16_max(float x) {        // over lanes l, l ^ 16, l ^ 32, l ^ 48
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap16(a, b);
  x = max2(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
  a = b = __builtin_bit_cast(uint32_t, x);
  swap32(a, b);
  return max2(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

typedef short tr16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 read_tr(const uint8_t *lds) {
  const tr16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) tr16x4_t *)(reinterpret_cast<uintptr_t>(lds)));
  return __builtin_bit_cast(uint2, v);
}

typedef const __attribute__((address_space(4))) int32_t cint32_t;
__device__ __forceinline__ int load_const(const int32_t *p, int64_t i) { return ((cint32_t *)p)[i]; }

template <typename QS, int G, int BS>
struct Prefill {
  using M = Mma<QS>;
  using V8 = typename M::V8;
  using V4 = typename M::V4;
  static constexpr int kPos = 16 / G;                   // positions per column group
  static constexpr int kQb = kWaves * kCg * kPos;       // query positions per workgroup
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group must divide 16");
  static_assert(BS == 16 || BS == 32, "block size 16 or 32");

  // head dims of lane group g4's 8-element run in MFMA j (A and B agree)
  static __device__ __forceinline__ int dbase(int j, int g4) { return 32 * j + 8 * g4; }

  static __device__ __forceinline__ void store4(void *out, int64_t idx, float4 o, float mul) {
    uint2 w;
    if constexpr (std::is_same<QS, BF16S>::value) {
      w.x = f32_to_bf16(o.x * mul) | (static_cast<uint32_t>(f32_to_bf16(o.y * mul)) << 16);
      w.y = f32_to_bf16(o.z * mul) | (static_cast<uint32_t>(f32_to_bf16(o.w * mul)) << 16);
    } else {
      w.x = f32_to_f16(o.x * mul) | (static_cast<uint32_t>(f32_to_f16(o.y * mul)) << 16);
      w.y = f32_to_f16(o.z * mul) | (static_cast<uint32_t>(f32_to_f16(o.w * mul)) << 16);
    }
    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + idx) = w;
  }

  static __device__ void run(const DecodeArgs &a) {
    __shared__ __align__(16) uint8_t s_k[2][kKeys * kRowBytes];
    __shared__ __align__(16) uint8_t s_v[2][kKeys * kRowBytes];
    const int tid = threadIdx.x;
    const int wave = uniform(static_cast<int>(tid >> 6));
    const int lane = tid & 63;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int S = a.num_seqs;
    const int Hkv = a.num_kv_heads;
    const int maxn = a.max_blocks * BS;

    // item -> (KV head, block r of the batch's query blocks); blocks are
    // counted per sequence, ceil(L / kQb) each, found by a wave-wide scan
    const int64_t item = blockIdx.x;
    const int kvh = static_cast<int>(item % Hkv);
    const int64_t r = item / Hkv;
    int seq = -1, nb_s = 0;
    int64_t k_in = 0;
    {
      int64_t base = 0;
      for (int c0 = 0; c0 < S; c0 += 64) {
        const int s = c0 + lane;
        uint32_t nb = 0;
        if (s < S) {
          const int L = a.query_start[s + 1] - a.query_start[s];
          nb = L > 0 ? static_cast<uint32_t>((static_cast<int64_t>(L) + kQb - 1) / kQb) : 0u;
        }
        const uint32_t incl = wave_incl_sum(nb);
        const int64_t total = __builtin_amdgcn_readlane(incl, 63);
        if (base + total > r) {
          const uint64_t m = __builtin_amdgcn_ballot_w64(base + static_cast<int64_t>(incl) > r);
          const int first = uniform(static_cast<int>(__builtin_ctzll(m)));
          seq = c0 + first;
          nb_s = static_cast<int>(__builtin_amdgcn_readlane(nb, first));
          k_in = r - (base + static_cast<int64_t>(__builtin_amdgcn_readlane(incl, first)) - nb_s);
          break;
        }
        base += total;
      }
    }
    // past the batch's blocks (the grid is an upper bound); a block index
    // outside its sequence's count only comes from a malformed prefix sum
    // whose block counts wrapped the 32-bit scan
    if (seq < 0 || k_in < 0 || k_in >= nb_s) return;

    const int q0 = load_const(a.query_start, seq);
    const int L = load_const(a.query_start, seq + 1) - q0;
    const int n = load_const(a.ctx, seq);
    const int qb = nb_s - 1 - static_cast<int>(k_in);          // last block first
    const int P0 = n - L;                                       // the first query's position
    const int pb0 = P0 + qb * kQb;                              // this block's first query position
    const int pb1 = min(n, pb0 + kQb);                          // one past its last
    // a malformed prefix sum (rows outside [0, num_tokens)) or length gives
    // NaN rows; only rows inside out are ever written
    const bool bad_rows = q0 < 0 || q0 + L > a.num_tokens;
    const bool bad_len = bad_rows || n < 0 || n > maxn || L > n;

    // this lane's column in each column group: position qp[cg], head h
    const int h = kvh * G + r16 % G;
    int qp[kCg];
    bool valid[kCg];
#pragma unroll
    for (int cg = 0; cg < kCg; ++cg) {
      qp[cg] = pb0 + (wave * kCg + cg) * kPos + r16 / G;
      valid[cg] = qp[cg] < pb1;
    }
    auto out_idx = [&](int cg) {           // the column's output row
      return (static_cast<int64_t>(q0 + qp[cg] - P0) * a.num_q_heads + h) * kHd;
    };
    if (bad_len) {
      const float nanv = __builtin_nanf("");
#pragma unroll
      for (int cg = 0; cg < kCg; ++cg) {
        const int64_t row =
            static_cast<int64_t>(q0) + static_cast<int64_t>(qb) * kQb + (wave * kCg + cg) * kPos + r16 / G;
        if (row < static_cast<int64_t>(q0) + L && row >= 0 && row < a.num_tokens)
#pragma unroll
          for (int r4 = 0; r4 < 8; ++r4)
            store4(a.out, (row * a.num_q_heads + h) * kHd + 32 * g4 + 4 * r4, make_float4(nanv, nanv, nanv, nanv),
                   1.0f);
      }
      return;
    }

    // q of each column as the MFMA B operand (zero for columns past the block)
    const uint32_t qsign = a.scale_log2 < 0.0f ? 0x80008000u : 0u;
    const float sl = fabsf(a.scale_log2);
    V8 qop[kCg][4];
#pragma unroll
    for (int cg = 0; cg < kCg; ++cg) {
      const uint16_t *qrow = static_cast<const uint16_t *>(a.q) +
                             (static_cast<int64_t>(q0 + qp[cg] - P0) * a.num_q_heads + h) * kHd;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint4 w = make_uint4(0u, 0u, 0u, 0u);
        if (valid[cg]) w = *reinterpret_cast<const uint4 *>(qrow + dbase(j, g4));
        // a negative scale moves to q (a sign flip, exact), so that the
        // score scale sl below is >= 0 and max(sl * s) = sl * max(s)
        w.x ^= qsign;
        w.y ^= qsign;
        w.z ^= qsign;
        w.w ^= qsign;
        qop[cg][j] = __builtin_bit_cast(V8, w);
      }
    }

    // keys [klo, khi): from the first position any column sees to the last
    // query's position
    const int khi = pb1;
    const int klo = window_lo(pb0 + 1, a.window);
    const int kt0 = klo / kKeys;
    const int ntiles = (khi + kKeys - 1) / kKeys - kt0;
    // this wave's columns: positions wq0 .. wq1 (none when wq0 >= pb1)
    const int wq0 = pb0 + wave * kCg * kPos;
    const int wq1 = min(pb1 - 1, wq0 + kCg * kPos - 1);
    const bool idle = wq0 >= pb1;
    const int wlo0 = window_lo(wq0 + 1, a.window);              // smallest first key of the wave's columns
    const int wlo1 = window_lo(wq1 + 1, a.window);              // largest
    int lo_col[kCg];
#pragma unroll
    for (int cg = 0; cg < kCg; ++cg) lo_col[cg] = window_lo(qp[cg] + 1, a.window);

    // staging: thread (row rr, 16-byte chunk ch) moves rows rr and rr + 16
    // of K and of V; table entries are clamped to [klo, khi)'s blocks so
    // released or unwritten entries are never read
    const int rr = tid >> 4, ch = tid & 15;
    const int64_t head_bytes = static_cast<int64_t>(BS) * kHd * 2;
    const int64_t blk_bytes = head_bytes * Hkv;
    const uint8_t *kpool = static_cast<const uint8_t *>(a.k_pool) + kvh * head_bytes;
    const uint8_t *vpool = static_cast<const uint8_t *>(a.v_pool) + kvh * head_bytes;
    const int32_t *trow = a.tables + static_cast<int64_t>(seq) * a.max_blocks;
    const int jmin = klo / BS, jmax = (khi - 1) / BS;
    bool bad = false;
    // The 16 positions from kb16 (a multiple of 16) sit in one block, so
    // their table entry is uniform (a scalar load) and so is the address of
    // their rows: a buffer resource over those 16 rows, with this thread's
    // chunk at a fixed offset.
    const int lane_off = rr * (kHd * 2) + ch * 16;
    auto rows_of = [&](const uint8_t *pool, int kb16) {
      const int j = uniform(min(max(kb16 / BS, jmin), jmax));
      int e = load_const(trow, j);
      if (static_cast<uint32_t>(e) >= static_cast<uint32_t>(a.num_blocks)) {
        bad = true;
        e = 0;
      }
      const int64_t base = static_cast<int64_t>(e) * blk_bytes + (kb16 % BS) * (kHd * 2);
      return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(pool + base), 0, 16 * kHd * 2, kRsrcWord3);
    };
    auto load16 = [&](__amdgpu_buffer_rsrc_t r) {
      typedef uint32_t w4 __attribute__((ext_vector_type(4)));
      const w4 v = __builtin_amdgcn_raw_buffer_load_b128(r, lane_off, 0, 0);
      return make_uint4(v[0], v[1], v[2], v[3]);
    };
    // the next tile's chunks, held in named registers (an array here ends up
    // in scratch memory, which would wait for the loads at once)
    uint4 sk0, sk1, sv0, sv1;
    auto fetch = [&](int t) {
      const int kbase = uniform((kt0 + t) * kKeys);
      sk0 = load16(rows_of(kpool, kbase));
      sv0 = load16(rows_of(vpool, kbase));
      sk1 = load16(rows_of(kpool, kbase + 16));
      sv1 = load16(rows_of(vpool, kbase + 16));
    };
    // V rows of positions outside [klo, khi) hold bytes of no position
    // attended here: their probabilities are 0, but NaN or Inf would survive
    // the product, so on the tiles that reach outside they are staged as
    // zeros (all-ones or all-zeros masks: a select of whole vectors becomes a
    // scratch-memory lookup)
    auto stage = [&](int buf, int t) {
      const int kbase = uniform((kt0 + t) * kKeys);
      uint4 *v0 = reinterpret_cast<uint4 *>(&s_v[buf][rr * kRowBytes + ch * 16]);
      uint4 *v1 = reinterpret_cast<uint4 *>(&s_v[buf][(rr + 16) * kRowBytes + ch * 16]);
      *reinterpret_cast<uint4 *>(&s_k[buf][rr * kRowBytes + ch * 16]) = sk0;
      *v0 = sv0;
      *reinterpret_cast<uint4 *>(&s_k[buf][(rr + 16) * kRowBytes + ch * 16]) = sk1;
      *v1 = sv1;
      // rows outside the range are then overwritten with zeros by the thread
      // that staged them (its LDS writes land in order), which keeps the
      // fetched registers flowing straight into the stores above
      if (kbase < klo || kbase + kKeys > khi) {
        const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
        if (!(kbase + rr >= klo && kbase + rr < khi)) *v0 = zero;
        if (!(kbase + rr + 16 >= klo && kbase + rr + 16 < khi)) *v1 = zero;
      }
    };

    // Transposing read (ds_read_b64_tr_b16): within each 16-lane block, lane
    // 4i + k receives element k of the 4-element pieces named by lanes i,
    // i + 4, i + 8 and i + 12.  Lane (r16, g4) names the piece of key
    // 4 g4 + r16 / 4 (16 more for the upper read) at dims 4 (r16 % 4) .. + 3
    // of the MFMA's 16, so lane (m, g4) receives dim m at keys 4 g4 .. + 3:
    // the key slots of the probabilities in B.
    const int vt_off = (4 * g4 + (r16 >> 2)) * kRowBytes + 8 * (r16 & 3);

    float m_run[kCg], l_run[kCg];
    f32x4_t acc[kCg][8];
#pragma unroll
    for (int cg = 0; cg < kCg; ++cg) {
      m_run[cg] = -INFINITY;
      l_run[cg] = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[cg][e] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }

    // One staged 32-key tile (keys kbase .. kbase + 31) against the wave's
    // columns.  q.K^T runs per 16-key half (A = 16 key rows); lane (r16, g4)
    // then holds, for its column r16, the keys of slots j < 8: half j / 4,
    // key 4 * g4 + j % 4 -- exactly the K-slot order of a 16x16x32 MFMA, so
    // P.V is eight 16x16x32 MFMAs over all 32 keys (MFMA e: A = V of head
    // dims 16e .. 16e + 15 in the same slot order, B = the probabilities in
    // place).
    //
    // Online softmax in the base-2 domain, updated once per tile.  The
    // running max m of a column is only moved (and acc, l rescaled) when the
    // tile's max exceeds it by more than kLazy: otherwise the exponents are
    // taken against the old m, which gives the same softmax (it is invariant
    // to the shift) with probabilities up to 2^kLazy, far inside the 16-bit
    // operand's range and with the same relative rounding.
    auto tile = [&](int buf, int kbase, bool masked) {
      float z[kCg][8];                 // raw dot products
      // the matrix-core bursts run at raised wave priority, so that a wave
      // entering one is issued ahead of the softmax work of the others
      __builtin_amdgcn_s_setprio(kMfmaPrio);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        V8 ka[4];
        const uint8_t *krow = &s_k[buf][(hh * 16 + r16) * kRowBytes];
#pragma unroll
        for (int j = 0; j < 4; ++j) ka[j] = __builtin_bit_cast(V8, *reinterpret_cast<const uint4 *>(krow + dbase(j, g4) * 2));
#pragma unroll
        for (int cg = 0; cg < kCg; ++cg) {
          f32x4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int j = 0; j < 4; ++j) sc = M::run(ka[j], qop[cg][j], sc);
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) z[cg][4 * hh + r4] = sc[r4];
        }
      }
      __builtin_amdgcn_s_setprio(0);
      // causal and window masks, on tiles that reach past a column's position
      // or start before its window (one uniform branch)
      if (masked) {
#pragma unroll
        for (int cg = 0; cg < kCg; ++cg) {
          const int hi_off = qp[cg] - kbase - 4 * g4, lo_off = lo_col[cg] - kbase - 4 * g4;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int off = 16 * (j >> 2) + (j & 3);
            z[cg][j] = (off <= hi_off && off >= lo_off) ? z[cg][j] : -INFINITY;
          }
        }
      }
      // Whether some column's maximum passes m_run + kLazy is decided on
      // each lane's own 8 keys (m_run is the same in the four lanes of a
      // column); the column maximum across lanes is only formed when it does.
      float lmx[kCg];
      bool need = false;
#pragma unroll
      for (int cg = 0; cg < kCg; ++cg) {
        lmx[cg] = max3(max3(z[cg][0], z[cg][1], z[cg][2]), max3(z[cg][3], z[cg][4], z[cg][5]), max2(z[cg][6], z[cg][7]));
        need |= lmx[cg] * sl > m_run[cg] + kLazy;                 // true on a column's first keys
      }
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
        for (int cg = 0; cg < kCg; ++cg) {
          const float mx = lanes16_max(lmx[cg]);
          const float mz = mx == -INFINITY ? -INFINITY : mx * sl;   // sl = 0 must not give NaN
          const float m_new = max2(m_run[cg], mz);
          // a column that has seen no key keeps m = -inf; alpha is then 0
          const float alpha = __builtin_amdgcn_exp2f(m_run[cg] - (m_new == -INFINITY ? 0.0f : m_new));
          m_run[cg] = m_new;
          l_run[cg] *= alpha;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[cg][e] *= alpha;
        }
      }
      V8 pb[kCg];
#pragma unroll
      for (int cg = 0; cg < kCg; ++cg) {
        const float neg_m = m_run[cg] == -INFINITY ? 0.0f : -m_run[cg];
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(fmaf(z[cg][j], sl, neg_m));
        if (masked) {
          // masked keys give exp2(-inf) = 0, except at sl = 0 (NaN)
#pragma unroll
          for (int j = 0; j < 8; ++j) p[j] = z[cg][j] == -INFINITY ? 0.0f : p[j];
        }
        const uint4 pk = make_uint4(M::pack2(p[0], p[1]), M::pack2(p[2], p[3]), M::pack2(p[4], p[5]),
                                    M::pack2(p[6], p[7]));
        // the row sum takes the same rounded probabilities P.V multiplies
        // (four two-term dot products with (1, 1))
        l_run[cg] = M::sum2(pk.w, M::sum2(pk.z, M::sum2(pk.y, M::sum2(pk.x, l_run[cg]))));
        pb[cg] = __builtin_bit_cast(V8, pk);
      }
      // O^T += V^T . P, MFMA e over head dims 16e .. 16e + 15: A holds, for
      // lane (m, g4), V of dim 16e + m at the lane's 8 key slots, which two
      // transposing LDS reads deliver from the row-major tile (each lane
      // names one 4-element row piece; see vt_off)
      __builtin_amdgcn_s_setprio(kMfmaPrio);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint8_t *vb = &s_v[buf][vt_off + 32 * e];
        const uint2 lo = read_tr(vb), hi = read_tr(vb + 16 * kRowBytes);
        const V8 va = __builtin_bit_cast(V8, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
        for (int cg = 0; cg < kCg; ++cg) acc[cg][e] = M::run(va, pb[cg], acc[cg][e]);
      }
      __builtin_amdgcn_s_setprio(0);
    };

    fetch(0);
    stage(0, 0);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      const int buf = t & 1;
      if (t + 1 < ntiles) fetch(t + 1);             // in flight during this tile's compute
      const int kbase = (kt0 + t) * kKeys;
      // tiles past every column of the wave, or before every window, are skipped
      if (!idle && kbase <= wq1 && kbase + kKeys - 1 >= wlo0) {
        const bool masked = kbase + kKeys - 1 > wq0 || kbase < wlo1 || kbase < klo || kbase + kKeys - 1 >= khi;
        tile(buf, kbase, masked);
      }
      if (t + 1 < ntiles) stage(buf ^ 1, t + 1);
      __syncthreads();
    }

    // acc[cg][e][r] is dim 16e + 4 g4 + r of column r16
    const float nanv = __builtin_nanf("");
#pragma unroll
    for (int cg = 0; cg < kCg; ++cg) {
      const float l = xor32_sum(xor16_sum(l_run[cg]));
      if (!valid[cg]) continue;
      const float mul = bad ? nanv : 1.0f / l;
      const int64_t idx = out_idx(cg) + 4 * g4;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        store4(a.out, idx + 16 * e, make_float4(acc[cg][e][0], acc[cg][e][1], acc[cg][e][2], acc[cg][e][3]), mul);
    }
  }
};

template <typename QS, int G, int BS>
__global__ __launch_bounds__(kWaves * 64) void prefill_kernel(DecodeArgs a) {
  Prefill<QS, G, BS>::run(a);
}

template <typename QS, int G, int BS>
hipError_t launch_g(const DecodeArgs &a, hipStream_t s) {
  constexpr int qb = Prefill<QS, G, BS>::kQb;
  // an upper bound on the batch's (KV head, query block) items; the surplus
  // workgroups find no block and exit
  const int64_t items = static_cast<int64_t>(a.num_kv_heads) * ((a.num_tokens + qb - 1) / qb + a.num_seqs);
  if (items > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_kernel<QS, G, BS>), dim3(static_cast<unsigned>(items)), dim3(kWaves * 64), 0, s, a);
  return hipGetLastError();
}

template <typename QS, int BS>
hipError_t launch_bs(const DecodeArgs &a, hipStream_t s) {
  switch (a.group) {
    case 1: return launch_g<QS, 1, BS>(a, s);
    case 2: return launch_g<QS, 2, BS>(a, s);
    case 4: return launch_g<QS, 4, BS>(a, s);
    case 8: return launch_g<QS, 8, BS>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename QS>
hipError_t launch_q(const DecodeArgs &a, hipStream_t s) {
  return a.block_size == 16 ? launch_bs<QS, 16>(a, s) : launch_bs<QS, 32>(a, s);
}

}  // namespace

bool prefill_fast_applies(int q_dtype, int kv_dtype, const DecodeArgs &a) {
  if (a.head_dim != kHd || (a.block_size != 16 && a.block_size != 32)) return false;
  if ((q_dtype != kBF16 && q_dtype != kF16) || kv_dtype != q_dtype) return false;
  return a.group == 1 || a.group == 2 || a.group == 4 || a.group == 8;
}

hipError_t launch_prefill_fast(int q_dtype, const DecodeArgs &a, hipStream_t s) {
  return q_dtype == kBF16 ? launch_q<BF16S>(a, s) : launch_q<F16S>(a, s);
}

}  // namespace pa_impl
