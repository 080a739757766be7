// Shared definitions for the gfx950 attention kernels: the launch argument
// block, element-type traits, the 32x32x16 MFMA wrappers and the mask rule.
//
// Mask rule ([P4] "FlashAttention 实战指南", section "进阶参数如何配置causal、
// window_size 与 MQA/GQA", and section "上手 FlashAttention 的三步走" for causal):
// with i' = i + (seqlen_k - seqlen_q), key j is visible from query i iff
// j < seqlen_k, (!causal || j <= i'), (left < 0 || j >= i' - left) and
// (right < 0 || j <= i' + right).  Every kernel reduces this to a per-query
// closed interval [key_lo(i), key_hi(i)].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

enum DType : int32_t { kF32 = 0, kF16 = 1, kBF16 = 2 };

// Everything a launch needs; filled and validated by the C ABI layer.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;        // (B, Hq, Nq) natural log
  const void* dout;  // backward only
  void* dq;
  void* dk;
  void* dv;
  float* dsum;       // (B, Hq, Nq_pad) workspace: D_i = sum_c dout*o (0 on padding rows)
  float* lse2;       // (B, Hq, Nq_pad) workspace: LSE*log2(e), +inf on padding / empty rows
  int64_t q_sb, q_sn, q_sh;
  int64_t k_sb, k_sn, k_sh;
  int64_t v_sb, v_sn, v_sh;
  int64_t o_sb, o_sn, o_sh;
  int32_t B, Nq, Nk, Hq, Hkv, G, D;
  int32_t dtype;
  float scale;       // multiplies q.k
  float scale_log2;  // scale * log2(e): exp(scale*x) == exp2(scale_log2*x)
  int32_t causal, wl, wr;  // wl/wr: -1 = unbounded
  int32_t delta;     // Nk - Nq (queries aligned to the end of the keys)
  int32_t xcd_remap; // 1: map consecutive workgroup ids onto one XCD's work
  // Element strides of the float32 row arrays: lse[b*lse_sb + h*lse_sh + i],
  // dsum / lse2[b*ws_sb + h*ws_sh + i].
  int64_t lse_sb, lse_sh;
  int64_t ws_sb, ws_sh;
  // Packed variable-length batches (NULL: every batch entry has Nq / Nk rows).
  // Sequence b holds rows cu_q[b] .. cu_q[b+1]-1 of q, o, dout, dq and rows
  // cu_k[b] .. cu_k[b+1]-1 of k, v, dk, dv; Nq / Nk are then the longest
  // lengths (they size the grid) and total_q / total_k the packed row counts.
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t total_q, total_k;
  // Score modifiers (kernels built with them only when mod != 0): slope of
  // (b, h) at alibi[b * alibi_sb + h] (NULL: none); cap = softcap / scale in
  // raw score units (+inf: none).
  const float* alibi;
  int64_t alibi_sb;
  float cap;
  float inv_scale;  // 1 / scale: turns a slope into raw score units
  float softcap;    // the parameter itself (0: none), for the float64 path
  int32_t mod;
};

// ---------------------------------------------------------------------------
// Score modifiers ([P4] "FlashAttention 实战指南", section "进阶参数如何配置
// causal、window_size 与 MQA/GQA": alibi_slopes decays scores with distance,
// softcap truncates the logits to [-softcap, softcap]).  In raw units
// (logit = scale * s): s is clamped to [-cap, cap] with cap = softcap/scale,
// then slope/scale * |i' - j| is subtracted; masking comes after.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float mod_score(float s, float cap, float slope_raw, float dist) {
  // One v_med3_f32 for the clamp (fminf/fmaxf would add NaN quieting).
  return fmaf(-slope_raw, fabsf(dist), __builtin_amdgcn_fmed3f(s, -cap, cap));
}
// Slope of (b, h) in raw score units (0 without ALiBi).
__device__ __forceinline__ float alibi_raw(const float* alibi, int64_t sb, float inv_scale, int b, int h) {
  return alibi ? alibi[b * sb + h] * inv_scale : 0.f;
}
// The same for a (b, h) shared by the whole wave: the slope is then kept in a
// scalar register instead of one VGPR per lane.
__device__ __forceinline__ float alibi_raw_uniform(const float* alibi, int64_t sb, float inv_scale, int b, int h) {
  return __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(alibi_raw(alibi, sb, inv_scale, b, h))));
}

// Binds the arguments to batch entry b of a packed variable-length batch:
// every pointer moves to the sequence's first row (the workspace rows to
// cu_q[b] + 128*b, leaving each sequence its own padding rows), the batch
// strides become 0 and Nq / Nk / delta become the sequence's own.  Offsets
// are clamped to the packed tensors and lengths to the launch's maxima, so
// inconsistent offsets can give wrong results but never an access outside
// the tensors.  A fixed-length batch is left as it is.
__device__ __forceinline__ void bind_seq(AttnArgs& a, int b) {
  if (!a.cu_q) return;
  const int q0 = min(max(a.cu_q[b], 0), a.total_q);
  const int q1 = min(max(a.cu_q[b + 1], q0), a.total_q);
  const int k0 = min(max(a.cu_k[b], 0), a.total_k);
  const int k1 = min(max(a.cu_k[b + 1], k0), a.total_k);
  const int64_t e = a.dtype == kF32 ? 4 : 2;
  auto adv = [e](const void* p, int64_t rows, int64_t sn) -> const void* {
    return p ? static_cast<const char*>(p) + rows * sn * e : p;
  };
  a.q = adv(a.q, q0, a.q_sn);
  a.dq = const_cast<void*>(adv(a.dq, q0, a.q_sn));
  a.o = const_cast<void*>(adv(a.o, q0, a.o_sn));
  a.dout = adv(a.dout, q0, a.o_sn);
  a.k = adv(a.k, k0, a.k_sn);
  a.dk = const_cast<void*>(adv(a.dk, k0, a.k_sn));
  a.v = adv(a.v, k0, a.v_sn);
  a.dv = const_cast<void*>(adv(a.dv, k0, a.v_sn));
  a.lse += q0;
  if (a.dsum) a.dsum += q0 + 128 * (int64_t)b;
  if (a.lse2) a.lse2 += q0 + 128 * (int64_t)b;
  a.q_sb = a.k_sb = a.v_sb = a.o_sb = 0;
  a.lse_sb = a.ws_sb = 0;
  a.Nq = min(q1 - q0, a.Nq);
  a.Nk = min(k1 - k0, a.Nk);
  a.delta = a.Nk - a.Nq;
}

// Launch arguments of attention against a KV cache (decode.hip).
struct KvArgs {
  const void* q;
  void* k_cache;
  void* v_cache;
  const void* k_new;  // NULL: no append
  const void* v_new;
  void* o;
  float* lse;                 // (B, Hq, Nq)
  const int32_t* cache_seqlens;  // (B) device
  float* ws_o;                // (B, Hq, Nq, S, D) partial O / l
  float* ws_lse;              // (B, Hq, Nq, S) partial LSE
  int64_t q_sb, q_sn, q_sh;
  int64_t kc_sb, kc_sn, kc_sh;
  int64_t vc_sb, vc_sn, vc_sh;
  int64_t kn_sb, kn_sn, kn_sh;
  int64_t vn_sb, vn_sn, vn_sh;
  int64_t o_sb, o_sn, o_sh;
  int32_t B, Nq, cap, Hq, Hkv, G, D, dtype;
  float scale, scale_log2;
  int32_t causal, wl, wr, append;
  int32_t S;          // key-range parts per (batch, kv head, row block)
  int32_t n_rb;       // blocks of 32 packed query rows (G * Nq rows)
  int32_t n_split;    // waves of the split phase: B * Hkv * n_rb * S
  int32_t n_append;   // waves that copy the new rows into the cache
  const float* alibi;  // score modifiers, as in AttnArgs (score_cap = softcap / scale)
  int64_t alibi_sb;
  float score_cap, inv_scale;
  int32_t mod;
  // Paged caches (page_size 0: contiguous (B, cap, H, d) caches).  Row j of
  // entry b is row j % page_size of page block_table[b * bt_sb + j / page_size]
  // (clamped to [0, num_pages)); the caches' batch strides are page strides.
  const int32_t* block_table;
  int64_t bt_sb;
  int32_t page_size, num_pages;
};

static constexpr float kLog2e = 1.4426950408889634f;
static constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Mask interval for one query row (i' = i + delta).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int key_lo(const AttnArgs& a, int i) {
  int lo = 0;
  if (a.wl >= 0) lo = max(lo, i + a.delta - a.wl);
  return lo;
}
__device__ __forceinline__ int key_hi(const AttnArgs& a, int i) {
  int hi = a.Nk - 1;
  if (a.causal) hi = min(hi, i + a.delta);
  if (a.wr >= 0) hi = min(hi, i + a.delta + a.wr);
  return hi;
}
// Range of queries that see at least one key of [k0, k1] (inclusive).
__device__ __forceinline__ int query_lo(const AttnArgs& a, int k0) {
  int lo = 0;
  if (a.causal) lo = max(lo, k0 - a.delta);
  if (a.wr >= 0) lo = max(lo, k0 - a.delta - a.wr);
  return lo;
}
__device__ __forceinline__ int query_hi(const AttnArgs& a, int k1) {
  int hi = a.Nq - 1;
  if (a.wl >= 0) hi = min(hi, k1 - a.delta + a.wl);
  return hi;
}

// ---------------------------------------------------------------------------
// Element types.  Raw 16-bit storage is uint16_t; MFMA operands are 8
// elements (16 bytes) per lane, carried as u32x4.
// ---------------------------------------------------------------------------
struct BF16 {
  static constexpr int kId = kBF16;
  __device__ __forceinline__ static f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ __forceinline__ static float to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
  }
  // Two floats -> packed pair (lo in bits 0..15), round to nearest even.
  __device__ __forceinline__ static uint32_t pack(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
  }
};

struct F16 {
  static constexpr int kId = kF16;
  __device__ __forceinline__ static f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ __forceinline__ static float to_f32(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
  }
  __device__ __forceinline__ static uint32_t pack(float lo, float hi) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    f16x2 r;
    r[0] = (_Float16)lo;
    r[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, r);
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over the lane pair (l, l^32) of a wave64.  One
// v_permlane32_swap of x with itself leaves {x[l], x[l^32]} in its two
// results (in an order that depends on the half), so max and sum need no LDS
// round trip; the sum has the same two operands in both lanes of the pair and
// is therefore the same bits in both.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// Workgroup -> work-item decode.  On MI355X consecutive workgroup ids are
// dispatched round-robin over the 8 XCDs, each with its own L2.  With
// xcd_remap, id w runs on XCD w % 8, and every "unit" (a (batch, kv head)
// pair) runs whole on one XCD, so that the workgroups sharing K/V also share
// an L2.  XCD x takes the units x, x + 8, x + 16, ...: with the kv heads
// innermost, every XCD then holds the same heads of every batch entry, which
// balances the XCDs also when the sequences of a packed batch differ in
// length.  Inside an XCD the order is tile-major with the heaviest tiles
// (largest causal prefix) first.
// ---------------------------------------------------------------------------
struct WorkItem {
  int unit;   // (batch * Hkv + kv head)
  int tile;   // tile index along the sequence
  int sub;    // index inside the unit's group (query head offset)
};

// Inside an XCD, consecutive slots behave as if handed to its four shader
// engines in turn, each workgroup waiting for a free CU of its own engine: a
// packed batch whose long sequence's workgroups took every other pair of
// slots (the rest empty) ran 35% slower than with groups of four slots of
// equal work.  With
// fixed lengths the units at one tile index do equal work, so the tile-major
// order keeps the engines even.  In a packed batch the units differ in
// length, and slots past a short sequence's end are empty.  With n_sub = 2
// (mod 4) items per (unit, tile), the items of tpg = 2 consecutive tiles of
// one unit take consecutive slots, so that every group of four slots holds
// nearly equal work, and the order of the two tiles alternates from group to
// group, so that over two groups every engine gets the same tiles' worth
// (in the forward with head pairs, a packed batch of the benchmark's heads
// took 9% less time, and a batch of one long and one short sequence 26% less,
// than in the tile-major order).  With
// an odd n_sub the same grouping over four tiles ran a packed MHA forward no
// faster than the tile-major order, which is kept there (work_tiles_per_group).
// n_tiles is padded to a multiple of tpg (padded_tiles); the padding tiles lie
// past every sequence's end.
// ---------------------------------------------------------------------------
__host__ __device__ __forceinline__ int work_tiles_per_group(const AttnArgs& a, int n_sub) {
  return (a.cu_q && n_sub % 4 == 2) ? 2 : 1;
}
// tpg is 1 or 2.
__host__ __device__ __forceinline__ int padded_tiles(int n_tiles, int tpg) { return (n_tiles + tpg - 1) & -tpg; }

// Query heads per workgroup of the forward and dQ kernels.  The 256 query
// rows of a workgroup are either 256 rows of one query head or, when the GQA
// group size is even, the same 128 rows of two query heads that read the same
// K/V head (one half of the waves one head, the other half the other).  Under
// a causal mask a workgroup's key range then ends where its last query row's
// does for both halves, instead of two 64-key tiles later than the first half
// needs (forward 1.4-1.9% faster at N = 8192, 13% at N = 512, batch 8).  A
// packed batch pairs heads only when the group size is a multiple of 4, so
// that each (unit, tile) keeps an even number of workgroups (decode_work: with
// one per (unit, tile) a packed batch of G = 2 ran 5% slower).
__host__ __device__ __forceinline__ int heads_per_workgroup(const AttnArgs& a) {
  return (a.G % (a.cu_q ? 4 : 2) == 0) ? 2 : 1;
}

__device__ __forceinline__ WorkItem decode_work(int w, int n_units, int n_tiles, int n_sub,
                                                bool heavy_last_first, bool xcd_remap, int tpg = 1) {
  WorkItem it;
  int t, per, xcd = 0;
  if (xcd_remap) {
    xcd = w & 7;
    const int slot = w >> 3;
    per = n_units >> 3;  // units per XCD (host guarantees n_units % 8 == 0)
    it.sub = slot % n_sub;
    t = slot / n_sub;
  } else {
    per = n_units;
    it.sub = w % n_sub;
    t = w / n_sub;
  }
  const int t1 = t & (tpg - 1), r = t >> (tpg >> 1);  // tpg is 1 or 2
  const int g = r / per;  // tile group
  const int tr = g * tpg + ((g & 1) ? (tpg - 1 - t1) : t1);
  it.unit = xcd_remap ? (r % per) * 8 + xcd : r % per;
  it.tile = heavy_last_first ? (n_tiles - 1 - tr) : tr;
  return it;
}

// ---------------------------------------------------------------------------
// Longest first for the key tiles of packed causal batches (no left window),
// in the dK/dV kernel.  Tile t (TILE keys) of a sequence of lq queries and lk
// keys is seen by max(0, lq - max(0, TILE*t - delta)) queries, delta = lk - lq,
// so the key tiles of a packed batch differ in work with their sequence's
// lengths, and the grid, sized by the longest sequence, holds many slots past
// a short sequence's end.  Slot s of an XCD (workgroup ids go round-robin over
// the 8 XCDs) therefore takes the s-th heaviest (unit, tile) pair of the units
// that XCD holds -- ties by unit, then tile, ascending -- and slots past the
// last pair leave at once, after all the work.  A tile that no query sees
// still runs (it writes zeros).  The pair is found by bisection on the work,
// one unit per lane (at most 64 units per XCD); every wave of a workgroup
// finds the same pair.  Returns false for a slot past the last pair.  (The
// forward and dQ kernels keep the tile-index order of decode_work: their
// tiles' work grows with the tile index alone, and the same bisection there
// ran the packed forward 2.7% slower.)
// ---------------------------------------------------------------------------
template <int TILE>
__device__ __forceinline__ bool lpt_causal_key_tile(const AttnArgs& a, int w, int n_units, int& unit, int& tile) {
  const int xcd = w & 7, s = w >> 3, per = n_units >> 3;
  const int lane = threadIdx.x & 63;
  int lq = 0, lk = 0, nt = 0;
  if (lane < per) {
    const int b = (lane * 8 + xcd) / a.Hkv;  // the lengths bind_seq gives the sequence
    const int q0 = min(max(a.cu_q[b], 0), a.total_q), q1 = min(max(a.cu_q[b + 1], q0), a.total_q);
    const int k0 = min(max(a.cu_k[b], 0), a.total_k), k1 = min(max(a.cu_k[b + 1], k0), a.total_k);
    lq = min(q1 - q0, a.Nq);
    lk = min(k1 - k0, a.Nk);
    nt = (lk + TILE - 1) / TILE;
  }
  const int delta = lk - lq;
  // Tiles of this lane's unit seen by at least W queries (W >= 0).
  auto count = [&](int W) -> int {
    const int e = lq - W + delta;
    return (lane < per && W <= lq && e >= 0) ? min(nt, e / TILE + 1) : 0;
  };
  constexpr unsigned long long kAll = ~0ull;
  if (__reduce_add_sync(kAll, count(0)) <= s) return false;
  int lo = 0, hi = a.Nq + 1;  // pairs of work >= lo exceed s; of work >= hi do not
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (__reduce_add_sync(kAll, count(mid)) > s)
      lo = mid;
    else
      hi = mid;
  }
  // The s-th pair has work lo; idx is its rank among the pairs of that work.
  int idx = s - __reduce_add_sync(kAll, count(lo + 1));
  const int neq = count(lo) - count(lo + 1);
  for (int u = 0; u < per; ++u) {
    const int n = __builtin_amdgcn_readlane(neq, u);
    if (idx < n) {
      const int lq_u = __builtin_amdgcn_readlane(lq, u), d_u = __builtin_amdgcn_readlane(delta, u);
      unit = u * 8 + xcd;
      // Work lq (or 0 for a unit without queries) is taken by the tiles from 0
      // up to delta / TILE; any other work by exactly one tile.
      tile = (lo == lq_u) ? idx : (lq_u - lo + d_u) / TILE;
      return true;
    }
    idx -= n;
  }
  return false;
}

}  // namespace fa
