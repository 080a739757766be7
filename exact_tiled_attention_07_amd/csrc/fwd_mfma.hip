// Forward attention for fp16/bf16 on gfx950 with 32x32x16 MFMA.
//
// The method ([P4] "FlashAttention 实战指南", section "长序列注意力为什么会爆内存"):
// Q, K and V are cut into tiles; one tile of queries stays on chip while K/V
// tiles stream through LDS; each K/V tile's scores and softmax are computed on
// chip, and an online softmax keeps the running row maximum and row sum so
// that the full score matrix never exists.  The output is the exact attention
// result; the kernel also writes the per-row log-sum-exp for the backward pass.
//
// gfx950 mapping.  One workgroup = 8 waves = 256 query rows: a tile of 256
// queries of one (batch, query head), or of 128 queries of two query heads
// that share a K/V head; each wave owns 32 query rows.  For every K/V tile of
// BN keys:
//   S^T (BN x 32) = K Q^T      A operand = K rows from LDS, B = Q (registers)
//   online softmax             lane l holds query l%32 and 16 keys per 32x32
//                              block, so row max/sum are in-register plus one
//                              exchange with lane l^32
//   O^T (D x 32) += V^T P^T    A operand = V^T read transposed from the
//                              row-major V tile, B = P^T from the softmax
// The O rescale by exp(m_old - m_new) is a per-lane scalar (one query per lane).
// Scores are kept in raw units; exp(scale*(s - m)) is evaluated as
// exp2(s*c - m*c) with c = scale*log2(e), one FMA and one v_exp_f32.
// K and V tiles sit in LDS row-major with a chunk swizzle (tile_io.hpp) and
// arrive by direct-to-LDS loads.  The two halves of the workgroup alternate
// between matrix products and softmax (below), so that on every SIMD one wave
// keeps the matrix core busy while the other does the vector work.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "tile_io.hpp"

namespace fa {

// Largest growth of the row maximum (in log2 units) absorbed without
// rescaling O and l: until the maximum has grown by more than this, the stale
// maximum keeps being the reference, so probabilities stay below 2^kLazyRescale.
// O and l always share the same reference, so the result is unchanged.
static constexpr float kLazyRescale = 8.0f;
// A lane's share of a tile's row sum below this bound proves that none of its
// probabilities exceeds 2^kLazyRescale (2^8 less 1/1024 of it, well beyond the
// rounding of the exponent and of exp2).
static constexpr float kLazyBound = 256.0f - 0.25f;

// Launch configuration (tuned on MI355X; overridable at build time).
#ifndef FA_FWD_BN
#define FA_FWD_BN 64  // keys per K/V tile
#endif
#ifndef FA_FWD_RING
#define FA_FWD_RING 3  // LDS operands in flight ahead of the MFMA that uses them
#endif


// ---------------------------------------------------------------------------
// Forward with two wave groups in ping-pong.
//
// Waves 0-3 (group A) and 4-7 (group B) each own 32 queries; waves w and w+4
// share a SIMD.  Per K/V tile m the work of a wave is an MFMA interval
// (O += V(m-1)^T P(m-1)^T, then S(m) = K(m) Q^T)
// and a softmax interval (mask, row max, lazy rescale, P = exp2(...)).
// Group B runs half a tile behind group A, with a barrier between intervals:
//     interval 2m:    A  MFMA(m)        B  softmax(m-1)
//     interval 2m+1:  A  softmax(m)     B  MFMA(m)
// so on every SIMD one wave feeds the matrix core while the other does the
// softmax.  K(m) is read in intervals 2m and 2m+1, V(m) in 2m+2 and 2m+3,
// each from two LDS buffers.  The tile loads are split between the groups so
// that neither MFMA interval carries all of their issue cost: group A loads
// K(m+1) at the end of its MFMA interval 2m, group B loads V(m+1) at the end
// of its MFMA interval 2m+1 (both after the interval's last transposing read,
// which the compiler would otherwise hold for the loads), each into a buffer
// whose last reader has finished, and each group waits for its loads at the
// end of its next (softmax) interval.
// ---------------------------------------------------------------------------
template <class T, int D, int BN, bool MOD>
struct FwdPP {
  static constexpr int NW = 8, HALF = 4;
  static constexpr int TILE = BN * D;  // elements of one K or V tile
  uint16_t* kbuf;                      // [2][TILE], swizzled row-major
  uint16_t* vbuf;                      // [2][TILE]
  const uint16_t* Kp;
  const uint16_t* Vp;
  int64_t k_sn, v_sn;
  int Nk, t_lo, n, lo_i, hi_i, lo_max, hi_min, wave, lane, hf;
  float c;
  u32x4 qf[D / 16];
  int kro[D / 16];     // per-lane LDS offsets of the K row chunks
  int vro[D / 32][2];  // per-lane LDS offsets of the transposing V reads
  DmaTile<D, BN, HALF> kd, vd;  // group A's shares of the K and V tile loads
  float mref, l;
  float cap, slope_r, dist0;  // score modifiers (MOD): clamp, raw slope, i' - 4*hf of this lane
  f32x16 oacc[D / 32];
  f32x16 s[BN / 32];  // scores of tile m between its MFMA and softmax intervals
  u32x4 ring[FA_FWD_RING];  // LDS operands in flight (the first NB - 1 read before the interval's barrier)
  u32x4 pf[BN / 16];  // P^T of tile m between its softmax and the next MFMA interval

  static constexpr int NPV = (BN / 16) * (D / 32), NS = (D / 16) * (BN / 32);

  // Operand o of an MFMA interval: o < NPV are the V^T operands of
  // O^T += V^T P^T (16-key step si = o / (D/32), column block db = o % (D/32)),
  // read transposed from the row-major V tile; the rest are the K row chunks
  // of S^T = K Q^T (step st, key block kb).
  __device__ __forceinline__ u32x4 operand(const char* Vs, const char* Ks, int o) const {
    if (o < NPV) {
      const int si = o / (D / 32), db = o % (D / 32);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Vs + si * 16 * 2 * D + vro[db][0]));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Vs + si * 16 * 2 * D + vro[db][1]));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      return u32x4{l2[0], l2[1], h2[0], h2[1]};
    }
    const int st = (o - NPV) / (BN / 32), kb = (o - NPV) % (BN / 32);
    return *reinterpret_cast<const u32x4*>(Ks + kb * 32 * 2 * D + kro[st]);
  }

  // MFMA interval of tile m (relative to t_lo); PAR = m & 1.  PV: run
  // O += V(m-1)^T P(m-1)^T (false in interval 0, where there is no tile -1);
  // SP: run S(m) = K(m) Q^T (false in interval n, after the last tile).  The
  // skipped products would add zeros to O, or scores that are never used.
  // Each LDS operand is read NB - 1 MFMAs ahead of its use.
  // s[kb][r] is key j0 + 32*kb + 8*(r/4) + 4*hf + r%4.
  template <int PAR, bool PV, bool SP>
  __device__ __forceinline__ void mfma_interval(int m, bool group_a) {
    constexpr int NB = FA_FWD_RING, O0 = PV ? 0 : NPV, O1 = SP ? NPV + NS : NPV;
    static_assert(NPV >= NB && NS >= NB, "interval shape");
    const char* Vs = reinterpret_cast<const char*>(vbuf + (1 - PAR) * TILE);
    const char* Ks = reinterpret_cast<const char*>(kbuf + PAR * TILE);
    if constexpr (SP) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) s[kb] = f32x16{};
    }
#pragma unroll
    for (int o = O0; o < O1; ++o) {
      if (o + NB - 1 < O1) ring[(o + NB - 1) % NB] = operand(Vs, Ks, o + NB - 1);
      __builtin_amdgcn_sched_barrier(0);
      if (o < NPV) {
        const int si = o / (D / 32), db = o % (D / 32);
        oacc[db] = T::mfma(ring[o % NB], pf[si], oacc[db]);
      } else {
        const int st = (o - NPV) / (BN / 32), kb = (o - NPV) % (BN / 32);
        s[kb] = T::mfma(ring[o % NB], qf[st], s[kb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // Tile loads, after the last transposing read of the interval (issued in
    // one burst: spread between the S products they stall them).  Group A
    // loads K(m+1) into the K buffer read in intervals 2m-2 and 2m-1; group B
    // loads V(m+1) into the V buffer whose last reader is this very interval
    // (B's product with V(m-1); A's was in interval 2m).
    if (group_a) {
      if (m + 1 < n) kd.issue_nonempty(Kp, k_sn, (t_lo + m + 1) * BN, Nk, kbuf + (1 - PAR) * TILE);
    } else {
      if (m + 1 < n) vd.issue_nonempty(Vp, v_sn, (t_lo + m + 1) * BN, Nk, vbuf + (1 - PAR) * TILE);
    }
  }

  // The first NB - 1 operands of the next MFMA interval (buffer parity PAR;
  // PV as in mfma_interval), read before the barrier that opens it, so that
  // its first MFMA does not wait out an LDS round trip after the barrier.
  // They come from tiles that an earlier barrier published.
  template <int PAR, bool PV>
  __device__ __forceinline__ void prefetch() {
    constexpr int NB = FA_FWD_RING, O0 = PV ? 0 : NPV;
    const char* Vs = reinterpret_cast<const char*>(vbuf + (1 - PAR) * TILE);
    const char* Ks = reinterpret_cast<const char*>(kbuf + PAR * TILE);
#pragma unroll
    for (int o = O0; o < O0 + NB - 1; ++o) ring[o % NB] = operand(Vs, Ks, o);
  }

  // Softmax interval of tile m: mask, row max, lazy rescale of O and l, P.
  __device__ __forceinline__ void softmax_interval(int m) {
    if (m < 0 || m >= n) return;
    const int j0 = (t_lo + m) * BN;
    if constexpr (MOD) {
      // s[kb][r] is key j0 + 32*kb + 8*(r/4) + 4*hf + r%4; dist0 = i' - 4*hf.
      const float base = dist0 - (float)j0;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[kb][r] = mod_score(s[kb][r], cap, slope_r, base - (float)(32 * kb + 8 * (r >> 2) + (r & 3)));
      }
    }
    const bool full = (j0 >= lo_max) && (j0 + BN - 1 <= hi_min);
    if (!full) {
      // Element key j = kbase + k_r (k_r a constant of the register) is
      // visible iff (j - lo) | (hi - j) has its sign bit clear; the sign bit,
      // spread over the word, selects -inf (bit pattern 0xff800000) with one
      // bitfield insert.  No lane masks are held in scalar registers.
      // (j0 passes through an empty asm so that the compiler does not turn
      // a0 and b0 into per-lane induction variables stepped on every tile,
      // which would put vector adds into the MFMA interval's load block.)
      int jj = j0;
      asm volatile("" : "+s"(jj));
      const int kbase = jj + 4 * hf;
      const int a0 = kbase - lo_i, b0 = hi_i - kbase;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kr = 32 * kb + 8 * (r >> 2) + (r & 3);
          const uint32_t out = (uint32_t)(((a0 + kr) | (b0 - kr)) >> 31);
          s[kb][r] = __uint_as_float((out & 0xff800000u) | (~out & __float_as_uint(s[kb][r])));
        }
      }
    }
    // The reference maximum moves only when some row of the wave grew by more
    // than 2^kLazyRescale; then O and l (which hold the tiles up to m - 1) are
    // rescaled.  P is first computed against the current reference: if every
    // lane's share of the tile's row sum stays below kLazyBound, no probability
    // exceeds 2^kLazyRescale, so no row maximum grew that far and the reference
    // and P stand.  Otherwise (or while some row has no reference yet) the row
    // maximum decides exactly as it would have up front, and P is recomputed
    // if the reference moved.  The bound sits a little below 2^kLazyRescale so
    // that the rounding of the two tests can never let a rescale slip through.
    // With score modifiers (a steep ALiBi slope moves the maximum on every
    // tile, and the clamp and distance make the vector work the longer half
    // of the interval) the row maximum is always taken first, so that P is
    // computed once.  Both orders take the same decisions.
    float ls = 0.f;
    bool check = true;
    if constexpr (!MOD) {
      ls = exp_pack(mref);
      check = __any(!(ls <= kLazyBound) || mref == -INFINITY);
    }
    if (check) {
      // Row maximum: four independent chains, then the lane pair.
      float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) m4[r & 3] = fmaxf(m4[r & 3], s[kb][r]);
      }
      const float mx = max_xor32(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
      if (__any((mx - mref) * c > kLazyRescale)) {  // false for NaN (both -inf)
        const float m_new = fmaxf(mref, mx);
        const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2((mref - m_new) * c);
        mref = m_new;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
        if constexpr (!MOD) ls = exp_pack(mref);
      }
    }
    if constexpr (MOD) ls = exp_pack(mref);
    l += ls;
  }

  // P^T = exp2(s*c - ref*c) rounded into pf; returns this lane's share of the
  // tile's row sum (of the unrounded probabilities), in four partial sums.
  __device__ __forceinline__ float exp_pack(float ref) {
    const float mc = (ref == -INFINITY) ? 0.f : ref * c;
    float l4[4];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = fast_exp2(fmaf(s[kb][8 * tt + e], c, -mc));
          if (kb == 0 && tt == 0 && e < 4)
            l4[e] = p[e];
          else
            l4[e & 3] += p[e];
        }
        pf[2 * kb + tt] = u32x4{T::pack(p[0], p[1]), T::pack(p[2], p[3]), T::pack(p[4], p[5]), T::pack(p[6], p[7])};
      }
    }
    return (l4[0] + l4[1]) + (l4[2] + l4[3]);
  }
};

template <class T, int D, int BN, bool MOD>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_pp_kernel(AttnArgs a) {
  using Ctx = FwdPP<T, D, BN, MOD>;
  constexpr int NW = Ctx::NW, BM = NW * 32, TILE = Ctx::TILE;
  __shared__ __attribute__((aligned(16))) uint16_t kbuf[2 * TILE];
  __shared__ __attribute__((aligned(16))) uint16_t vbuf[2 * TILE];
  static_assert(2 * TILE * 2 <= 65536, "LDS offsets of one buffer pair must fit the 16-bit immediate");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const bool group_a = wave < Ctx::HALF;

  // With an even GQA group the two wave groups take the same 128 query rows
  // of two query heads that share the K/V head (heads_per_workgroup).
  const int hp = heads_per_workgroup(a);
  const int lg_rows = (hp == 2) ? 7 : 8;                 // query rows per head: BM / hp
  static_assert(BM == 256, "rows per head are 256 or 128");
  const int wr = (hp == 2) ? (wave & (Ctx::HALF - 1)) : wave;  // row block of this wave
  const int n_sub = a.G >> (hp - 1);
  const int tpg = work_tiles_per_group(a, n_sub);
  const int n_qt = padded_tiles((a.Nq + (1 << lg_rows) - 1) >> lg_rows, tpg);
  const bool heavy_last = (a.causal || a.wr >= 0) && a.wl < 0;
  const WorkItem it = decode_work(blockIdx.x, a.B * a.Hkv, n_qt, n_sub, heavy_last, a.xcd_remap, tpg);
  const int b = it.unit / a.Hkv, hk = it.unit % a.Hkv;
  // (wave-uniform: read from the first lane, so that the head's pointers stay scalar)
  const int hq = hk * a.G + it.sub * hp + ((hp == 2) ? (__builtin_amdgcn_readfirstlane(wave) / Ctx::HALF) : 0);
  const int q0 = it.tile << lg_rows;
  const int qrow = q0 + wr * 32 + l32;  // the query of this lane's column
  bind_seq(a, b);
  if (q0 >= a.Nq) return;  // past the end of a shorter packed sequence (whole workgroup)

  Ctx x;
  x.kbuf = kbuf;
  x.vbuf = vbuf;
  x.Kp = static_cast<const uint16_t*>(a.k) + b * a.k_sb + hk * a.k_sh;
  x.Vp = static_cast<const uint16_t*>(a.v) + b * a.v_sb + hk * a.v_sh;
  x.k_sn = a.k_sn;
  x.v_sn = a.v_sn;
  x.Nk = a.Nk;
  x.wave = wave;
  x.lane = lane;
  x.hf = hf;
  x.c = a.scale_log2;
  if constexpr (MOD) {
    x.cap = a.cap;
    x.slope_r = alibi_raw_uniform(a.alibi, a.alibi_sb, a.inv_scale, b, hq);
    x.dist0 = (float)(qrow + a.delta - 4 * hf);
  }
  const uint16_t* Qp = static_cast<const uint16_t*>(a.q) + b * a.q_sb + hq * a.q_sh;

  // Q as the B operand of S^T = K Q^T: lane holds d = 16*st + 8*hf + (0..7)
  // (zeros past a head dim below D).
  if (qrow < a.Nq) {
    const uint16_t* qr = Qp + (int64_t)qrow * a.q_sn;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) x.qf[st] = load_cols(qr, 16 * st + 8 * hf, a.D);
  } else {
#pragma unroll
    for (int st = 0; st < D / 16; ++st) x.qf[st] = u32x4{0u, 0u, 0u, 0u};
  }

  // Visible keys of this lane's query, and the workgroup's key tiles.
  x.lo_i = key_lo(a, qrow);
  x.hi_i = key_hi(a, qrow);
  const int q_last = min(q0 + (1 << lg_rows), a.Nq) - 1;
  const int kv_lo = key_lo(a, q0), kv_hi = key_hi(a, q_last);
  // Tiles that every query of this wave sees in full skip the element mask.
  const int wq0 = q0 + 32 * __builtin_amdgcn_readfirstlane(wr);
  x.lo_max = key_lo(a, min(wq0 + 31, a.Nq - 1));
  x.hi_min = key_hi(a, wq0);
  x.t_lo = kv_lo / BN;
  x.n = (kv_hi >= kv_lo) ? kv_hi / BN - x.t_lo + 1 : 0;

  // Per-lane LDS byte offsets, fixed for the whole kernel.
#pragma unroll
  for (int st = 0; st < D / 16; ++st) x.kro[st] = Swz<D>::off(l32, 2 * st + hf);
  {
    const int G = lane >> 4, j = lane & 15;
    const int vhf = G >> 1, gsub = G & 1, ep = j >> 2, q = j & 3;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int cc = 4 * db + 2 * gsub + (q >> 1);
      x.vro[db][0] = Swz<D>::off(4 * vhf + ep, cc) + 8 * (q & 1);
      x.vro[db][1] = Swz<D>::off(8 + 4 * vhf + ep, cc) + 8 * (q & 1);
    }
  }

  x.mref = -INFINITY;
  x.l = 0.f;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) x.oacc[db] = f32x16{};

  // Group A loads the K tiles, group B the V tiles; K(0) and V(0) here.
  x.kd.init(wave % Ctx::HALF, lane, a.k_sn, a.D / 8);
  x.vd.init(wave % Ctx::HALF, lane, a.v_sn, a.D / 8);
  if (x.n > 0) {
    if (group_a)
      x.kd.issue(x.Kp, a.k_sn, x.t_lo * BN, a.Nk, kbuf);
    else
      x.vd.issue(x.Vp, a.v_sn, x.t_lo * BN, a.Nk, vbuf);
    wait_all_loads();
  }
  __syncthreads();

  // 2(n+1) intervals; both groups pass the same barriers.  Interval 0 runs
  // only S(0) and interval n only the last P V product; m is odd in the tail.
  const int n = x.n;
  if (n > 0) {
    int m = 1;
    if (group_a) {
      x.template prefetch<0, false>();
      x.template mfma_interval<0, false, true>(0, true);
      lds_barrier();
      x.softmax_interval(0);
      wait_all_loads();
      x.template prefetch<1, true>();
      lds_barrier();
      for (; m + 1 < n; m += 2) {
        x.template mfma_interval<1, true, true>(m, true);
        lds_barrier();
        x.softmax_interval(m);
        wait_all_loads();
        x.template prefetch<0, true>();
        lds_barrier();
        x.template mfma_interval<0, true, true>(m + 1, true);
        lds_barrier();
        x.softmax_interval(m + 1);
        wait_all_loads();
        x.template prefetch<1, true>();
        lds_barrier();
      }
      if (m == n) {
        x.template mfma_interval<1, true, false>(m, true);
        lds_barrier();
        wait_all_loads();
        lds_barrier();
      } else {
        x.template mfma_interval<1, true, true>(m, true);
        lds_barrier();
        x.softmax_interval(m);
        wait_all_loads();
        x.template prefetch<0, true>();
        lds_barrier();
        x.template mfma_interval<0, true, false>(n, true);
        lds_barrier();
        wait_all_loads();
        lds_barrier();
      }
    } else {
      wait_all_loads();
      x.template prefetch<0, false>();
      lds_barrier();
      x.template mfma_interval<0, false, true>(0, false);
      lds_barrier();
      for (; m + 1 < n; m += 2) {
        x.softmax_interval(m - 1);
        wait_all_loads();
        x.template prefetch<1, true>();
        lds_barrier();
        x.template mfma_interval<1, true, true>(m, false);
        lds_barrier();
        x.softmax_interval(m);
        wait_all_loads();
        x.template prefetch<0, true>();
        lds_barrier();
        x.template mfma_interval<0, true, true>(m + 1, false);
        lds_barrier();
      }
      x.softmax_interval(m - 1);
      wait_all_loads();
      x.template prefetch<1, true>();
      lds_barrier();
      if (m == n) {
        x.template mfma_interval<1, true, false>(m, false);
        lds_barrier();
      } else {
        x.template mfma_interval<1, true, true>(m, false);
        lds_barrier();
        x.softmax_interval(m);
        wait_all_loads();
        x.template prefetch<0, true>();
        lds_barrier();
        x.template mfma_interval<0, true, false>(n, false);
        lds_barrier();
      }
    }
  }

  // Epilogue: O = O / l, LSE = scale*mref + ln(l).  Lanes l and l^32 hold
  // different keys of the same query, so their partial sums are added here.
  const float lt = sum_xor32(x.l);
  const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
  if (qrow < a.Nq) {
    uint16_t* op = static_cast<uint16_t*>(a.o) + b * a.o_sb + hq * a.o_sh + (int64_t)qrow * a.o_sn;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * db + 8 * g4 + 4 * hf;
        const u32x2 w{T::pack(x.oacc[db][4 * g4] * inv, x.oacc[db][4 * g4 + 1] * inv),
                      T::pack(x.oacc[db][4 * g4 + 2] * inv, x.oacc[db][4 * g4 + 3] * inv)};
        if (d0 < a.D) *reinterpret_cast<u32x2*>(op + d0) = w;
      }
    }
    if (hf == 0)
      a.lse[b * a.lse_sb + hq * a.lse_sh + qrow] = (lt > 0.f) ? (x.mref * a.scale + logf(lt)) : -INFINITY;
  }
}

template <class T, int D, int BN, int NW>
static hipError_t launch_fwd_t(const AttnArgs& a, hipStream_t stream) {
  constexpr int BM = NW * 32;
  const int hp = heads_per_workgroup(a);
  const int n_qt = padded_tiles((a.Nq + BM / hp - 1) / (BM / hp), work_tiles_per_group(a, a.G / hp));
  const int64_t total = (int64_t)a.B * a.Hkv * n_qt * (a.G / hp);
  if (total == 0) return hipSuccess;
  AttnArgs args = a;
  args.xcd_remap = a.xcd_remap && ((a.B * a.Hkv) % 8 == 0);
  static_assert(NW == FwdPP<T, D, BN, false>::NW, "the forward runs 8 waves");
  if (a.mod)
    hipLaunchKernelGGL((fwd_pp_kernel<T, D, BN, true>), dim3((unsigned)total), dim3(NW * 64), 0, stream, args);
  else
    hipLaunchKernelGGL((fwd_pp_kernel<T, D, BN, false>), dim3((unsigned)total), dim3(NW * 64), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_fwd_mfma(const AttnArgs& a, hipStream_t stream) {
  // Head dims below 64 / 128 run the 64 / 128 kernels with the rest masked.
  if (a.dtype == kBF16) {
    if (a.D > 64 && a.D <= 128) return launch_fwd_t<BF16, 128, FA_FWD_BN, 8>(a, stream);
    if (a.D >= 8 && a.D <= 64) return launch_fwd_t<BF16, 64, FA_FWD_BN, 8>(a, stream);
  } else if (a.dtype == kF16) {
    if (a.D > 64 && a.D <= 128) return launch_fwd_t<F16, 128, FA_FWD_BN, 8>(a, stream);
    if (a.D >= 8 && a.D <= 64) return launch_fwd_t<F16, 64, FA_FWD_BN, 8>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
