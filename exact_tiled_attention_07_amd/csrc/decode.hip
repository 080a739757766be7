// Attention against a KV cache with a split key range ("incremental decoding",
// [P4] "FlashAttention 实战指南", section "增量解码场景flash_attn_with_kvcache":
// the new keys and values are appended to the cache in place, cache_seqlens
// gives each batch entry's valid length, and num_splits divides the key range
// so that few queries against a long cache still fill the GPU).
//
// For batch entry b with L_b = cache_seqlens[b] valid rows:
//   append   k_new[b, i] -> k_cache[b, L_b + i], same for v (i < Nq), when
//            new keys are given; the key count is then Lk_b = L_b + Nq, else
//            Lk_b = L_b (both clamped to the cache capacity);
//   attend   the Nq queries of b to cache rows [0, Lk_b) with the same mask
//            rule as the main path, queries aligned to the end of the keys
//            (i' = i + Lk_b - Nq).
//
// Two kernels:
//   kv_split    one wave per (batch, kv head, block of 32 query rows, part):
//               the G query heads x Nq queries of a K/V head are packed as the
//               32 columns of S^T = K Q^T, so every K/V row read from HBM serves
//               all of them.  K and V go through the wave's own LDS tiles.  No
//               barriers: each wave only reads what it wrote.  The visible key
//               tiles of the wave's rows are cut into S contiguous runs of
//               equal length, one per part; each part writes its O / l and
//               LSE (float32) to the workspace.  Keys at or past L_b come straight
//               from k_new / v_new, so the in-place append can run in the same
//               launch: the waves after the split waves copy the new rows into
//               the cache (16 bytes per lane), and no split wave reads them
//               there;
//   kv_merge    per query row, O = sum_s exp(LSE_s - LSE) O_s with
//               LSE = ln sum_s exp(LSE_s) (empty parts weigh 0).
#include "common.hpp"
#include "launch.hpp"
#include "tile_io.hpp"

namespace fa {

// ---------------------------------------------------------------------------
// Append: k_new[b, i, h] -> k_cache[b, L_b + i, h] for L_b + i < capacity.
// Chunk idx of 2 * B * Nq * Hkv * (D / 8) 16-byte chunks (keys, then values).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void kv_append_chunk(const KvArgs& k, int64_t idx) {
  const int cpr = k.D * 2 / 16;  // 16-byte chunks per row
  const int64_t per_tensor = (int64_t)k.B * k.Nq * k.Hkv * cpr;
  if (idx >= 2 * per_tensor) return;
  const int which = idx >= per_tensor;  // 0: keys, 1: values
  int64_t r = which ? idx - per_tensor : idx;
  const int c = (int)(r % cpr);
  r /= cpr;
  const int h = (int)(r % k.Hkv);
  r /= k.Hkv;
  const int i = (int)(r % k.Nq);
  const int b = (int)(r / k.Nq);
  const int L = min(max(k.cache_seqlens[b], 0), k.cap);
  const int dst_row = L + i;
  if (dst_row >= k.cap) return;
  const char* src = static_cast<const char*>(which ? k.v_new : k.k_new) +
                    2 * (b * (which ? k.vn_sb : k.kn_sb) + (int64_t)i * (which ? k.vn_sn : k.kn_sn) +
                         h * (which ? k.vn_sh : k.kn_sh)) + 16 * c;
  // Contiguous caches: entry b, row dst_row.  Paged: page of dst_row, row in it.
  int64_t blk = b, row = dst_row;
  if (k.page_size) {
    blk = min(max(k.block_table[b * k.bt_sb + dst_row / k.page_size], 0), k.num_pages - 1);
    row = dst_row % k.page_size;
  }
  char* dst = static_cast<char*>(which ? k.v_cache : k.k_cache) +
              2 * (blk * (which ? k.vc_sb : k.kc_sb) + row * (which ? k.vc_sn : k.kc_sn) +
                   h * (which ? k.vc_sh : k.kc_sh)) + 16 * c;
  *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
}

// Visible key interval [lo, hi] of query i of batch entry b (Lk keys).
__device__ __forceinline__ void kv_row_range(const KvArgs& k, int i, int Lk, int& lo, int& hi) {
  const int ip = i + Lk - k.Nq;
  lo = 0;
  hi = Lk - 1;
  if (k.causal) hi = min(hi, ip);
  if (k.wl >= 0) lo = max(lo, ip - k.wl);
  if (k.wr >= 0) hi = min(hi, ip + k.wr);
}

// ---------------------------------------------------------------------------
// Split decode.  Lane (l32, hf) owns query row R = 32*rb + l32 of the packed
// G x Nq rows (head g = R / Nq, query i = R % Nq); per tile of 32 keys
//   S^T (32 keys x 32 rows) = K Q^T   A = K rows, B = Q rows (registers)
//   online softmax per lane (row), with the forward's lazy rescale
//   O^T (D x 32 rows) += V^T P^T      A = V^T from the wave's LDS tile
// K and V tiles are read with coalesced 16-byte loads (four 256-byte rows
// per instruction at D = 128), KV_DEPTH tiles ahead of their use, and go
// through the wave's own swizzled LDS tiles: K is read back as row operands,
// V transposed.
// ---------------------------------------------------------------------------
static constexpr float kKvLazyRescale = 8.0f;
#ifndef FA_KV_DEPTH
#define FA_KV_DEPTH 1
#endif
#ifndef FA_KV_WAVES
#define FA_KV_WAVES 2  // minimum waves per SIMD the register allocation must allow
#endif

template <int D>
struct KvStage {
  static constexpr int CPL = 32 * D * 2 / 16 / 64;  // 16-byte chunks per lane of a 32-row tile
  u32x4 kr[CPL];
  u32x4 vr[CPL];
};

template <class T, int D, int DEPTH, bool MOD, bool PAGED>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(FA_KV_WAVES))) void kv_split_kernel(KvArgs k) {
  constexpr int NST = D / 16;  // 16-wide d steps
  constexpr int CPL = KvStage<D>::CPL;
  __shared__ __attribute__((aligned(16))) uint16_t vt[32 * D];
  __shared__ __attribute__((aligned(16))) uint16_t kt[32 * D];

  const int lane = threadIdx.x, l32 = lane & 31, hf = lane >> 5;
  if ((int)blockIdx.x >= k.n_split) {  // append waves
    kv_append_chunk(k, ((int64_t)blockIdx.x - k.n_split) * 64 + lane);
    return;
  }
  // blockIdx.x = ((b * Hkv + hk) * n_rb + rb) * S + s
  int w = blockIdx.x;
  const int s = w % k.S;
  w /= k.S;
  const int rb = w % k.n_rb;
  w /= k.n_rb;
  const int hk = w % k.Hkv;
  const int b = w / k.Hkv;

  const int rows = k.G * k.Nq;
  const int R = 32 * rb + l32;
  const bool valid = R < rows;
  const int g = valid ? R / k.Nq : 0, i = valid ? R % k.Nq : 0;
  const int hq = hk * k.G + g;
  const int L = min(max(k.cache_seqlens[b], 0), k.cap);  // rows in the cache before the append
  const int Lk = k.append ? min(L + k.Nq, k.cap) : L;

  int lo_r = 0, hi_r = -1;
  if (valid) kv_row_range(k, i, Lk, lo_r, hi_r);
  // Key range of the wave's rows, split into S contiguous tile shares.
  const int rlo = valid && hi_r >= lo_r ? lo_r : 0x7fffffff;
  const int rhi = valid && hi_r >= lo_r ? hi_r : -1;
  int wlo = rlo, whi = rhi;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    wlo = min(wlo, __shfl_xor(wlo, o, 64));
    whi = max(whi, __shfl_xor(whi, o, 64));
  }
  int t_beg = 0, t_end = 0;
  if (whi >= wlo) {
    const int t0 = wlo / 32, t1 = whi / 32 + 1;
    const int per = (t1 - t0 + k.S - 1) / k.S;
    t_beg = min(t0 + s * per, t1);
    t_end = min(t_beg + per, t1);
  }

  // Q rows as B operands: lane holds d = 16*st + 8*hf + (0..7) of its row.
  u32x4 qf[NST];
  if (valid) {
    const uint16_t* qr = static_cast<const uint16_t*>(k.q) + b * k.q_sb + (int64_t)i * k.q_sn + hq * k.q_sh;
#pragma unroll
    for (int st = 0; st < NST; ++st) qf[st] = load_cols(qr, 16 * st + 8 * hf, k.D);
  } else {
#pragma unroll
    for (int st = 0; st < NST; ++st) qf[st] = u32x4{0u, 0u, 0u, 0u};
  }

  // Cache base of this (entry, head); paged caches add the page of each tile.
  const uint16_t* Kc = static_cast<const uint16_t*>(k.k_cache) + (PAGED ? 0 : b * k.kc_sb) + hk * k.kc_sh;
  const uint16_t* Vc = static_cast<const uint16_t*>(k.v_cache) + (PAGED ? 0 : b * k.vc_sb) + hk * k.vc_sh;
  // Key j >= L is new row j - L (only when appending: otherwise Lk = L).
  const uint16_t* Kn = static_cast<const uint16_t*>(k.k_new) + b * k.kn_sb + hk * k.kn_sh;
  const uint16_t* Vn = static_cast<const uint16_t*>(k.v_new) + b * k.vn_sb + hk * k.vn_sh;
  auto krow = [&](int j) { return j < L ? Kc + (int64_t)j * k.kc_sn : Kn + (int64_t)(j - L) * k.kn_sn; };
  auto vrow = [&](int j) { return j < L ? Vc + (int64_t)j * k.vc_sn : Vn + (int64_t)(j - L) * k.vn_sn; };
  // Coalesced chunk c of a lane: tile row crow[c], 16-byte column chunk ccol[c];
  // coff[c] is its place in a swizzled LDS tile.
  int crow[CPL], ccol[CPL], coff[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int ch = lane + 64 * c;
    crow[c] = ch / (D / 8);
    ccol[c] = ch % (D / 8);
    coff[c] = Swz<D>::off(crow[c], ccol[c]);
  }
  SwzOffsets<D> off;
  off.init(lane);
  const float cs = k.scale_log2;
  // Score modifiers: this lane's raw slope and i' - 4*hf (query aligned to the end of the keys).
  float slope_r = 0.f, dist0 = 0.f;
  if constexpr (MOD) {
    slope_r = alibi_raw(k.alibi, k.alibi_sb, k.inv_scale, b, hq);
    dist0 = (float)(i + Lk - k.Nq - 4 * hf);
  }

  // Every K/V element is read once: the non-temporal hint keeps the stream
  // from displacing reusable lines (measured 10% faster on MI355X).
  // A lane's column chunk is the same in every row it loads (64 is a multiple
  // of D / 8).  With a head dim below D, a lane whose chunk lies past it loads
  // chunk 0 of the same row instead (valid memory, no select): that copy only
  // meets the zero columns of Q in S and lands in O columns that are never
  // stored.
  static_assert(64 % (D / 8) == 0, "one column chunk per lane");
  const int cload = (lane % (D / 8)) < k.D / 8 ? lane % (D / 8) : 0;
  auto ld = [](const uint16_t* p) -> u32x4 {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  };
  // Tiles that lie wholly in the cache (all but at most the last two of a
  // range) load through buffer resources: one scalar base per tile plus fixed
  // 32-bit lane offsets, which issue without the 64-bit address arithmetic
  // per chunk (and without stalling behind other waves' MFMAs).
  // Chunk c of a lane is row crow[0] + c * (512 / D) of the tile: the lane part
  // of the offset is fixed, the chunk part is a scalar.
  static_assert(64 % (D / 8) == 0, "chunk rows step by a whole number of rows");
  const uint32_t koff = (uint32_t)(crow[0] * k.kc_sn * 2 + 16 * cload);
  const uint32_t voff = (uint32_t)(crow[0] * k.vc_sn * 2 + 16 * cload);
  auto ld_tile = [&](const uint16_t* kb, const uint16_t* vb, KvStage<D>& st) {
    const __amdgpu_buffer_rsrc_t rk = raw_rsrc(kb, (uint32_t)(32 * k.kc_sn * 2));
    const __amdgpu_buffer_rsrc_t rv = raw_rsrc(vb, (uint32_t)(32 * k.vc_sn * 2));
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ks = c * (512 / D) * (int)k.kc_sn * 2, vs = c * (512 / D) * (int)k.vc_sn * 2;
      st.kr[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, (int)koff, ks, kNonTemporal));
      st.vr[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, (int)voff, vs, kNonTemporal));
    }
  };
  // Rows past the end of the keys repeat the last one (their scores are masked).
  auto load_tile = [&](int t, KvStage<D>& st) {
    if constexpr (PAGED) {
      // The 32 rows of a tile lie in one page (page_size is a multiple of 32).
      const int p = (32 * t) / k.page_size;
      const int64_t pg = min(max(k.block_table[b * k.bt_sb + p], 0), k.num_pages - 1);
      const int r0 = p * k.page_size;
      const uint16_t* Kp = Kc + pg * k.kc_sb;
      const uint16_t* Vp = Vc + pg * k.vc_sb;
      if (32 * t + 31 < L) {
        ld_tile(Kp + (int64_t)(32 * t - r0) * k.kc_sn, Vp + (int64_t)(32 * t - r0) * k.vc_sn, st);
        return;
      }
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int j = min(32 * t + crow[c], Lk - 1);
        st.kr[c] = ld((j < L ? Kp + (int64_t)(j - r0) * k.kc_sn : Kn + (int64_t)(j - L) * k.kn_sn) + 8 * cload);
        st.vr[c] = ld((j < L ? Vp + (int64_t)(j - r0) * k.vc_sn : Vn + (int64_t)(j - L) * k.vn_sn) + 8 * cload);
      }
    } else {
      if (32 * t + 31 < L) {
        ld_tile(Kc + (int64_t)(32 * t) * k.kc_sn, Vc + (int64_t)(32 * t) * k.vc_sn, st);
        return;
      }
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int j = min(32 * t + crow[c], Lk - 1);
        st.kr[c] = ld(krow(j) + 8 * cload);
        st.vr[c] = ld(vrow(j) + 8 * cload);
      }
    }
  };

  float mref = -INFINITY, l = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};

  // One tile: stage to LDS, refill the stage with tile t + DEPTH, then the
  // products.  LDS operations of a wave complete in order, so the previous
  // tile's reads are done before these writes land and the writes precede
  // the reads below.
  auto step = [&](int t, KvStage<D>& st) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(vt) + coff[c]) = st.vr[c];
      *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(kt) + coff[c]) = st.kr[c];
    }
    if (t + DEPTH < t_end) load_tile(t + DEPTH, st);
    // S^T = K Q^T; s[r] is key 32t + 8*(r/4) + 4*hf + r%4.
    f32x16 sv = f32x16{};
#pragma unroll
    for (int c = 0; c < NST; ++c) sv = T::mfma(off.row_chunk(reinterpret_cast<const char*>(kt), 0, c), qf[c], sv);
    const int j0 = 32 * t;
    if constexpr (MOD) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sv[r] = mod_score(sv[r], k.score_cap, slope_r, dist0 - (float)(j0 + 8 * (r >> 2) + (r & 3)));
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = j0 + 8 * (r >> 2) + 4 * hf + (r & 3);
      if (key < lo_r || key > hi_r) sv[r] = -INFINITY;
    }
    float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int r = 0; r < 16; ++r) m4[r & 3] = fmaxf(m4[r & 3], sv[r]);
    const float mx = max_xor32(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
    if (__any((mx - mref) * cs > kKvLazyRescale)) {
      const float m_new = fmaxf(mref, mx);
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2((mref - m_new) * cs);
      mref = m_new;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
    }
    const float mc = (mref == -INFINITY) ? 0.f : mref * cs;
    u32x4 pf[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = fast_exp2(fmaf(sv[8 * tt + e], cs, -mc));
        l += p[e];
      }
      pf[tt] = u32x4{T::pack(p[0], p[1]), T::pack(p[2], p[3]), T::pack(p[4], p[5]), T::pack(p[6], p[7])};
    }
    // O^T += V^T P^T.
#pragma unroll
    for (int si = 0; si < 2; ++si) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        oacc[db] = T::mfma(off.tr_operand(reinterpret_cast<const char*>(vt), si, db), pf[si], oacc[db]);
    }
  };

  KvStage<D> stage[DEPTH];
#pragma unroll
  for (int j = 0; j < DEPTH; ++j)
    if (t_beg + j < t_end) load_tile(t_beg + j, stage[j]);
  for (int t = t_beg; t < t_end; t += DEPTH) {
#pragma unroll
    for (int j = 0; j < DEPTH; ++j)
      if (t + j < t_end) step(t + j, stage[j]);
  }

  // Partial result of this part: O / l and LSE (natural log), per row.
  const float lt = sum_xor32(l);
  if (valid) {
    const int64_t row = ((int64_t)(b * k.Hq + hq) * k.Nq + i) * k.S + s;
    if (hf == 0) k.ws_lse[row] = (lt > 0.f) ? (mref * k.scale + logf(lt)) : -INFINITY;
    if (!(lt > 0.f)) return;  // an empty part weighs 0 in the merge, which then never reads its O
    float* po = k.ws_o + row * D;
    const float inv = 1.f / lt;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * db + 8 * g4 + 4 * hf;
        *reinterpret_cast<f32x4*>(po + d0) = f32x4{oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv,
                                                   oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Merge of the parts of one query row, one wave per row.  Lane (cg, ps) owns
// columns 4*cg .. 4*cg+3 and the parts s = ps (mod NSUB): per chunk of 64
// parts, lane j computes part j's weight exp(LSE_j - max) from one load, the
// weights are passed around by shuffles, and each lane then issues the loads
// of all its non-empty parts at once (eight at a time), so a row costs a few
// memory round trips whatever the part count.  Empty parts (LSE = -inf,
// weight 0) are never read.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <class T, int D>
__global__ __launch_bounds__(256) void kv_merge_kernel(KvArgs k) {
  constexpr int NG = D / 4;       // column groups of 4
  constexpr int NSUB = 64 / NG;   // part subsets
  constexpr int PPL = 64 / NSUB;  // parts of a 64-part chunk per lane
  static_assert(64 % NG == 0, "column groups must divide the wave");
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b * Hq + hq) * Nq + i
  const int lane = threadIdx.x & 63;
  if (row >= (int64_t)k.B * k.Hq * k.Nq) return;
  const int cg = lane % NG, ps = lane / NG;
  const float* lse_s = k.ws_lse + row * k.S;
  const float* po = k.ws_o + row * k.S * D + 4 * cg;
  float m = -INFINITY;
  for (int s = lane; s < k.S; s += 64) m = fmaxf(m, lse_s[s]);
  m = wave_max(m);
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (m != -INFINITY) {
    for (int c0 = 0; c0 < k.S; c0 += 64) {
      const float wl = (c0 + lane < k.S) ? __expf(lse_s[c0 + lane] - m) : 0.f;
      den += wl;
#pragma unroll
      for (int u0 = 0; u0 < PPL; u0 += 8) {
        float wgt[8];
        f32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int sp = ps + NSUB * (u0 + u);  // part within the chunk
          wgt[u] = __shfl(wl, sp, 64);
          v[u] = wgt[u] > 0.f ? *reinterpret_cast<const f32x4*>(po + (int64_t)(c0 + sp) * D)
                              : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += wgt[u] * v[u];
      }
    }
    den = wave_sum(den);
  }
  // Sum the part subsets (lanes with the same column group).
#pragma unroll
  for (int o = NG; o < 64; o <<= 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const int i = (int)(row % k.Nq);
  const int64_t bh = row / k.Nq;
  const int hq = (int)(bh % k.Hq);
  const int b = (int)(bh / k.Hq);
  if (ps == 0 && 4 * cg < k.D) {
    uint16_t* op = static_cast<uint16_t*>(k.o) + b * k.o_sb + (int64_t)i * k.o_sn + hq * k.o_sh + 4 * cg;
    *reinterpret_cast<u32x2*>(op) = u32x2{T::pack(acc[0] * inv, acc[1] * inv), T::pack(acc[2] * inv, acc[3] * inv)};
  }
  if (lane == 0) k.lse[row] = (den > 0.f) ? m + logf(den) : -INFINITY;
}

template <class T, int D>
static hipError_t launch_kv_t(const KvArgs& k, hipStream_t stream) {
  const dim3 grid((unsigned)(k.n_split + k.n_append));
  if (k.page_size) {
    if (k.mod)
      hipLaunchKernelGGL((kv_split_kernel<T, D, FA_KV_DEPTH, true, true>), grid, dim3(64), 0, stream, k);
    else
      hipLaunchKernelGGL((kv_split_kernel<T, D, FA_KV_DEPTH, false, true>), grid, dim3(64), 0, stream, k);
  } else {
    if (k.mod)
      hipLaunchKernelGGL((kv_split_kernel<T, D, FA_KV_DEPTH, true, false>), grid, dim3(64), 0, stream, k);
    else
      hipLaunchKernelGGL((kv_split_kernel<T, D, FA_KV_DEPTH, false, false>), grid, dim3(64), 0, stream, k);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)k.B * k.Hq * k.Nq;
  hipLaunchKernelGGL((kv_merge_kernel<T, D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, k);
  return hipGetLastError();
}

hipError_t launch_kvcache(const KvArgs& k, hipStream_t stream) {
  // Head dims below 64 / 128 run the 64 / 128 kernels with the rest masked.
  if (k.dtype == kBF16) {
    if (k.D > 64 && k.D <= 128) return launch_kv_t<BF16, 128>(k, stream);
    if (k.D >= 8 && k.D <= 64) return launch_kv_t<BF16, 64>(k, stream);
  } else if (k.dtype == kF16) {
    if (k.D > 64 && k.D <= 128) return launch_kv_t<F16, 128>(k, stream);
    if (k.D >= 8 && k.D <= 64) return launch_kv_t<F16, 64>(k, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
