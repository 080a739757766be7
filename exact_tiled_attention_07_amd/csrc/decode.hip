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
// Three kernels:
//   kv_append   the copy (16 bytes per lane);
//   kv_split    one wave per (batch, kv head, block of 32 query rows, part):
//               the G query heads x Nq queries of a K/V head are packed as the
//               32 columns of S^T = K Q^T, so every K/V row read from HBM serves
//               all of them.  K goes from global memory straight into MFMA A
//               operands; V goes through registers into the wave's own LDS
//               tile, read back transposed for O^T += V^T P^T.  No barriers:
//               each wave only reads what it wrote.  The part's key tiles are a
//               contiguous share of the visible range; it writes its O / l and
//               LSE (float32) to the workspace;
//   kv_merge    per query row, O = sum_s exp(LSE_s - LSE) O_s with
//               LSE = ln sum_s exp(LSE_s) (empty parts weigh 0).
#include "common.hpp"
#include "launch.hpp"
#include "tile_io.hpp"

namespace fa {

// ---------------------------------------------------------------------------
// Append: k_new[b, i, h] -> k_cache[b, L_b + i, h] for L_b + i < capacity.
// One 16-byte chunk per lane; grid covers B * Nq * Hkv rows, 2 tensors.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kv_append_kernel(KvArgs k) {
  const int cpr = k.D * 2 / 16;  // 16-byte chunks per row
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
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
  char* dst = static_cast<char*>(which ? k.v_cache : k.k_cache) +
              2 * (b * (which ? k.vc_sb : k.kc_sb) + (int64_t)dst_row * (which ? k.vc_sn : k.kc_sn) +
                   h * (which ? k.vc_sh : k.kc_sh)) + 16 * c;
  *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
}

// Number of keys of batch entry b after the append.
__device__ __forceinline__ int kv_len(const KvArgs& k, int b) {
  const int L = min(max(k.cache_seqlens[b], 0), k.cap);
  return k.append ? min(L + k.Nq, k.cap) : L;
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
//   S^T (32 keys x 32 rows) = K Q^T   A = K rows (registers), B = Q rows
//   online softmax per lane (row), with the forward's lazy rescale
//   O^T (D x 32 rows) += V^T P^T      A = V^T from the wave's LDS tile
// ---------------------------------------------------------------------------
static constexpr float kKvLazyRescale = 8.0f;

template <class T, int D>
__global__ __launch_bounds__(64) void kv_split_kernel(KvArgs k) {
  constexpr int NST = D / 16;           // 16-wide d steps
  constexpr int VCH = 32 * D * 2 / 16;  // 16-byte chunks of a 32-row V tile
  constexpr int VPL = VCH / 64;         // chunks per lane
  __shared__ __attribute__((aligned(16))) uint16_t vt[32 * D];

  const int lane = threadIdx.x, l32 = lane & 31, hf = lane >> 5;
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
  const int Lk = kv_len(k, b);

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
    const uint16_t* qr = static_cast<const uint16_t*>(k.q) + b * k.q_sb + (int64_t)i * k.q_sn + hq * k.q_sh + 8 * hf;
#pragma unroll
    for (int st = 0; st < NST; ++st) qf[st] = *reinterpret_cast<const u32x4*>(qr + 16 * st);
  } else {
#pragma unroll
    for (int st = 0; st < NST; ++st) qf[st] = u32x4{0u, 0u, 0u, 0u};
  }

  const uint16_t* Kc = static_cast<const uint16_t*>(k.k_cache) + b * k.kc_sb + hk * k.kc_sh;
  const uint16_t* Vc = static_cast<const uint16_t*>(k.v_cache) + b * k.vc_sb + hk * k.vc_sh;
  // Per-lane parts of a tile load: K operand row l32, d chunk 2*st + hf; V
  // chunk (row, column chunk) for the swizzled LDS tile.
  int voff[VPL];
  int vrow[VPL], vcol[VPL];
#pragma unroll
  for (int c = 0; c < VPL; ++c) {
    const int ch = lane + 64 * c;
    vrow[c] = ch / (D / 8);
    vcol[c] = ch % (D / 8);
    voff[c] = Swz<D>::off(vrow[c], vcol[c]);
  }
  SwzOffsets<D> off;
  off.init(lane);
  const float cs = k.scale_log2;

  auto load_tile = [&](int t, u32x4 (&kr)[NST], u32x4 (&vr)[VPL]) {
    const int kk = min(32 * t + l32, Lk - 1);  // rows past the end repeat the last one (masked)
    const uint16_t* kp = Kc + (int64_t)kk * k.kc_sn + 8 * hf;
#pragma unroll
    for (int st = 0; st < NST; ++st) kr[st] = *reinterpret_cast<const u32x4*>(kp + 16 * st);
#pragma unroll
    for (int c = 0; c < VPL; ++c) {
      const int vk = min(32 * t + vrow[c], Lk - 1);
      vr[c] = *reinterpret_cast<const u32x4*>(Vc + (int64_t)vk * k.vc_sn + 8 * vcol[c]);
    }
  };

  float mref = -INFINITY, l = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};

  u32x4 kr[NST], vr[VPL];
  if (t_beg < t_end) load_tile(t_beg, kr, vr);
  for (int t = t_beg; t < t_end; ++t) {
    // V(t) into the wave's tile (LDS operations of a wave complete in order,
    // so the previous tile's reads are done and these writes precede the
    // reads below).
#pragma unroll
    for (int c = 0; c < VPL; ++c) *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(vt) + voff[c]) = vr[c];
    u32x4 kc[NST];
#pragma unroll
    for (int st = 0; st < NST; ++st) kc[st] = kr[st];
    if (t + 1 < t_end) load_tile(t + 1, kr, vr);

    // S^T = K Q^T; s[r] is key 32t + 8*(r/4) + 4*hf + r%4.
    f32x16 sv = f32x16{};
#pragma unroll
    for (int st = 0; st < NST; ++st) sv = T::mfma(kc[st], qf[st], sv);
    const int j0 = 32 * t;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = j0 + 8 * (r >> 2) + 4 * hf + (r & 3);
      if (key < lo_r || key > hi_r) sv[r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sv[r]);
    mx = fmaxf(mx, xor32(mx));
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
  }

  // Partial result of this part: O / l and LSE (natural log), per row.
  const float lt = l + xor32(l);
  if (valid) {
    const int64_t row = ((int64_t)(b * k.Hq + hq) * k.Nq + i) * k.S + s;
    float* po = k.ws_o + row * D;
    const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * db + 8 * g4 + 4 * hf;
        *reinterpret_cast<f32x4*>(po + d0) = f32x4{oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv,
                                                   oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv};
      }
    }
    if (hf == 0) k.ws_lse[row] = (lt > 0.f) ? (mref * k.scale + logf(lt)) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Merge of the S parts of one query row: 64 lanes per row, lane handles
// columns 2*lane and 2*lane + 1 (lanes past D/2 idle).
// ---------------------------------------------------------------------------
template <class T, int D>
__global__ __launch_bounds__(256) void kv_merge_kernel(KvArgs k) {
  static_assert(D % 2 == 0 && D <= 128, "two columns per lane");
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b * Hq + hq) * Nq + i
  const int lane = threadIdx.x & 63;
  if (row >= (int64_t)k.B * k.Hq * k.Nq) return;
  const int i = (int)(row % k.Nq);
  const int64_t bh = row / k.Nq;
  const int hq = (int)(bh % k.Hq);
  const int b = (int)(bh / k.Hq);
  const float* lse_s = k.ws_lse + row * k.S;
  float m = -INFINITY;
  for (int s = 0; s < k.S; ++s) m = fmaxf(m, lse_s[s]);
  const int c0 = 2 * lane;
  const bool has = c0 < D;
  float a0 = 0.f, a1 = 0.f, den = 0.f;
  if (m != -INFINITY) {
    for (int s = 0; s < k.S; ++s) {
      const float wgt = __expf(lse_s[s] - m);  // 0 for empty parts (LSE = -inf)
      den += wgt;
      if (has) {
        const float* po = k.ws_o + (row * k.S + s) * D + c0;
        a0 = fmaf(wgt, po[0], a0);
        a1 = fmaf(wgt, po[1], a1);
      }
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  if (has) {
    uint16_t* op = static_cast<uint16_t*>(k.o) + b * k.o_sb + (int64_t)i * k.o_sn + hq * k.o_sh + c0;
    *reinterpret_cast<uint32_t*>(op) = T::pack(a0 * inv, a1 * inv);
  }
  if (lane == 0) k.lse[row] = (den > 0.f) ? m + logf(den) : -INFINITY;
}

template <class T, int D>
static hipError_t launch_kv_t(const KvArgs& k, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (k.append) {
    const int64_t chunks = 2 * (int64_t)k.B * k.Nq * k.Hkv * (D * 2 / 16);
    hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream, k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t waves = (int64_t)k.B * k.Hkv * k.n_rb * k.S;
  hipLaunchKernelGGL((kv_split_kernel<T, D>), dim3((unsigned)waves), dim3(64), 0, stream, k);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t rows = (int64_t)k.B * k.Hq * k.Nq;
  hipLaunchKernelGGL((kv_merge_kernel<T, D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, k);
  return hipGetLastError();
}

hipError_t launch_kvcache(const KvArgs& k, hipStream_t stream) {
  if (k.dtype == kBF16) {
    if (k.D == 128) return launch_kv_t<BF16, 128>(k, stream);
    if (k.D == 64) return launch_kv_t<BF16, 64>(k, stream);
  } else if (k.dtype == kF16) {
    if (k.D == 128) return launch_kv_t<F16, 128>(k, stream);
    if (k.D == 64) return launch_kv_t<F16, 64>(k, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
