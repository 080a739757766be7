// Forward attention for fp16/bf16 on gfx950 with 32x32x16 MFMA.
//
// The method ([P4] "FlashAttention 实战指南", section "长序列注意力为什么会爆内存"):
// Q, K and V are cut into tiles; one tile of queries stays on chip while K/V
// tiles stream through LDS; each K/V tile's scores and softmax are computed on
// chip, and an online softmax keeps the running row maximum and row sum so
// that the full score matrix never exists.  The output is the exact attention
// result; the kernel also writes the per-row log-sum-exp for the backward pass.
//
// gfx950 mapping.  One workgroup = NW waves = a tile of BM = 32*NW queries of
// one (batch, query head); each wave owns 32 query rows.  For every K/V tile of
// BN keys:
//   S^T (BN x 32) = K Q^T      A operand = K rows from LDS, B = Q (registers)
//   online softmax             lane l holds query l%32 and 16 keys per 32x32
//                              block, so row max/sum are in-register plus one
//                              exchange with lane l^32
//   O^T (D x 32) += V^T P^T    A operand = V^T from a transposed LDS copy,
//                              B = P^T straight from the softmax registers
// The O rescale by exp(m_old - m_new) is a per-lane scalar (one query per lane).
// Scores are kept in raw units; exp(scale*(s - m)) is evaluated as
// exp2(s*c - m*c) with c = scale*log2(e), one FMA and one v_exp_f32.
// K and V tiles sit in LDS row-major with a chunk swizzle (tile_io.hpp); V^T
// operands come straight from the row-major tile through the transposing LDS
// read.  Tiles are double buffered: each step first issues the direct-to-LDS
// loads of tile t+1 into the other buffer, then computes tile t; one barrier
// per tile.
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

// Launch configuration (tuned on MI355X; overridable at build time).
#ifndef FA_FWD_BN
#define FA_FWD_BN 64  // keys per K/V tile
#endif
#ifndef FA_FWD_NW
#define FA_FWD_NW 8  // waves per workgroup (32 queries each)
#endif
#ifndef FA_FWD_WPE
#define FA_FWD_WPE 2  // waves per SIMD the register allocation targets
#endif
#ifndef FA_FWD_PRIO
#define FA_FWD_PRIO 0  // raise wave priority around MFMA phases (measured: no gain)
#endif

// Per-workgroup state of the forward kernel; step<BUF>() processes one K/V tile
// held in LDS buffer BUF while the next tile is loaded into the other buffer.
template <class T, int D, int BN, int NW>
struct FwdCtx {
  static constexpr int TILE = BN * D;  // elements of one K or V tile
  uint16_t* smem;                      // [buf][K tile, V tile], swizzled row-major
  const uint16_t* Kp;
  const uint16_t* Vp;
  int64_t k_sn, v_sn;
  int Nk, t_hi, lo_i, hi_i, lo_max, hi_min, wave, lane, hf;
  float c;
  u32x4 qf[D / 16];
  int kro[D / 16];     // per-lane LDS offsets of the K row chunks
  int vro[D / 32][2];  // per-lane LDS offsets of the transposing V reads
  DmaTile<D, BN, NW> kd, vd;
  float mref, l;
  f32x16 oacc[D / 32];

  template <int BUF>
  __device__ __forceinline__ void step(int t) {
    const char* Ks = reinterpret_cast<const char*>(smem + BUF * 2 * TILE);
    const char* Vs = Ks + TILE * 2;
    const int j0 = t * BN;
    if (t < t_hi) {
      kd.issue(Kp, k_sn, j0 + BN, Nk, smem + (1 - BUF) * 2 * TILE, wave);
      vd.issue(Vp, v_sn, j0 + BN, Nk, smem + (1 - BUF) * 2 * TILE + TILE, wave);
    }

    // S^T = K Q^T.  s[kb][r] is key j0 + 32*kb + 8*(r/4) + 4*hf + r%4.
    // MFMA phases run at raised wave priority so that, of the waves sharing a
    // SIMD, the one feeding the matrix core issues first and the other fills
    // the VALU with softmax work.
    f32x16 s[BN / 32];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) s[kb] = f32x16{};
    if (FA_FWD_PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
        s[kb] = T::mfma(*reinterpret_cast<const u32x4*>(Ks + kb * 32 * 2 * D + kro[st]), qf[st], s[kb]);
    }
    if (FA_FWD_PRIO) __builtin_amdgcn_s_setprio(0);

    // Causal / window / sequence-end masking, only on tiles that need it.
    const bool full = (j0 >= lo_max) && (j0 + BN - 1 <= hi_min);
    if (!full) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (key < lo_i || key > hi_i) s[kb][r] = -INFINITY;
        }
      }
    }

    // Online softmax.  The reference maximum moves only when some row of the
    // wave grew by more than 2^kLazyRescale; then O and l are rescaled.
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    }
    mx = fmaxf(mx, xor32(mx));
    if (__any((mx - mref) * c > kLazyRescale)) {  // false for NaN (both -inf)
      const float m_new = fmaxf(mref, mx);
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2((mref - m_new) * c);
      mref = m_new;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
    }
    const float mc = (mref == -INFINITY) ? 0.f : mref * c;
    u32x4 pf[BN / 16];  // P^T as B operands, one per 16 keys
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = fast_exp2(fmaf(s[kb][8 * tt + e], c, -mc));
          l += p[e];
        }
        pf[2 * kb + tt] = u32x4{T::pack(p[0], p[1]), T::pack(p[2], p[3]), T::pack(p[4], p[5]),
                                T::pack(p[6], p[7])};
      }
    }

    // O^T += V^T P^T, V^T read transposed from the row-major tile.
    if (FA_FWD_PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int si = 0; si < BN / 16; ++si) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(Vs + si * 16 * 2 * D + vro[db][0]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(Vs + si * 16 * 2 * D + vro[db][1]));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        oacc[db] = T::mfma(u32x4{l2[0], l2[1], h2[0], h2[1]}, pf[si], oacc[db]);
      }
    }
    if (FA_FWD_PRIO) __builtin_amdgcn_s_setprio(0);
    wait_all_loads();  // the next tile has landed in this wave's share of LDS
    __syncthreads();
  }
};

template <class T, int D, int BN, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(FA_FWD_WPE, FA_FWD_WPE))) void fwd_mfma_kernel(AttnArgs a) {
  constexpr int BM = NW * 32;
  using Ctx = FwdCtx<T, D, BN, NW>;
  constexpr int TILE = Ctx::TILE;
  // Two buffers, each one K tile then one V tile, filled by direct-to-LDS loads.
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * TILE];
  static_assert(2 * 2 * TILE * 2 <= 65536, "LDS offsets must fit the 16-bit immediate");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;

  const int n_qt = (a.Nq + BM - 1) / BM;
  const bool heavy_last = (a.causal || a.wr >= 0) && a.wl < 0;
  const WorkItem it = decode_work(blockIdx.x, a.B * a.Hkv, n_qt, a.G, heavy_last, a.xcd_remap);
  const int b = it.unit / a.Hkv, hk = it.unit % a.Hkv;
  const int hq = hk * a.G + it.sub;
  const int q0 = it.tile * BM;
  const int qrow = q0 + wave * 32 + l32;  // the query of this lane's column

  Ctx x;
  x.smem = smem;
  x.Kp = static_cast<const uint16_t*>(a.k) + b * a.k_sb + hk * a.k_sh;
  x.Vp = static_cast<const uint16_t*>(a.v) + b * a.v_sb + hk * a.v_sh;
  x.k_sn = a.k_sn;
  x.v_sn = a.v_sn;
  x.Nk = a.Nk;
  x.wave = wave;
  x.lane = lane;
  x.hf = hf;
  x.c = a.scale_log2;
  const uint16_t* Qp = static_cast<const uint16_t*>(a.q) + b * a.q_sb + hq * a.q_sh;

  // Q as the B operand of S^T = K Q^T: lane holds d = 16*st + 8*hf + (0..7).
  if (qrow < a.Nq) {
    const uint16_t* qr = Qp + (int64_t)qrow * a.q_sn + 8 * hf;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) x.qf[st] = *reinterpret_cast<const u32x4*>(qr + 16 * st);
  } else {
#pragma unroll
    for (int st = 0; st < D / 16; ++st) x.qf[st] = u32x4{0u, 0u, 0u, 0u};
  }

  // Visible keys of this lane's query, and the workgroup's key range.
  x.lo_i = key_lo(a, qrow);
  x.hi_i = key_hi(a, qrow);
  const int q_last = min(q0 + BM, a.Nq) - 1;
  const int kv_lo = key_lo(a, q0), kv_hi = key_hi(a, q_last);
  x.lo_max = key_lo(a, q_last);
  x.hi_min = key_hi(a, q0);
  const int t_lo = kv_lo / BN;
  x.t_hi = (kv_hi >= kv_lo) ? kv_hi / BN : t_lo - 1;

  // Per-lane LDS byte offsets, fixed for the whole kernel; tile, buffer,
  // key-block and 16-key-step offsets are compile-time immediates.
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

  x.kd.init(wave, lane, a.k_sn);
  x.vd.init(wave, lane, a.v_sn);
  if (t_lo <= x.t_hi) {
    x.kd.issue(x.Kp, a.k_sn, t_lo * BN, a.Nk, smem, wave);
    x.vd.issue(x.Vp, a.v_sn, t_lo * BN, a.Nk, smem + TILE, wave);
    wait_all_loads();
  }
  __syncthreads();

  int t = t_lo;
  for (; t + 1 <= x.t_hi; t += 2) {
    x.template step<0>(t);
    x.template step<1>(t + 1);
  }
  if (t <= x.t_hi) x.template step<0>(t);

  // Epilogue: O = O / l, LSE = scale*mref + ln(l).  Lanes l and l^32 hold
  // different keys of the same query, so their partial sums are added here.
  const float lt = x.l + xor32(x.l);
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
        *reinterpret_cast<u32x2*>(op + d0) = w;
      }
    }
    if (hf == 0)
      a.lse[((int64_t)b * a.Hq + hq) * a.Nq + qrow] = (lt > 0.f) ? (x.mref * a.scale + logf(lt)) : -INFINITY;
  }
}

template <class T, int D, int BN, int NW>
static hipError_t launch_fwd_t(const AttnArgs& a, hipStream_t stream) {
  constexpr int BM = NW * 32;
  const int n_qt = (a.Nq + BM - 1) / BM;
  const int64_t total = (int64_t)a.B * a.Hkv * n_qt * a.G;
  if (total == 0) return hipSuccess;
  AttnArgs args = a;
  args.xcd_remap = a.xcd_remap && ((a.B * a.Hkv) % 8 == 0);
  hipLaunchKernelGGL((fwd_mfma_kernel<T, D, BN, NW>), dim3((unsigned)total), dim3(NW * 64), 0,
                     stream, args);
  return hipGetLastError();
}

hipError_t launch_fwd_mfma(const AttnArgs& a, hipStream_t stream) {
  if (a.dtype == kBF16) {
    if (a.D == 128) return launch_fwd_t<BF16, 128, FA_FWD_BN, FA_FWD_NW>(a, stream);
    if (a.D == 64) return launch_fwd_t<BF16, 64, FA_FWD_BN, FA_FWD_NW>(a, stream);
  } else if (a.dtype == kF16) {
    if (a.D == 128) return launch_fwd_t<F16, 128, FA_FWD_BN, FA_FWD_NW>(a, stream);
    if (a.D == 64) return launch_fwd_t<F16, 64, FA_FWD_BN, FA_FWD_NW>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
