// Backward attention for fp16/bf16 on gfx950 with 32x32x16 MFMA.
//
// The backward pass does not keep the attention matrix: it recomputes each
// probability tile from Q, K and the forward log-sum-exp when it is needed
// ([P4] "FlashAttention 实战指南", section "长序列注意力为什么会爆内存",
// recomputation traded for memory).  The gradient formulas are the exact
// derivative of the forward:
//   P = exp(scale*QK^T - LSE),  dP = dO V^T,  D_i = sum_c dO_ic O_ic,
//   dS = P * (dP - D),  dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K.
//
// Three kernels, none with atomics (results are bitwise repeatable):
//   preprocess  D_i for every query row (fp32 workspace)
//   dK/dV       one workgroup per (batch, kv head, tile of 128 keys) with
//               score waves and gradient waves (described at the kernel):
//                 S  = Q K^T,  dP = dO V^T       (score waves)
//                 dV^T += dO^T P,  dK^T += Q^T dS (gradient waves, one item later)
//               GQA sums over the group inside the workgroup.
//   dQ          one workgroup per (batch, query head, tile of 32*NW queries);
//               the forward's layout (one query per lane):
//                 S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T
// The dQ kernel recomputes S and dP (7 tile products per score pair instead of
// 5) in exchange for no atomic accumulation and no dQ workspace.
// All staged tiles are row-major in LDS with the chunk swizzle of tile_io.hpp
// and double buffered (one barrier per tile); operands whose reduction axis
// runs along the tile rows come from the transposing LDS read.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "tile_io.hpp"

namespace fa {

// ---------------------------------------------------------------------------
// Row statistics for the backward kernels, one float each per (b, h, row) in
// arrays padded to Nq_pad = ceil(Nq / 128) * 128 rows:
//   dsum[row] = D_i = sum_c dout[i, c] * o[i, c]    (0 for padding rows)
//   lse2[row] = LSE_i * log2(e)                      (+inf for padding rows and
//               for rows that see no key, so exp2(s*c - lse2) is exactly 0)
// Any dtype; 16 lanes per row.
// ---------------------------------------------------------------------------
template <int ELT>  // element bytes: 4 (fp32) or 2 (fp16/bf16)
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(AttnArgs a) {
  constexpr int EPC = 16 / ELT;  // elements per 16-byte chunk
  const int nq_pad = (a.Nq + 127) / 128 * 128;  // of the longest sequence for packed batches
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const int64_t rows = (int64_t)a.B * nq_pad * a.Hq;
  // fp32 inputs accumulate in float64 (exact products); 16-bit inputs in fp32.
  using Acc = typename std::conditional<ELT == 4, double, float>::type;
  Acc acc = 0;
  int h = 0, i = 0, b = 0;
  bool active = false;  // row inside its sequence's padded range
  if (row < rows) {
    h = (int)(row % a.Hq);
    const int64_t t = row / a.Hq;
    i = (int)(t % nq_pad);
    b = (int)(t / nq_pad);
    bind_seq(a, b);
    active = i < (a.Nq + 127) / 128 * 128;
    if (i < a.Nq) {
      const int64_t base = (b * a.o_sb + (int64_t)i * a.o_sn + h * a.o_sh) * ELT;
      const char* dop = static_cast<const char*>(a.dout) + base;
      const char* op = static_cast<const char*>(a.o) + base;
      for (int cc = sub; cc * EPC < a.D; cc += 16) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(dop + cc * 16);
        const u32x4 y = *reinterpret_cast<const u32x4*>(op + cc * 16);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if constexpr (ELT == 4) {
            acc = fma((double)__uint_as_float(x[w]), (double)__uint_as_float(y[w]), acc);
          } else if (a.dtype == kBF16) {
            acc = fmaf(BF16::to_f32(x[w] & 0xffffu), BF16::to_f32(y[w] & 0xffffu), acc);
            acc = fmaf(BF16::to_f32(x[w] >> 16), BF16::to_f32(y[w] >> 16), acc);
          } else {
            acc = fmaf(F16::to_f32(x[w] & 0xffffu), F16::to_f32(y[w] & 0xffffu), acc);
            acc = fmaf(F16::to_f32(x[w] >> 16), F16::to_f32(y[w] >> 16), acc);
          }
        }
      }
    }
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
  if (active && sub == 0) {
    const int64_t o = b * a.ws_sb + h * a.ws_sh + i;
    a.dsum[o] = (float)acc;
    float l2 = INFINITY;
    if (i < a.Nq) {
      const float L = a.lse[b * a.lse_sb + h * a.lse_sh + i];
      if (L != -INFINITY) l2 = L * kLog2e;
    }
    a.lse2[o] = l2;
  }
}

hipError_t launch_bwd_preprocess(const AttnArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * ((a.Nq + 127) / 128 * 128) * a.Hq;
  if (rows == 0) return hipSuccess;
  const unsigned grid = (unsigned)((rows + 15) / 16);
  if (a.dtype == kF32)
    hipLaunchKernelGGL(bwd_preprocess_kernel<4>, dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_preprocess_kernel<2>, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// Launch configuration (tuned on MI355X; overridable at build time).
#ifndef FA_DKDV_BMQ
#define FA_DKDV_BMQ 64  // queries per dK/dV iteration
#endif
#ifndef FA_DKDV_GRING
#define FA_DKDV_GRING 2  // transposed operand pairs in flight in the dK/dV gradient waves
#endif
#ifndef FA_DQ_RING
#define FA_DQ_RING 3  // LDS operands in flight ahead of the MFMA that uses them
#endif
#ifndef FA_DQ_BN
#define FA_DQ_BN 64  // keys per dQ iteration
#endif
#ifndef FA_DQ_NW
#define FA_DQ_NW 8  // waves per dQ workgroup (32 queries each)
#endif
#ifndef FA_DQ_WPE
#define FA_DQ_WPE 2
#endif

// ---------------------------------------------------------------------------
// dK / dV with specialised waves.
//
// One workgroup per (batch, kv head, tile of 32*KW keys) runs 2*KW waves:
//   score waves    (0 .. KW-1)   hold the K and V rows of their 32 keys as MFMA
//                  B operands; per item they compute S = Q K^T and dP = dO V^T,
//                  then P = exp2(s*c - lse2) and dS = P * (dP - D), and write P
//                  and dS to LDS exactly as the B-operand registers they are
//                  (16 bytes per lane);
//   gradient waves (KW .. 2KW-1) hold dK^T and dV^T accumulators; gradient
//                  wave KW + k owns key blocks 2*(k/2) and 2*(k/2) + 1 and the
//                  d blocks of group k % 2 (D/64 of them); one item later they
//                  read P and dS of their key blocks back and accumulate
//                  dV^T += dO^T P and dK^T += Q^T dS, with dO^T and Q^T read
//                  transposed from the item's tiles, each transposed operand
//                  feeding both key blocks' MFMAs.
// Score wave k and gradient wave KW + k share a SIMD.  Each item takes two
// barriers: before the first the score waves run their MFMAs while the
// gradient waves fetch P and dS and issue the next item's tile loads; after
// it the gradient waves run their MFMAs while
// the score waves do the exponentials.  So the matrix core of every SIMD
// always has one wave feeding it, and the vector work hides behind it.
// Q/dO tiles rotate through three LDS slots (the item being scored, the item
// being accumulated, and the next item's loads in flight); P/dS need one
// buffer, read before the first barrier and written after it.
// ---------------------------------------------------------------------------
template <int D, int BMQ>
struct DkdvWsLayout {
  static constexpr int KW = 4;                      // key blocks (32 keys) per workgroup
  static constexpr int NW = 2 * KW;                 // waves per workgroup
  static constexpr int BNK = 32 * KW;               // keys per workgroup
  static constexpr int TILE = BMQ * D;              // elements of one Q or dO tile
  static constexpr int SLOT = 2 * TILE * 2;         // bytes of one Q + dO slot
  static constexpr int NSLOT = 3;
  static constexpr int IMG = (BMQ / 16) * 64 * 16;  // bytes of one wave's P (or dS) operands
  static constexpr int RST = 2 * BMQ * 4;           // lse2[BMQ] then dsum[BMQ]
  static constexpr int OFF_PDS = NSLOT * SLOT;
  static constexpr int OFF_RST = OFF_PDS + KW * 2 * IMG;
  static constexpr int BYTES = OFF_RST + NSLOT * RST;
};

template <class T, int D, int BMQ, bool MOD>
struct DkdvWs {
  using L = DkdvWsLayout<D, BMQ>;
  char* smem;  // [slot][Q tile, dO tile], [score wave][P, dS images], [slot][lse2, dsum]
  const AttnArgs* a;
  int b, hk, k0, k_last, key, qt_lo, n_qt, n_items, wave, kb, lane, hf;
  int kp, dg;  // gradient waves: key-block pair and d-block group they accumulate
  // A gradient wave owns key blocks 2*kp, 2*kp + 1 and d blocks NDW*dg .. NDW*dg + NDW - 1.
  static constexpr int NDW = D / 64;
  int gtr[NDW][2];  // off.tr of this gradient wave's d blocks (set_grad_blocks)
  float c;
  SwzOffsets<D> off;
  // The gradient waves load the next item's Q and dO tiles and row
  // statistics at the start of an item, while they have no MFMAs to run and
  // the score waves start their products at once (a CU's tile loads pass its
  // address unit at a limited rate, so a wave that issues them waits).  A
  // wave whose transposing LDS reads follow its own direct-to-LDS loads in
  // program order is made to wait for those loads by the compiler, even where
  // they cannot overlap; the gradient waves wait for theirs before the item's
  // first barrier anyway.
  DmaTile<D, BMQ, L::KW> qd, dd;

  // Work items run over query tiles from the last one down, with the heads of
  // the group innermost: the workgroups of one K/V head that run at the same
  // time read the same Q/dO tiles at about the same time, and those come from
  // L2.  Cursor (tile from the top, head) of an item:
  struct Cursor {
    int t, g;
    __device__ __forceinline__ void next(int G) {
      if (++g == G) {
        g = 0;
        ++t;
      }
    }
  };
  __device__ __forceinline__ int row_of(const Cursor& cu) const { return (qt_lo + n_qt - 1 - cu.t) * BMQ; }

  __device__ __forceinline__ char* slot_tiles(int slot) const { return smem + slot * L::SLOT; }
  __device__ __forceinline__ char* slot_stats(int slot) const { return smem + L::OFF_RST + slot * L::RST; }

  // Wave kb of a group loads its share of one item's Q tile (and wave KW-1
  // the item's row statistics) if Q, and of its dO tile if DO, into slot
  // `slot`.
  template <bool Q, bool DO>
  __device__ __forceinline__ void issue(const Cursor& cu, int slot) {
    const int i0 = row_of(cu), hq = hk * a->G + cu.g;
    if (Q)
      qd.issue(static_cast<const uint16_t*>(a->q) + b * a->q_sb + hq * a->q_sh, a->q_sn, i0, a->Nq,
               reinterpret_cast<uint16_t*>(slot_tiles(slot)));
    if (DO)
      dd.issue(static_cast<const uint16_t*>(a->dout) + b * a->o_sb + hq * a->o_sh, a->o_sn, i0, a->Nq,
               reinterpret_cast<uint16_t*>(slot_tiles(slot) + L::TILE * 2));
    if (Q && kb == L::KW - 1) {
      const int64_t ro = b * a->ws_sb + hq * a->ws_sh + i0;
      uint16_t* r = reinterpret_cast<uint16_t*>(slot_stats(slot));
      if (lane < BMQ / 4) {  // lse2[BMQ] then dsum[BMQ]
        buffer_dma16(raw_rsrc(a->lse2 + ro, BMQ * 4), 16 * lane, r);
        buffer_dma16(raw_rsrc(a->dsum + ro, BMQ * 4), 16 * lane, r + BMQ * 2);
      }
    }
  }

  // Gradient waves: key-block pair and d-block group of wave index gw in
  // the group (d-block offsets picked with a select, so that the offset
  // table keeps constant indices).
  __device__ __forceinline__ void set_grad_blocks(int gw) {
    kp = gw / 2;
    dg = gw % 2;
#pragma unroll
    for (int dd = 0; dd < NDW; ++dd) {
      gtr[dd][0] = dg ? off.tr[NDW + dd][0] : off.tr[dd][0];
      gtr[dd][1] = dg ? off.tr[NDW + dd][1] : off.tr[dd][1];
    }
  }
  // Transposed operand of this gradient wave's d block dd, 16-row step si.
  __device__ __forceinline__ u32x4 gtr_operand(const char* tile, int si, int dd) const {
    const char* t = tile + si * 16 * 2 * D;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(t + gtr[dd][0]));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(t + gtr[dd][1]));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
  }
  __device__ __forceinline__ char* img(int which) const { return img_of(kb, which); }
  __device__ __forceinline__ char* img_of(int kbw, int which) const {
    return smem + L::OFF_PDS + (kbw * 2 + which) * L::IMG + lane * 16;
  }

  // S = Q K^T and dP = dO V^T of one item, 16 d-columns (one step st) at a
  // time; the row chunks of step st + NB - 1 are read while the MFMAs of step
  // st run.
  __device__ __forceinline__ void score_products(const char* Qs, const char* dOs, const u32x4 (&kf)[D / 16],
                                                 const u32x4 (&vf)[D / 16], f32x16 (&s)[BMQ / 32],
                                                 f32x16 (&dp)[BMQ / 32]) {
    constexpr int NST = D / 16, NB = 3;
    u32x4 qo[NB][BMQ / 32], go[NB][BMQ / 32];
#pragma unroll
    for (int qb = 0; qb < BMQ / 32; ++qb) s[qb] = dp[qb] = f32x16{};
#pragma unroll
    for (int st = 0; st < NB - 1; ++st) {
#pragma unroll
      for (int qb = 0; qb < BMQ / 32; ++qb) {
        qo[st][qb] = off.row_chunk(Qs, qb, st);
        go[st][qb] = off.row_chunk(dOs, qb, st);
      }
    }
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      if (st + NB - 1 < NST) {
#pragma unroll
        for (int qb = 0; qb < BMQ / 32; ++qb) {
          qo[(st + NB - 1) % NB][qb] = off.row_chunk(Qs, qb, st + NB - 1);
          go[(st + NB - 1) % NB][qb] = off.row_chunk(dOs, qb, st + NB - 1);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int qb = 0; qb < BMQ / 32; ++qb) {
        s[qb] = T::mfma(qo[st % NB][qb], kf[st], s[qb]);
        dp[qb] = T::mfma(go[st % NB][qb], vf[st], dp[qb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // dV^T += dO^T P and dK^T += Q^T dS of one item for this gradient wave's
  // two key blocks and NDW d blocks, over the (16-query step si, d block)
  // pairs; each transposed operand feeds the MFMAs of both key blocks (a
  // transposing LDS read takes more LDS time per byte than a plain 16-byte
  // read), and those of pair p + NB - 1 are read while the MFMAs of pair p run.
  __device__ __forceinline__ void grad_products(const char* Qs, const char* dOs, const u32x4 (&pf)[2][BMQ / 16],
                                                const u32x4 (&dsf)[2][BMQ / 16], f32x16 (&dka)[D / 32],
                                                f32x16 (&dva)[D / 32]) {
    constexpr int NP = (BMQ / 16) * NDW, NB = FA_DKDV_GRING;
    static_assert(NP >= NB, "pairs");
    u32x4 ao[NB], aq[NB];
#pragma unroll
    for (int pr = 0; pr < NB - 1; ++pr) {
      ao[pr] = gtr_operand(dOs, pr / NDW, pr % NDW);
      aq[pr] = gtr_operand(Qs, pr / NDW, pr % NDW);
    }
#pragma unroll
    for (int pr = 0; pr < NP; ++pr) {
      if (pr + NB - 1 < NP) {
        const int nx = pr + NB - 1;
        ao[nx % NB] = gtr_operand(dOs, nx / NDW, nx % NDW);
        aq[nx % NB] = gtr_operand(Qs, nx / NDW, nx % NDW);
      }
      __builtin_amdgcn_sched_barrier(0);
      const int si = pr / NDW, dd = pr % NDW;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        dva[kk * NDW + dd] = T::mfma(ao[pr % NB], pf[kk][si], dva[kk * NDW + dd]);
        dka[kk * NDW + dd] = T::mfma(aq[pr % NB], dsf[kk][si], dka[kk * NDW + dd]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // One item of a score wave: item w (if w < n_items) sits in slot `slot`;
  // the gradient waves load item w + 1 (cursor nx) into slot `nslot` meanwhile.
  __device__ __forceinline__ void score_step(int w, int slot, int nslot, Cursor& cu, Cursor& nx,
                                             const u32x4 (&kf)[D / 16], const u32x4 (&vf)[D / 16]) {
    // [qb][r] is query i0 + 32*qb + 8*(r/4) + 4*hf + r%4.
    f32x16 s[BMQ / 32], dp[BMQ / 32];
    if (w < n_items) score_products(slot_tiles(slot), slot_tiles(slot) + L::TILE * 2, kf, vf, s, dp);
    lds_barrier();  // the gradient waves have taken the previous item's P and dS
    if (w < n_items) {
      const int i0 = row_of(cu);
      const int i_end = min(i0 + BMQ, a->Nq) - 1;
      const bool full = (key_lo(*a, i_end) <= k0) && (key_hi(*a, i0) >= k_last);
      float slope_r = 0.f, base = 0.f;
      if constexpr (MOD) {
        slope_r = alibi_raw_uniform(a->alibi, a->alibi_sb, a->inv_scale, b, hk * a->G + cu.g);
        base = (float)(i0 + a->delta - key + 4 * hf);  // i' - key of element [0][0]
      }
      const float* lse2s = reinterpret_cast<const float*>(slot_stats(slot));
      const float* dsums = lse2s + BMQ;
      char* pimg = img(0);
      char* dimg = img(1);
#pragma unroll
      for (int qb = 0; qb < BMQ / 32; ++qb) {
        f32x4 l4[4], d4[4];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          l4[g4] = *reinterpret_cast<const f32x4*>(lse2s + 32 * qb + 8 * g4 + 4 * hf);
          d4[g4] = *reinterpret_cast<const f32x4*>(dsums + 32 * qb + 8 * g4 + 4 * hf);
        }
        if constexpr (MOD) {
          // Score modifiers, before the mask.  Where the clamp blocks the
          // gradient, dP is replaced by D, which makes dS = P * (dP - D)
          // exactly 0 without keeping a gate per element.
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            if (!(fabsf(s[qb][r]) < a->cap)) dp[qb][r] = d4[r >> 2][r & 3];
            s[qb][r] = mod_score(s[qb][r], a->cap, slope_r, base + (float)(32 * qb + 8 * (r >> 2) + (r & 3)));
          }
        }
        if (!full) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int i = i0 + 32 * qb + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (int(key < key_lo(*a, i)) | int(key > key_hi(*a, i))) s[qb][r] = -INFINITY;
          }
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          float pb[8], db_[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = 8 * tt + e;
            const float pr = fast_exp2(fmaf(s[qb][r], c, -l4[r >> 2][r & 3]));
            pb[e] = pr;
            db_[e] = pr * (dp[qb][r] - d4[r >> 2][r & 3]);
          }
          const int si = 2 * qb + tt;
          *reinterpret_cast<u32x4*>(pimg + si * 1024) =
              u32x4{T::pack(pb[0], pb[1]), T::pack(pb[2], pb[3]), T::pack(pb[4], pb[5]), T::pack(pb[6], pb[7])};
          *reinterpret_cast<u32x4*>(dimg + si * 1024) = u32x4{T::pack(db_[0], db_[1]), T::pack(db_[2], db_[3]),
                                                              T::pack(db_[4], db_[5]), T::pack(db_[6], db_[7])};
        }
      }
    }
    wait_all_loads();  // this wave's share of item w + 1 has landed
    lds_barrier();     // P/dS of item w written; item w + 1 loaded
    cu.next(a->G);
    nx.next(a->G);
  }

  // One item of a gradient wave: load the Q and dO tiles and statistics of
  // item w + 1 (cursor nx) into slot nslot, which held item w - 2; accumulate
  // item w - 1 (slot `pslot`).
  __device__ __forceinline__ void grad_step(int w, int pslot, int nslot, Cursor& nx, f32x16 (&dka)[D / 32],
                                            f32x16 (&dva)[D / 32]) {
    u32x4 pf[2][BMQ / 16], dsf[2][BMQ / 16];
    if (w + 1 < n_items) issue<true, true>(nx, nslot);
    nx.next(a->G);
    if (w >= 1) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const char* pimg = img_of(2 * kp + kk, 0);
        const char* dimg = img_of(2 * kp + kk, 1);
#pragma unroll
        for (int si = 0; si < BMQ / 16; ++si) {
          pf[kk][si] = *reinterpret_cast<const u32x4*>(pimg + si * 1024);
          dsf[kk][si] = *reinterpret_cast<const u32x4*>(dimg + si * 1024);
        }
      }
    }
    wait_all_loads();  // this wave's share of item w + 1 has landed (before any transposing read)
    lds_barrier();     // P/dS of item w - 1 are in registers
    if (w >= 1) grad_products(slot_tiles(pslot), slot_tiles(pslot) + L::TILE * 2, pf, dsf, dka, dva);
    lds_barrier();
  }

  __device__ __forceinline__ void score_loop() {
    u32x4 kf[D / 16], vf[D / 16];
    const uint16_t* Kp = static_cast<const uint16_t*>(a->k) + b * a->k_sb + hk * a->k_sh;
    const uint16_t* Vp = static_cast<const uint16_t*>(a->v) + b * a->v_sb + hk * a->v_sh;
    if (key < a->Nk) {
      const uint16_t* kr = Kp + (int64_t)key * a->k_sn;
      const uint16_t* vr = Vp + (int64_t)key * a->v_sn;
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        kf[st] = load_cols(kr, 16 * st + 8 * hf, a->D);
        vf[st] = load_cols(vr, 16 * st + 8 * hf, a->D);
      }
    } else {
#pragma unroll
      for (int st = 0; st < D / 16; ++st) kf[st] = vf[st] = u32x4{0u, 0u, 0u, 0u};
    }
    Cursor cu{0, 0}, nx{0, 0};
    nx.next(a->G);  // cursor of item w + 1
    int slot = 0;
    for (int w = 0; w <= n_items; ++w) {
      const int nslot = (slot == L::NSLOT - 1) ? 0 : slot + 1;
      score_step(w, slot, nslot, cu, nx, kf, vf);
      slot = nslot;
    }
  }

  __device__ __forceinline__ void grad_loop(f32x16 (&dka)[D / 32], f32x16 (&dva)[D / 32]) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) dka[db] = dva[db] = f32x16{};
    Cursor nx{0, 0};
    nx.next(a->G);             // cursor of item w + 1
    int pslot = L::NSLOT - 1;  // slot of item w - 1
    for (int w = 0; w <= n_items; ++w) {
      grad_step(w, pslot, pslot == 0 ? 2 : pslot - 1, nx, dka, dva);  // item w + 1 sits where w - 2 did
      pslot = (pslot == L::NSLOT - 1) ? 0 : pslot + 1;
    }
  }
};

template <class T, int D, int BMQ, bool MOD>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_ws_kernel(AttnArgs a) {
  using L = DkdvWsLayout<D, BMQ>;
  static_assert(L::NW * 64 == 512, "launch bounds assume 8 waves");
  static_assert(BMQ <= 128 && 128 % BMQ == 0, "row statistics are padded to 128 rows");
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int tpg = work_tiles_per_group(a, 1);
  const int n_kt = padded_tiles((a.Nk + L::BNK - 1) / L::BNK, tpg);
  // Under a causal mask the first key tiles see the most queries: run them
  // first (for a packed batch, the heaviest tiles of all its sequences first).
  WorkItem it;
  if (a.cu_q && a.causal && a.wl < 0 && a.xcd_remap && a.B * a.Hkv <= 8 * 64) {
    int unit = 0, tile = 0;
    if (!lpt_causal_key_tile<L::BNK>(a, blockIdx.x, a.B * a.Hkv, unit, tile)) return;
    it.unit = unit;
    it.tile = tile;
    it.sub = 0;
  } else {
    it = decode_work(blockIdx.x, a.B * a.Hkv, n_kt, 1, false, a.xcd_remap, tpg);
  }

  DkdvWs<T, D, BMQ, MOD> x;
  x.smem = smem;
  x.a = &a;
  x.b = it.unit / a.Hkv;
  x.hk = it.unit % a.Hkv;
  x.k0 = it.tile * L::BNK;
  bind_seq(a, x.b);
  if (x.k0 >= a.Nk) return;  // past the end of a shorter packed sequence (whole workgroup)
  x.wave = wave;
  x.kb = wave % L::KW;
  x.lane = lane;
  x.hf = lane >> 5;
  x.key = x.k0 + x.kb * 32 + (lane & 31);  // this lane's key (accumulator column) in a score wave
  x.c = a.scale_log2;
  x.k_last = min(x.k0 + L::BNK, a.Nk) - 1;
  const int i_lo = query_lo(a, x.k0), i_hi = query_hi(a, x.k_last);
  x.qt_lo = i_lo / BMQ;
  x.n_qt = (i_hi >= i_lo) ? i_hi / BMQ - x.qt_lo + 1 : 0;
  x.n_items = x.n_qt * a.G;  // (query tile, query head of the group) pairs
  x.off.init(lane);
  x.set_grad_blocks(wave % L::KW);
  x.qd.init(x.kb, lane, a.q_sn, a.D / 8);
  x.dd.init(x.kb, lane, a.o_sn, a.D / 8);

  if (x.n_items > 0 && wave < L::KW) {
    x.template issue<true, true>(typename DkdvWs<T, D, BMQ, MOD>::Cursor{0, 0}, 0);
    wait_all_loads();
  }
  __syncthreads();
  if (wave < L::KW) {
    x.score_loop();
    return;
  }
  f32x16 dka[D / 32], dva[D / 32];
  x.grad_loop(dka, dva);

  // Store dK = scale * dK and dV: block kk * NDW + dd holds key block
  // 2*kp + kk (lane's key in it: lane % 32) and d rows
  // 32*(NDW*dg + dd) + 8*g4 + 4*hf + 0..3.
  constexpr int NDW = DkdvWs<T, D, BMQ, MOD>::NDW;
  const float sc = a.scale;
  const int nk = a.Nk, hd = a.D;
  const int64_t k_sn = a.k_sn, v_sn = a.v_sn;
  uint16_t* const dkb = static_cast<uint16_t*>(a.dk) + x.b * a.k_sb + x.hk * a.k_sh;
  uint16_t* const dvb = static_cast<uint16_t*>(a.dv) + x.b * a.v_sb + x.hk * a.v_sh;
  const int key0 = x.k0 + 2 * x.kp * 32 + (lane & 31);
  const int dcol0 = 32 * NDW * x.dg + 4 * x.hf;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int key = key0 + 32 * kk;
    uint16_t* dkp = dkb + (int64_t)key * k_sn;
    uint16_t* dvp = dvb + (int64_t)key * v_sn;
#pragma unroll
    for (int dd = 0; dd < NDW; ++dd) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = dcol0 + 32 * dd + 8 * g4;
        const f32x16& ka = dka[kk * NDW + dd];
        const f32x16& va = dva[kk * NDW + dd];
        if (key < nk && d0 < hd) {
          *reinterpret_cast<u32x2*>(dkp + d0) = u32x2{T::pack(ka[4 * g4] * sc, ka[4 * g4 + 1] * sc),
                                                      T::pack(ka[4 * g4 + 2] * sc, ka[4 * g4 + 3] * sc)};
          *reinterpret_cast<u32x2*>(dvp + d0) =
              u32x2{T::pack(va[4 * g4], va[4 * g4 + 1]), T::pack(va[4 * g4 + 2], va[4 * g4 + 3])};
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <class T, int D, int BN, int NW, bool MOD>
struct DqCtx {
  static constexpr int TILE = BN * D;
  uint16_t* smem;  // [buf][K tile, V tile]
  const uint16_t* Kp;
  const uint16_t* Vp;
  int64_t k_sn, v_sn;
  int Nk, t_hi, lo_i, hi_i, lo_max, hi_min, wave, hf;
  float c, lse2, dsum;
  float cap, slope_r, dist0;  // score modifiers (MOD): clamp, raw slope, i' - 4*hf of this lane
  u32x4 qf[D / 16], df[D / 16];
  f32x16 dqa[D / 32];
  SwzOffsets<D> off;
  // Waves NW - NLW .. NW - 1 (one of the two waves of each SIMD) issue the
  // K/V tile loads while the other half start their products at once: a
  // CU's tile loads pass its address unit at a limited rate, so a wave that
  // issues them waits.
  static constexpr int NLW = NW / 2;
  DmaTile<D, BN, NLW> kd, vd;

  template <int BUF>
  __device__ __forceinline__ void step(int t) {
    const char* Ks = reinterpret_cast<const char*>(smem + BUF * 2 * TILE);
    const char* Vs = Ks + TILE * 2;
    const int j0 = t * BN;
    if (t < t_hi) {
      if (wave >= NW - NLW) {
        kd.issue_nonempty(Kp, k_sn, j0 + BN, Nk, smem + (1 - BUF) * 2 * TILE);
        vd.issue_nonempty(Vp, v_sn, j0 + BN, Nk, smem + (1 - BUF) * 2 * TILE + TILE);
      }
    }
    // S^T = K Q^T and dP^T = V dO^T; element [kb][r] is key j0 + 32*kb + 8*(r/4) + 4*hf + r%4.
    // Operand o: step st = o / (2 * BN/32), key block kb, K (even o) or V (odd o)
    // row chunk; each is read NB - 1 MFMAs ahead of its use.
    f32x16 s[BN / 32], dp[BN / 32];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) s[kb] = dp[kb] = f32x16{};
    {
      constexpr int NB = FA_DQ_RING, NO = (D / 16) * (BN / 32) * 2;
      auto opnd = [&](int o) {
        const int st = o / (2 * (BN / 32)), kb = (o / 2) % (BN / 32);
        return (o & 1) ? off.row_chunk(Vs, kb, st) : off.row_chunk(Ks, kb, st);
      };
      u32x4 ring[NB];
#pragma unroll
      for (int o = 0; o < NB - 1; ++o) ring[o] = opnd(o);
#pragma unroll
      for (int o = 0; o < NO; ++o) {
        if (o + NB - 1 < NO) ring[(o + NB - 1) % NB] = opnd(o + NB - 1);
        __builtin_amdgcn_sched_barrier(0);
        const int st = o / (2 * (BN / 32)), kb = (o / 2) % (BN / 32);
        if (o & 1) dp[kb] = T::mfma(ring[o % NB], df[st], dp[kb]);
        else s[kb] = T::mfma(ring[o % NB], qf[st], s[kb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (MOD) {
      // The modifiers in place, before the mask: where the clamp blocks the
      // gradient, dP is replaced by D, which makes dS = P * (dP - D) exactly
      // 0; then the score becomes the modified logit.  (A separate pass keeps
      // the dS loop below as light as the plain kernel's.)
      const float base = dist0 - (float)j0;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (!(fabsf(s[kb][r]) < cap)) dp[kb][r] = dsum;
          s[kb][r] = mod_score(s[kb][r], cap, slope_r, base - (float)(32 * kb + 8 * (r >> 2) + (r & 3)));
        }
      }
    }
    const bool full = (j0 >= lo_max) && (j0 + BN - 1 <= hi_min);
    if (!full) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = j0 + 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (kk < lo_i || kk > hi_i) s[kb][r] = -INFINITY;
        }
      }
    }
    // dS^T = P^T * (dP^T - D) as B operands, then dQ^T += K^T dS^T; the first
    // transposed K operands of the dQ product are read before the dS loop, so
    // that they have arrived when its MFMAs start.
    constexpr int QNB = FA_DQ_RING, QNO = (BN / 16) * (D / 32);
    u32x4 qring[QNB];
#pragma unroll
    for (int o = 0; o < QNB - 1; ++o) qring[o] = off.tr_operand(Ks, o / (D / 32), o % (D / 32));
    __builtin_amdgcn_sched_barrier(0);
    u32x4 dsf[BN / 16];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float ds[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * tt + e;
          const float pr = fast_exp2(fmaf(s[kb][r], c, -lse2));
          ds[e] = pr * (dp[kb][r] - dsum);
        }
        dsf[2 * kb + tt] = u32x4{T::pack(ds[0], ds[1]), T::pack(ds[2], ds[3]), T::pack(ds[4], ds[5]),
                                 T::pack(ds[6], ds[7])};
      }
    }
    {
#pragma unroll
      for (int o = 0; o < QNO; ++o) {
        if (o + QNB - 1 < QNO) {
          const int nx = o + QNB - 1;
          qring[nx % QNB] = off.tr_operand(Ks, nx / (D / 32), nx % (D / 32));
        }
        __builtin_amdgcn_sched_barrier(0);
        dqa[o % (D / 32)] = T::mfma(qring[o % QNB], dsf[o / (D / 32)], dqa[o % (D / 32)]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    wait_all_loads();
    __syncthreads();
  }
};

template <class T, int D, int BN, int NW, bool MOD>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(FA_DQ_WPE, FA_DQ_WPE))) void bwd_dq_kernel(AttnArgs a) {
  constexpr int BM = NW * 32;
  using Ctx = DqCtx<T, D, BN, NW, MOD>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * Ctx::TILE];
  static_assert(2 * 2 * Ctx::TILE * 2 <= 65536, "LDS offsets must fit the 16-bit immediate");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  // With an even GQA group, waves 0 .. NW/2 - 1 and NW/2 .. NW - 1 take the
  // same 128 query rows of two query heads that share the K/V head, as in the
  // forward, so that both halves end at the same causal key tile.
  static_assert(BM == 256, "rows per head are 256 or 128");
  const int hp = heads_per_workgroup(a);
  const int lg_rows = (hp == 2) ? 7 : 8;  // query rows per head: BM / hp
  const int wr = (hp == 2) ? (wave & (NW / 2 - 1)) : wave;
  const int n_sub = a.G >> (hp - 1);
  const int tpg = work_tiles_per_group(a, n_sub);
  const int n_qt = padded_tiles((a.Nq + (1 << lg_rows) - 1) >> lg_rows, tpg);
  const bool heavy_last = (a.causal || a.wr >= 0) && a.wl < 0;
  const WorkItem it = decode_work(blockIdx.x, a.B * a.Hkv, n_qt, n_sub, heavy_last, a.xcd_remap, tpg);
  const int b = it.unit / a.Hkv, hk = it.unit % a.Hkv;
  // (wave-uniform: read from the first lane, so that the head's pointers stay scalar)
  const int hq = hk * a.G + it.sub * hp + ((hp == 2) ? (__builtin_amdgcn_readfirstlane(wave) / (NW / 2)) : 0);
  const int q0 = it.tile << lg_rows;
  const int qrow = q0 + wr * 32 + l32;
  bind_seq(a, b);
  if (q0 >= a.Nq) return;  // past the end of a shorter packed sequence (whole workgroup)

  Ctx x;
  x.smem = smem;
  x.Kp = static_cast<const uint16_t*>(a.k) + b * a.k_sb + hk * a.k_sh;
  x.Vp = static_cast<const uint16_t*>(a.v) + b * a.v_sb + hk * a.v_sh;
  x.k_sn = a.k_sn;
  x.v_sn = a.v_sn;
  x.Nk = a.Nk;
  x.wave = wave;
  x.hf = hf;
  x.c = a.scale_log2;
  if constexpr (MOD) {
    x.cap = a.cap;
    x.slope_r = alibi_raw_uniform(a.alibi, a.alibi_sb, a.inv_scale, b, hq);
    x.dist0 = (float)(qrow + a.delta - 4 * hf);
  }
  const uint16_t* Qp = static_cast<const uint16_t*>(a.q) + b * a.q_sb + hq * a.q_sh;
  const uint16_t* dOp = static_cast<const uint16_t*>(a.dout) + b * a.o_sb + hq * a.o_sh;
  x.lse2 = INFINITY;
  x.dsum = 0.f;
  if (qrow < a.Nq) {
    const uint16_t* qr = Qp + (int64_t)qrow * a.q_sn;
    const uint16_t* dr = dOp + (int64_t)qrow * a.o_sn;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      x.qf[st] = load_cols(qr, 16 * st + 8 * hf, a.D);
      x.df[st] = load_cols(dr, 16 * st + 8 * hf, a.D);
    }
    const int64_t ri = b * a.ws_sb + hq * a.ws_sh + qrow;
    x.lse2 = a.lse2[ri];
    x.dsum = a.dsum[ri];
  } else {
#pragma unroll
    for (int st = 0; st < D / 16; ++st) x.qf[st] = x.df[st] = u32x4{0u, 0u, 0u, 0u};
  }

  x.lo_i = key_lo(a, qrow);
  x.hi_i = key_hi(a, qrow);
  const int q_last = min(q0 + (1 << lg_rows), a.Nq) - 1;
  const int kv_lo = key_lo(a, q0), kv_hi = key_hi(a, q_last);
  x.lo_max = key_lo(a, q_last);
  x.hi_min = key_hi(a, q0);
  const int t_lo = kv_lo / BN;
  x.t_hi = (kv_hi >= kv_lo) ? kv_hi / BN : t_lo - 1;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) x.dqa[db] = f32x16{};
  x.off.init(lane);
  x.kd.init(max(wave - (NW - Ctx::NLW), 0), lane, a.k_sn, a.D / 8);
  x.vd.init(max(wave - (NW - Ctx::NLW), 0), lane, a.v_sn, a.D / 8);

  if (t_lo <= x.t_hi) {
    if (wave >= NW - Ctx::NLW) {
      x.kd.issue(x.Kp, a.k_sn, t_lo * BN, a.Nk, smem);
      x.vd.issue(x.Vp, a.v_sn, t_lo * BN, a.Nk, smem + Ctx::TILE);
    }
    wait_all_loads();
  }
  __syncthreads();
  int t = t_lo;
  for (; t + 1 <= x.t_hi; t += 2) {
    x.template step<0>(t);
    x.template step<1>(t + 1);
  }
  if (t <= x.t_hi) x.template step<0>(t);

  if (qrow < a.Nq) {
    uint16_t* dqp = static_cast<uint16_t*>(a.dq) + b * a.q_sb + hq * a.q_sh + (int64_t)qrow * a.q_sn;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * db + 8 * g4 + 4 * hf;
        if (d0 >= a.D) continue;
        *reinterpret_cast<u32x2*>(dqp + d0) =
            u32x2{T::pack(x.dqa[db][4 * g4] * sc, x.dqa[db][4 * g4 + 1] * sc),
                  T::pack(x.dqa[db][4 * g4 + 2] * sc, x.dqa[db][4 * g4 + 3] * sc)};
      }
    }
  }
}

template <class T, int D>
static hipError_t launch_bwd_t(const AttnArgs& a, hipStream_t stream, int stages) {
  hipError_t e = hipSuccess;
  if (stages & kStagePrepare) {
    e = launch_bwd_preprocess(a, stream);
    if (e != hipSuccess) return e;
  }
  AttnArgs args = a;
  args.xcd_remap = a.xcd_remap && ((a.B * a.Hkv) % 8 == 0);
  using WL = DkdvWsLayout<D, FA_DKDV_BMQ>;
  const int n_kt = padded_tiles((a.Nk + WL::BNK - 1) / WL::BNK, work_tiles_per_group(a, 1));
  const int64_t grid_kv = (int64_t)a.B * a.Hkv * n_kt;
  if (grid_kv > 0 && (stages & kStageDkdv)) {
    if (a.mod)
      hipLaunchKernelGGL((bwd_dkdv_ws_kernel<T, D, FA_DKDV_BMQ, true>), dim3((unsigned)grid_kv), dim3(WL::NW * 64),
                         0, stream, args);
    else
      hipLaunchKernelGGL((bwd_dkdv_ws_kernel<T, D, FA_DKDV_BMQ, false>), dim3((unsigned)grid_kv),
                         dim3(WL::NW * 64), 0, stream, args);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  static_assert(FA_DQ_NW == 8, "the dQ kernel pairs query heads over its two halves of 4 waves");
  const int hp = heads_per_workgroup(a), rows = FA_DQ_NW * 32 / hp;
  const int n_qt = padded_tiles((a.Nq + rows - 1) / rows, work_tiles_per_group(a, a.G / hp));
  const int64_t grid_q = (int64_t)a.B * a.Hkv * n_qt * (a.G / hp);
  if (grid_q > 0 && (stages & kStageDq)) {
    if (a.mod)
      // 32-key tiles at d = 128: the modifiers' per-element work does not fit
      // the registers of 64-key tiles there without spilling.
      hipLaunchKernelGGL((bwd_dq_kernel<T, D, (D == 128 ? 32 : FA_DQ_BN), FA_DQ_NW, true>), dim3((unsigned)grid_q),
                         dim3(FA_DQ_NW * 64), 0, stream, args);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<T, D, FA_DQ_BN, FA_DQ_NW, false>), dim3((unsigned)grid_q),
                         dim3(FA_DQ_NW * 64), 0, stream, args);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_bwd_mfma(const AttnArgs& a, hipStream_t stream, int stages) {
  // Head dims below 64 / 128 run the 64 / 128 kernels with the rest masked.
  if (a.dtype == kBF16) {
    if (a.D > 64 && a.D <= 128) return launch_bwd_t<BF16, 128>(a, stream, stages);
    if (a.D >= 8 && a.D <= 64) return launch_bwd_t<BF16, 64>(a, stream, stages);
  } else if (a.dtype == kF16) {
    if (a.D > 64 && a.D <= 128) return launch_bwd_t<F16, 128>(a, stream, stages);
    if (a.D >= 8 && a.D <= 64) return launch_bwd_t<F16, 64>(a, stream, stages);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
