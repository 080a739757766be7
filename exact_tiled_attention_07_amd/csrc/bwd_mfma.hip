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
//   dK/dV       one workgroup per (batch, kv head, tile of 32*NW keys); each
//               wave keeps its 32 keys' K and V in registers and its dK^T, dV^T
//               accumulators in registers, loops over the query heads of the
//               group and the visible query tiles (one pipelined loop):
//                 S  = Q K^T        (A = Q row chunks in LDS, B = K registers)
//                 dP = dO V^T       (A = dO row chunks in LDS, B = V registers)
//                 dV^T += dO^T P    (A = dO read transposed from LDS, B = P)
//                 dK^T += Q^T dS    (A = Q read transposed from LDS, B = dS)
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
// D_i = sum_c dout[i, c] * o[i, c]   (any dtype; 16 lanes per row)
// ---------------------------------------------------------------------------
template <int ELT>  // element bytes: 4 (fp32) or 2 (fp16/bf16)
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(AttnArgs a) {
  constexpr int EPC = 16 / ELT;  // elements per 16-byte chunk
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const int64_t rows = (int64_t)a.B * a.Nq * a.Hq;
  // fp32 inputs accumulate in float64 (exact products); 16-bit inputs in fp32.
  using Acc = typename std::conditional<ELT == 4, double, float>::type;
  Acc acc = 0;
  int h = 0, i = 0, b = 0;
  if (row < rows) {
    h = (int)(row % a.Hq);
    const int64_t t = row / a.Hq;
    i = (int)(t % a.Nq);
    b = (int)(t / a.Nq);
    const char* dop = static_cast<const char*>(a.dout) +
                      (b * a.o_sb + (int64_t)i * a.o_sn + h * a.o_sh) * ELT;
    const char* op = static_cast<const char*>(a.o) + (b * a.o_sb + (int64_t)i * a.o_sn + h * a.o_sh) * ELT;
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
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
  if (row < rows && sub == 0) a.dsum[((int64_t)b * a.Hq + h) * a.Nq + i] = (float)acc;
}

hipError_t launch_bwd_preprocess(const AttnArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.Nq * a.Hq;
  if (rows == 0) return hipSuccess;
  const unsigned grid = (unsigned)((rows + 15) / 16);
  if (a.dtype == kF32)
    hipLaunchKernelGGL(bwd_preprocess_kernel<4>, dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_preprocess_kernel<2>, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// log2-domain LSE of a query row; a row that sees no key (LSE = -inf) gets +inf
// so that every recomputed probability exp2(s*c - lse2) of it is exactly 0.
__device__ __forceinline__ float lse_log2(float lse) {
  return (lse == -INFINITY) ? INFINITY : lse * kLog2e;
}

// ---------------------------------------------------------------------------
// dK / dV
// ---------------------------------------------------------------------------
template <class T, int D, int BMQ, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dkdv_kernel(AttnArgs a) {
  constexpr int NT = NW * 64;
  constexpr int BNK = NW * 32;  // keys per workgroup
  constexpr int TILE = BMQ * D;
  using Tile = SwzTile<D, BMQ, NT>;
  // Two buffers of (Q tile, dO tile), swizzled row-major, plus per-row LSE/D.
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * TILE];
  __shared__ __attribute__((aligned(16))) float rowstat[2][2][BMQ];  // [buf][lse2, D][row]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;

  const int n_kt = (a.Nk + BNK - 1) / BNK;
  // Under a causal mask the first key tiles see the most queries: run them first.
  const WorkItem it = decode_work(blockIdx.x, a.B * a.Hkv, n_kt, 1, false, a.xcd_remap);
  const int b = it.unit / a.Hkv, hk = it.unit % a.Hkv;
  const int k0 = it.tile * BNK;
  const int key = k0 + wave * 32 + l32;  // this lane's key (accumulator column)

  const uint16_t* Kp = static_cast<const uint16_t*>(a.k) + b * a.k_sb + hk * a.k_sh;
  const uint16_t* Vp = static_cast<const uint16_t*>(a.v) + b * a.v_sb + hk * a.v_sh;

  // K and V as B operands (lane: key, d = 16*st + 8*hf + 0..7).
  u32x4 kf[D / 16], vf[D / 16];
  if (key < a.Nk) {
    const uint16_t* kr = Kp + (int64_t)key * a.k_sn + 8 * hf;
    const uint16_t* vr = Vp + (int64_t)key * a.v_sn + 8 * hf;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      kf[st] = *reinterpret_cast<const u32x4*>(kr + 16 * st);
      vf[st] = *reinterpret_cast<const u32x4*>(vr + 16 * st);
    }
  } else {
#pragma unroll
    for (int st = 0; st < D / 16; ++st) kf[st] = vf[st] = u32x4{0u, 0u, 0u, 0u};
  }

  f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dka[db] = dva[db] = f32x16{};

  const int k_last = min(k0 + BNK, a.Nk) - 1;
  const int i_lo = query_lo(a, k0), i_hi = query_hi(a, k_last);
  const int qt_lo = i_lo / BMQ;
  const int n_qt = (i_hi >= i_lo) ? i_hi / BMQ - qt_lo + 1 : 0;
  const int n_items = n_qt * a.G;  // (query head of the group, query tile) pairs
  const float c = a.scale_log2;

  // Loader state for work item w: head hk*G + w / n_qt, tile qt_lo + w % n_qt.
  Tile qt, dt;
  qt.init(tid);
  dt.init(tid);
  float st_lse = INFINITY, st_d = 0.f;
  auto load_item = [&](int w) {
    const int g = w / n_qt, i0 = (qt_lo + w % n_qt) * BMQ;
    const int hq = hk * a.G + g;
    qt.load(static_cast<const uint16_t*>(a.q) + b * a.q_sb + hq * a.q_sh, a.q_sn, i0, a.Nq);
    dt.load(static_cast<const uint16_t*>(a.dout) + b * a.o_sb + hq * a.o_sh, a.o_sn, i0, a.Nq);
    if (tid < BMQ) {
      const int i = i0 + tid;
      const int64_t ri = ((int64_t)b * a.Hq + hq) * a.Nq + i;
      st_lse = (i < a.Nq) ? lse_log2(a.lse[ri]) : INFINITY;
      st_d = (i < a.Nq) ? a.dsum[ri] : 0.f;
    }
  };
  auto store_item = [&](int buf) {
    qt.store(smem + buf * 2 * TILE);
    dt.store(smem + buf * 2 * TILE + TILE);
    if (tid < BMQ) {
      rowstat[buf][0][tid] = st_lse;
      rowstat[buf][1][tid] = st_d;
    }
  };

  if (n_items > 0) {
    load_item(0);
    store_item(0);
  }
  __syncthreads();
  if (n_items > 1) load_item(1);

  for (int w = 0; w < n_items; ++w) {
    const int buf = w & 1;
    const int i0 = (qt_lo + w % n_qt) * BMQ;
    const uint16_t* Qs = smem + buf * 2 * TILE;
    const uint16_t* dOs = Qs + TILE;
    const float* lse2s = rowstat[buf][0];
    const float* dsums = rowstat[buf][1];

    // S = Q K^T; s[qb][r] is query i0 + 32*qb + 8*(r/4) + 4*hf + r%4.
    f32x16 s[BMQ / 32];
#pragma unroll
    for (int qb = 0; qb < BMQ / 32; ++qb) s[qb] = f32x16{};
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
#pragma unroll
      for (int qb = 0; qb < BMQ / 32; ++qb)
        s[qb] = T::mfma(swz_chunk<D>(Qs, 32 * qb + l32, 2 * st + hf), kf[st], s[qb]);
    }
    // dP = dO V^T (independent of S, issued before the softmax math).
    f32x16 dp[BMQ / 32];
#pragma unroll
    for (int qb = 0; qb < BMQ / 32; ++qb) dp[qb] = f32x16{};
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
#pragma unroll
      for (int qb = 0; qb < BMQ / 32; ++qb)
        dp[qb] = T::mfma(swz_chunk<D>(dOs, 32 * qb + l32, 2 * st + hf), vf[st], dp[qb]);
    }
    // Mask: exact per-element test only where the tile pair is not fully visible.
    const int i_end = min(i0 + BMQ, a.Nq) - 1;
    const bool full = (key_lo(a, i_end) <= k0) && (key_hi(a, i0) >= k_last);
    if (!full) {
#pragma unroll
      for (int qb = 0; qb < BMQ / 32; ++qb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = i0 + 32 * qb + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (key < key_lo(a, i) || key > key_hi(a, i)) s[qb][r] = -INFINITY;
        }
      }
    }
    // P = exp2(s*c - lse2) and dS = P * (dP - D), both as B operands.
    u32x4 pf[BMQ / 16], dsf[BMQ / 16];
#pragma unroll
    for (int qb = 0; qb < BMQ / 32; ++qb) {
      float p[16], ds[16];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2s + 32 * qb + 8 * g4 + 4 * hf);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dsums + 32 * qb + 8 * g4 + 4 * hf);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g4 + e;
          p[r] = fast_exp2(fmaf(s[qb][r], c, -l4[e]));
          ds[r] = p[r] * (dp[qb][r] - d4[e]);
        }
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const float* pp = &p[8 * tt];
        const float* qq = &ds[8 * tt];
        pf[2 * qb + tt] = u32x4{T::pack(pp[0], pp[1]), T::pack(pp[2], pp[3]), T::pack(pp[4], pp[5]),
                                T::pack(pp[6], pp[7])};
        dsf[2 * qb + tt] = u32x4{T::pack(qq[0], qq[1]), T::pack(qq[2], qq[3]), T::pack(qq[4], qq[5]),
                                 T::pack(qq[6], qq[7])};
      }
    }
    // dV^T += dO^T P and dK^T += Q^T dS, operands read transposed from the tiles.
#pragma unroll
    for (int si = 0; si < BMQ / 16; ++si) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        dva[db] = T::mfma(swz_tr_operand<D>(dOs, si, db, lane), pf[si], dva[db]);
        dka[db] = T::mfma(swz_tr_operand<D>(Qs, si, db, lane), dsf[si], dka[db]);
      }
    }

    if (w + 1 < n_items) store_item(buf ^ 1);
    __syncthreads();
    if (w + 2 < n_items) load_item(w + 2);
  }

  // Store dK = scale * dK and dV: lane holds d rows 32*db + 8*g4 + 4*hf + 0..3.
  if (key < a.Nk) {
    uint16_t* dkp = static_cast<uint16_t*>(a.dk) + b * a.k_sb + hk * a.k_sh + (int64_t)key * a.k_sn;
    uint16_t* dvp = static_cast<uint16_t*>(a.dv) + b * a.v_sb + hk * a.v_sh + (int64_t)key * a.v_sn;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * db + 8 * g4 + 4 * hf;
        *reinterpret_cast<u32x2*>(dkp + d0) =
            u32x2{T::pack(dka[db][4 * g4] * sc, dka[db][4 * g4 + 1] * sc),
                  T::pack(dka[db][4 * g4 + 2] * sc, dka[db][4 * g4 + 3] * sc)};
        *reinterpret_cast<u32x2*>(dvp + d0) =
            u32x2{T::pack(dva[db][4 * g4], dva[db][4 * g4 + 1]), T::pack(dva[db][4 * g4 + 2], dva[db][4 * g4 + 3])};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <class T, int D, int BN, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dq_kernel(AttnArgs a) {
  constexpr int NT = NW * 64;
  constexpr int BM = NW * 32;
  constexpr int TILE = BN * D;
  using Tile = SwzTile<D, BN, NT>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * TILE];  // [buf][K, V]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;

  const int n_qt = (a.Nq + BM - 1) / BM;
  const bool heavy_last = (a.causal || a.wr >= 0) && a.wl < 0;
  const WorkItem it = decode_work(blockIdx.x, a.B * a.Hkv, n_qt, a.G, heavy_last, a.xcd_remap);
  const int b = it.unit / a.Hkv, hk = it.unit % a.Hkv;
  const int hq = hk * a.G + it.sub;
  const int q0 = it.tile * BM;
  const int qrow = q0 + wave * 32 + l32;

  const uint16_t* Qp = static_cast<const uint16_t*>(a.q) + b * a.q_sb + hq * a.q_sh;
  const uint16_t* dOp = static_cast<const uint16_t*>(a.dout) + b * a.o_sb + hq * a.o_sh;
  const uint16_t* Kp = static_cast<const uint16_t*>(a.k) + b * a.k_sb + hk * a.k_sh;
  const uint16_t* Vp = static_cast<const uint16_t*>(a.v) + b * a.v_sb + hk * a.v_sh;

  u32x4 qf[D / 16], df[D / 16];
  float lse2 = INFINITY, dsum = 0.f;
  if (qrow < a.Nq) {
    const uint16_t* qr = Qp + (int64_t)qrow * a.q_sn + 8 * hf;
    const uint16_t* dr = dOp + (int64_t)qrow * a.o_sn + 8 * hf;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      qf[st] = *reinterpret_cast<const u32x4*>(qr + 16 * st);
      df[st] = *reinterpret_cast<const u32x4*>(dr + 16 * st);
    }
    const int64_t ri = ((int64_t)b * a.Hq + hq) * a.Nq + qrow;
    lse2 = lse_log2(a.lse[ri]);
    dsum = a.dsum[ri];
  } else {
#pragma unroll
    for (int st = 0; st < D / 16; ++st) qf[st] = df[st] = u32x4{0u, 0u, 0u, 0u};
  }

  const int lo_i = key_lo(a, qrow), hi_i = key_hi(a, qrow);
  const int q_last = min(q0 + BM, a.Nq) - 1;
  const int kv_lo = key_lo(a, q0), kv_hi = key_hi(a, q_last);
  const int lo_max = key_lo(a, q_last), hi_min = key_hi(a, q0);
  const int t_lo = kv_lo / BN;
  const int t_hi = (kv_hi >= kv_lo) ? kv_hi / BN : t_lo - 1;
  const float c = a.scale_log2;

  f32x16 dqa[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dqa[db] = f32x16{};

  Tile kt, vt;
  kt.init(tid);
  vt.init(tid);
  if (t_lo <= t_hi) {
    kt.load(Kp, a.k_sn, t_lo * BN, a.Nk);
    vt.load(Vp, a.v_sn, t_lo * BN, a.Nk);
    kt.store(smem);
    vt.store(smem + TILE);
  }
  __syncthreads();
  if (t_lo + 1 <= t_hi) {
    kt.load(Kp, a.k_sn, (t_lo + 1) * BN, a.Nk);
    vt.load(Vp, a.v_sn, (t_lo + 1) * BN, a.Nk);
  }
  for (int t = t_lo; t <= t_hi; ++t) {
    const int j0 = t * BN;
    const int buf = (t - t_lo) & 1;
    const uint16_t* Ks = smem + buf * 2 * TILE;
    const uint16_t* Vs = Ks + TILE;
    // S^T = K Q^T and dP^T = V dO^T; element [kb][r] is key j0 + 32*kb + 8*(r/4) + 4*hf + r%4.
    f32x16 s[BN / 32], dp[BN / 32];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) s[kb] = dp[kb] = f32x16{};
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
        s[kb] = T::mfma(swz_chunk<D>(Ks, 32 * kb + l32, 2 * st + hf), qf[st], s[kb]);
        dp[kb] = T::mfma(swz_chunk<D>(Vs, 32 * kb + l32, 2 * st + hf), df[st], dp[kb]);
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
    // dS^T = P^T * (dP^T - D) as B operands, then dQ^T += K^T dS^T.
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
#pragma unroll
    for (int si = 0; si < BN / 16; ++si) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        dqa[db] = T::mfma(swz_tr_operand<D>(Ks, si, db, lane), dsf[si], dqa[db]);
    }

    if (t < t_hi) {
      kt.store(smem + (buf ^ 1) * 2 * TILE);
      vt.store(smem + (buf ^ 1) * 2 * TILE + TILE);
    }
    __syncthreads();
    if (t + 2 <= t_hi) {
      kt.load(Kp, a.k_sn, j0 + 2 * BN, a.Nk);
      vt.load(Vp, a.v_sn, j0 + 2 * BN, a.Nk);
    }
  }

  if (qrow < a.Nq) {
    uint16_t* dqp = static_cast<uint16_t*>(a.dq) + b * a.q_sb + hq * a.q_sh + (int64_t)qrow * a.q_sn;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * db + 8 * g4 + 4 * hf;
        *reinterpret_cast<u32x2*>(dqp + d0) =
            u32x2{T::pack(dqa[db][4 * g4] * sc, dqa[db][4 * g4 + 1] * sc),
                  T::pack(dqa[db][4 * g4 + 2] * sc, dqa[db][4 * g4 + 3] * sc)};
      }
    }
  }
}

template <class T, int D>
static hipError_t launch_bwd_t(const AttnArgs& a, hipStream_t stream) {
  constexpr int NW = 4;
  constexpr int BMQ = 64;        // queries per dK/dV iteration
  constexpr int BN_DQ = 64;      // keys per dQ iteration
  hipError_t e = launch_bwd_preprocess(a, stream);
  if (e != hipSuccess) return e;
  AttnArgs args = a;
  args.xcd_remap = a.xcd_remap && ((a.B * a.Hkv) % 8 == 0);
  const int n_kt = (a.Nk + NW * 32 - 1) / (NW * 32);
  const int64_t grid_kv = (int64_t)a.B * a.Hkv * n_kt;
  if (grid_kv > 0) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, BMQ, NW>), dim3((unsigned)grid_kv), dim3(NW * 64), 0,
                       stream, args);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int n_qt = (a.Nq + NW * 32 - 1) / (NW * 32);
  const int64_t grid_q = (int64_t)a.B * a.Hkv * n_qt * a.G;
  if (grid_q > 0) {
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, BN_DQ, NW>), dim3((unsigned)grid_q), dim3(NW * 64), 0,
                       stream, args);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_bwd_mfma(const AttnArgs& a, hipStream_t stream) {
  if (a.dtype == kBF16) {
    if (a.D == 128) return launch_bwd_t<BF16, 128>(a, stream);
    if (a.D == 64) return launch_bwd_t<BF16, 64>(a, stream);
  } else if (a.dtype == kF16) {
    if (a.D == 128) return launch_bwd_t<F16, 128>(a, stream);
    if (a.D == 64) return launch_bwd_t<F16, 64>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
