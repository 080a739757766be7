// Attention for fp32 inputs on the vector ALU (no down-conversion anywhere).
//
// Same method as the MFMA kernels ([P4] "FlashAttention 实战指南", section
// "长序列注意力为什么会爆内存": tiles in on-chip memory, online softmax,
// recomputation in the backward pass), written for fp32 end to end:
// 256 threads per workgroup, 64x64 tiles of scores, each thread owning a 4x4
// sub-block (rows tr + 16*ii, columns tc + 16*jj) so that a row's 64 scores sit
// in 16 consecutive lanes and are reduced with 4 lane exchanges.
// D is a runtime value (multiple of 4, at most DP); LDS rows are padded to an
// odd pitch so that 16 lanes reading 16 different rows hit 16 different banks.
// Every dot product and long accumulation (scores, dP, O, the row sums, dQ, dK,
// dV) is carried in float64: a product of two fp32 values is exact in fp64,
// and on gfx950 a float64 FMA issues at the same rate as an unpacked fp32 one.
// Sums over thousands of keys or queries therefore round only once, and the
// exponent argument (s - m)*scale*log2(e) is formed before rounding to fp32.
#include "common.hpp"
#include "launch.hpp"

namespace fa {

namespace {

constexpr int kT = 64;  // tile rows and columns

// Load rows row0.. of a (row, D) fp32 tensor into LDS dst[row][0..DP) (pitch P),
// zero-filling rows >= nrows and columns >= D.
template <int DP, int P>
__device__ __forceinline__ void load_rows_f32(float* dst, const float* base, int64_t stride, int row0,
                                              int nrows, int D, int tid) {
  constexpr int C4 = DP / 4;
  for (int idx = tid; idx < kT * C4; idx += 256) {
    const int r = idx / C4, c = (idx % C4) * 4;
    f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
    if (row0 + r < nrows && c < D) v = *reinterpret_cast<const f32x4*>(base + (int64_t)(row0 + r) * stride + c);
    float* d = dst + r * P + c;
    d[0] = v[0];
    d[1] = v[1];
    d[2] = v[2];
    d[3] = v[3];
  }
}

// acc[ii][jj] = sum_c A[tr+16ii][c] * B[tc+16jj][c]   (A, B row-major in LDS), in float64
template <int P>
__device__ __forceinline__ void tile_abt(double (&acc)[4][4], const float* A, const float* B, int D, int tr,
                                         int tc) {
#pragma unroll
  for (int ii = 0; ii < 4; ++ii)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) acc[ii][jj] = 0.0;
  for (int c = 0; c < D; ++c) {
    double x[4], y[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) x[ii] = A[(tr + 16 * ii) * P + c];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) y[jj] = B[(tc + 16 * jj) * P + c];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) acc[ii][jj] = fma(x[ii], y[jj], acc[ii][jj]);
  }
}

// out[ii][jj] += sum_k W[tr+16ii][k] * X[k][tc+16jj]  (W: kT x kT, pitch kT+1; X pitch P),
// accumulated in float64.
template <int DP, int P>
__device__ __forceinline__ void tile_wx(double (&out)[4][DP / 16], const float* W, const float* X, int tr,
                                        int tc) {
  for (int k = 0; k < kT; ++k) {
    double w[4], x[DP / 16];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) w[ii] = W[(tr + 16 * ii) * (kT + 1) + k];
#pragma unroll
    for (int jj = 0; jj < DP / 16; ++jj) x[jj] = X[k * P + tc + 16 * jj];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int jj = 0; jj < DP / 16; ++jj) out[ii][jj] = fma(w[ii], x[jj], out[ii][jj]);
  }
}

__device__ __forceinline__ double row16_max(double x) {
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) x = fmax(x, __shfl_xor(x, off, 16));
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) x += __shfl_xor(x, off, 16);
  return x;
}

template <int DP>
__device__ __forceinline__ void store_rows_f32(float* base, int64_t stride, int row0, int nrows, int D,
                                               const double (&v)[4][DP / 16], double mul, int tr, int tc) {
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int r = row0 + tr + 16 * ii;
    if (r >= nrows) continue;
#pragma unroll
    for (int jj = 0; jj < DP / 16; ++jj) {
      const int cidx = tc + 16 * jj;
      if (cidx < D) base[(int64_t)r * stride + cidx] = (float)(v[ii][jj] * mul);
    }
  }
}

}  // namespace

// Score modifiers in float64 and raw units (logit = scale * s): s clamped to
// +-softcap/scale, then slope/scale * |i' - j| subtracted (common.hpp).
struct ModF64 {
  bool on;
  double cap, slope;
  __device__ ModF64(const AttnArgs& a, int b, int h)
      : on(a.mod != 0),
        cap(a.softcap > 0.f ? (double)a.softcap / (double)a.scale : INFINITY),
        slope(a.alibi ? (double)a.alibi[b * a.alibi_sb + h] / (double)a.scale : 0.0) {}
  // Modified score of raw score s at distance i' - j.
  __device__ __forceinline__ double apply(double s, int dist) const {
    return fmin(fmax(s, -cap), cap) - slope * (double)abs(dist);
  }
  // Whether the clamp passes the gradient at raw score s.
  __device__ __forceinline__ bool pass(double s) const { return fabs(s) < cap; }
};

// ---------------------------------------------------------------------------
// Forward.
// ---------------------------------------------------------------------------
template <int DP>
__global__ __launch_bounds__(256) void f32_fwd_kernel(AttnArgs a) {
  constexpr int P = DP + 1;
  __shared__ float Qs[kT * P], Ks[kT * P], Vs[kT * P], Ps[kT * (kT + 1)];
  const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
  const int n_qt = (a.Nq + kT - 1) / kT;
  const int qt = blockIdx.x % n_qt;
  const int hq = (blockIdx.x / n_qt) % a.Hq;
  const int b = blockIdx.x / (n_qt * a.Hq);
  const int hk = hq / a.G;
  const int q0 = qt * kT;
  bind_seq(a, b);
  if (q0 >= a.Nq) return;  // past the end of a shorter packed sequence (whole workgroup)
  const float* Qp = static_cast<const float*>(a.q) + b * a.q_sb + hq * a.q_sh;
  const float* Kp = static_cast<const float*>(a.k) + b * a.k_sb + hk * a.k_sh;
  const float* Vp = static_cast<const float*>(a.v) + b * a.v_sb + hk * a.v_sh;

  load_rows_f32<DP, P>(Qs, Qp, a.q_sn, q0, a.Nq, a.D, tid);
  int lo[4], hi[4];
  double m[4];
  double l[4];
  double o[4][DP / 16];
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    lo[ii] = key_lo(a, q0 + tr + 16 * ii);
    hi[ii] = key_hi(a, q0 + tr + 16 * ii);
    m[ii] = -INFINITY;
    l[ii] = 0.0;
#pragma unroll
    for (int jj = 0; jj < DP / 16; ++jj) o[ii][jj] = 0.0;
  }
  const int q_last = min(q0 + kT, a.Nq) - 1;
  const int kv_lo = key_lo(a, q0), kv_hi = key_hi(a, q_last);
  const int t_lo = kv_lo / kT, t_hi = (kv_hi >= kv_lo) ? kv_hi / kT : t_lo - 1;
  const double c = (double)a.scale * 1.4426950408889634;
  const ModF64 md(a, b, hq);

  for (int t = t_lo; t <= t_hi; ++t) {
    const int j0 = t * kT;
    __syncthreads();
    load_rows_f32<DP, P>(Ks, Kp, a.k_sn, j0, a.Nk, a.D, tid);
    load_rows_f32<DP, P>(Vs, Vp, a.v_sn, j0, a.Nk, a.D, tid);
    __syncthreads();
    double s[4][4];
    tile_abt<P>(s, Qs, Ks, a.D, tr, tc);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      double mx = -INFINITY;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int key = j0 + tc + 16 * jj;
        if (md.on) s[ii][jj] = md.apply(s[ii][jj], q0 + tr + 16 * ii + a.delta - key);
        if (key < lo[ii] || key > hi[ii]) s[ii][jj] = -INFINITY;
        mx = fmax(mx, s[ii][jj]);
      }
      mx = row16_max(mx);
      const double m_new = fmax(m[ii], mx);
      const double m_use = (m_new == -INFINITY) ? 0.0 : m_new;
      const float alpha = fast_exp2((float)((m[ii] - m_use) * c));
      float rs = 0.f;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float p = fast_exp2((float)((s[ii][jj] - m_use) * c));
        rs += p;
        Ps[(tr + 16 * ii) * (kT + 1) + tc + 16 * jj] = p;
      }
      l[ii] = l[ii] * (double)alpha + (double)row16_sum(rs);
      m[ii] = m_new;
#pragma unroll
      for (int jj = 0; jj < DP / 16; ++jj) o[ii][jj] *= (double)alpha;
    }
    __syncthreads();
    tile_wx<DP, P>(o, Ps, Vs, tr, tc);
  }

  float* Op = static_cast<float*>(a.o) + b * a.o_sb + hq * a.o_sh;
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int r = q0 + tr + 16 * ii;
    if (r < a.Nq) {
#pragma unroll
      for (int jj = 0; jj < DP / 16; ++jj) {
        const int cidx = tc + 16 * jj;
        if (cidx < a.D) Op[(int64_t)r * a.o_sn + cidx] = (l[ii] > 0.0) ? (float)(o[ii][jj] / l[ii]) : 0.f;
      }
      if (tc == 0)
        a.lse[b * a.lse_sb + hq * a.lse_sh + r] =
            (l[ii] > 0.0) ? (float)(m[ii] * a.scale + log(l[ii])) : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// Backward: dQ per query tile.
// ---------------------------------------------------------------------------
template <int DP>
__global__ __launch_bounds__(256) void f32_bwd_dq_kernel(AttnArgs a) {
  constexpr int P = DP + 1;
  __shared__ float Qs[kT * P], dOs[kT * P], Ks[kT * P], Vs[kT * P], Ps[kT * (kT + 1)];
  const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
  const int n_qt = (a.Nq + kT - 1) / kT;
  const int qt = blockIdx.x % n_qt;
  const int hq = (blockIdx.x / n_qt) % a.Hq;
  const int b = blockIdx.x / (n_qt * a.Hq);
  const int hk = hq / a.G;
  const int q0 = qt * kT;
  bind_seq(a, b);
  if (q0 >= a.Nq) return;  // past the end of a shorter packed sequence (whole workgroup)
  const float* Qp = static_cast<const float*>(a.q) + b * a.q_sb + hq * a.q_sh;
  const float* dOp = static_cast<const float*>(a.dout) + b * a.o_sb + hq * a.o_sh;
  const float* Kp = static_cast<const float*>(a.k) + b * a.k_sb + hk * a.k_sh;
  const float* Vp = static_cast<const float*>(a.v) + b * a.v_sb + hk * a.v_sh;
  load_rows_f32<DP, P>(Qs, Qp, a.q_sn, q0, a.Nq, a.D, tid);
  load_rows_f32<DP, P>(dOs, dOp, a.o_sn, q0, a.Nq, a.D, tid);

  int lo[4], hi[4];
  double lse2[4], dsum[4];
  double dq[4][DP / 16];
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int r = q0 + tr + 16 * ii;
    lo[ii] = key_lo(a, r);
    hi[ii] = key_hi(a, r);
    const int64_t ri = b * a.lse_sb + hq * a.lse_sh + r;
    const int64_t rp = b * a.ws_sb + hq * a.ws_sh + r;  // workspace row
    const float L = (r < a.Nq) ? a.lse[ri] : -INFINITY;
    lse2[ii] = (L == -INFINITY) ? INFINITY : (double)L * 1.4426950408889634;
    dsum[ii] = (r < a.Nq) ? (double)a.dsum[rp] : 0.0;
#pragma unroll
    for (int jj = 0; jj < DP / 16; ++jj) dq[ii][jj] = 0.0;
  }
  const int q_last = min(q0 + kT, a.Nq) - 1;
  const int kv_lo = key_lo(a, q0), kv_hi = key_hi(a, q_last);
  const int t_lo = kv_lo / kT, t_hi = (kv_hi >= kv_lo) ? kv_hi / kT : t_lo - 1;
  const double c = (double)a.scale * 1.4426950408889634;
  const ModF64 md(a, b, hq);

  for (int t = t_lo; t <= t_hi; ++t) {
    const int j0 = t * kT;
    __syncthreads();
    load_rows_f32<DP, P>(Ks, Kp, a.k_sn, j0, a.Nk, a.D, tid);
    load_rows_f32<DP, P>(Vs, Vp, a.v_sn, j0, a.Nk, a.D, tid);
    __syncthreads();
    double s[4][4], dp[4][4];
    tile_abt<P>(s, Qs, Ks, a.D, tr, tc);
    tile_abt<P>(dp, dOs, Vs, a.D, tr, tc);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int key = j0 + tc + 16 * jj;
        bool pass = true;
        if (md.on) {
          pass = md.pass(s[ii][jj]);
          s[ii][jj] = md.apply(s[ii][jj], q0 + tr + 16 * ii + a.delta - key);
        }
        const bool vis = key >= lo[ii] && key <= hi[ii];
        const double p = vis ? (double)fast_exp2((float)(s[ii][jj] * c - lse2[ii])) : 0.0;
        Ps[(tr + 16 * ii) * (kT + 1) + tc + 16 * jj] = pass ? (float)(p * (dp[ii][jj] - dsum[ii])) : 0.f;
      }
    }
    __syncthreads();
    tile_wx<DP, P>(dq, Ps, Ks, tr, tc);
  }
  float* dQp = static_cast<float*>(a.dq) + b * a.q_sb + hq * a.q_sh;
  store_rows_f32<DP>(dQp, a.q_sn, q0, a.Nq, a.D, dq, (double)a.scale, tr, tc);
}

// ---------------------------------------------------------------------------
// Backward: dK and dV per key tile (the transposed problem: rows are keys).
// ---------------------------------------------------------------------------
template <int DP>
__global__ __launch_bounds__(256) void f32_bwd_dkdv_kernel(AttnArgs a) {
  constexpr int P = DP + 1;
  __shared__ float Ks[kT * P], Vs[kT * P], Qs[kT * P], dOs[kT * P], Ps[kT * (kT + 1)];
  __shared__ double lse2s[kT], dsums[kT];
  const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
  const int n_kt = (a.Nk + kT - 1) / kT;
  const int kt = blockIdx.x % n_kt;
  const int hk = (blockIdx.x / n_kt) % a.Hkv;
  const int b = blockIdx.x / (n_kt * a.Hkv);
  const int k0 = kt * kT;
  bind_seq(a, b);
  if (k0 >= a.Nk) return;  // past the end of a shorter packed sequence (whole workgroup)
  const float* Kp = static_cast<const float*>(a.k) + b * a.k_sb + hk * a.k_sh;
  const float* Vp = static_cast<const float*>(a.v) + b * a.v_sb + hk * a.v_sh;
  load_rows_f32<DP, P>(Ks, Kp, a.k_sn, k0, a.Nk, a.D, tid);
  load_rows_f32<DP, P>(Vs, Vp, a.v_sn, k0, a.Nk, a.D, tid);

  double dk[4][DP / 16], dv[4][DP / 16];
#pragma unroll
  for (int ii = 0; ii < 4; ++ii)
#pragma unroll
    for (int jj = 0; jj < DP / 16; ++jj) dk[ii][jj] = dv[ii][jj] = 0.0;

  const int k_last = min(k0 + kT, a.Nk) - 1;
  const int i_lo = query_lo(a, k0), i_hi = query_hi(a, k_last);
  const int t_lo = i_lo / kT, t_hi = (i_hi >= i_lo) ? i_hi / kT : t_lo - 1;
  const double c = (double)a.scale * 1.4426950408889634;

  for (int g = 0; g < a.G; ++g) {
    const int hq = hk * a.G + g;
    const ModF64 md(a, b, hq);
    const float* Qp = static_cast<const float*>(a.q) + b * a.q_sb + hq * a.q_sh;
    const float* dOp = static_cast<const float*>(a.dout) + b * a.o_sb + hq * a.o_sh;
    const int64_t rbase = b * a.lse_sb + hq * a.lse_sh;
    const int64_t pbase = b * a.ws_sb + hq * a.ws_sh;  // workspace rows
    for (int t = t_lo; t <= t_hi; ++t) {
      const int i0 = t * kT;
      __syncthreads();
      load_rows_f32<DP, P>(Qs, Qp, a.q_sn, i0, a.Nq, a.D, tid);
      load_rows_f32<DP, P>(dOs, dOp, a.o_sn, i0, a.Nq, a.D, tid);
      if (tid < kT) {
        const int i = i0 + tid;
        const float L = (i < a.Nq) ? a.lse[rbase + i] : -INFINITY;
        lse2s[tid] = (L == -INFINITY) ? INFINITY : (double)L * 1.4426950408889634;
        dsums[tid] = (i < a.Nq) ? (double)a.dsum[pbase + i] : 0.0;
      }
      __syncthreads();
      // S^T[key][query] and dP^T[key][query].
      double s[4][4], dp[4][4];
      float ds[4][4];
      tile_abt<P>(s, Ks, Qs, a.D, tr, tc);
      tile_abt<P>(dp, Vs, dOs, a.D, tr, tc);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int i = i0 + tc + 16 * jj;
        const int lo = key_lo(a, i), hi = key_hi(a, i);
        const double l2 = lse2s[tc + 16 * jj], dd = dsums[tc + 16 * jj];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int key = k0 + tr + 16 * ii;
          bool pass = true;
          if (md.on) {
            pass = md.pass(s[ii][jj]);
            s[ii][jj] = md.apply(s[ii][jj], i + a.delta - key);
          }
          const bool vis = key >= lo && key <= hi;
          const float p = vis ? fast_exp2((float)(s[ii][jj] * c - l2)) : 0.f;
          Ps[(tr + 16 * ii) * (kT + 1) + tc + 16 * jj] = p;
          ds[ii][jj] = pass ? (float)((double)p * (dp[ii][jj] - dd)) : 0.f;
        }
      }
      __syncthreads();
      tile_wx<DP, P>(dv, Ps, dOs, tr, tc);
      __syncthreads();
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) Ps[(tr + 16 * ii) * (kT + 1) + tc + 16 * jj] = ds[ii][jj];
      __syncthreads();
      tile_wx<DP, P>(dk, Ps, Qs, tr, tc);
    }
  }
  float* dKp = static_cast<float*>(a.dk) + b * a.k_sb + hk * a.k_sh;
  float* dVp = static_cast<float*>(a.dv) + b * a.v_sb + hk * a.v_sh;
  store_rows_f32<DP>(dKp, a.k_sn, k0, a.Nk, a.D, dk, (double)a.scale, tr, tc);
  store_rows_f32<DP>(dVp, a.v_sn, k0, a.Nk, a.D, dv, 1.0, tr, tc);
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
hipError_t launch_fwd_f32(const AttnArgs& a, hipStream_t stream) {
  const int64_t grid = (int64_t)a.B * a.Hq * ((a.Nq + kT - 1) / kT);
  if (grid == 0) return hipSuccess;
  if (a.D <= 64)
    hipLaunchKernelGGL(f32_fwd_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(f32_fwd_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_f32(const AttnArgs& a, hipStream_t stream, int stages) {
  hipError_t e = hipSuccess;
  if (stages & kStagePrepare) {
    e = launch_bwd_preprocess(a, stream);
    if (e != hipSuccess) return e;
  }
  const int64_t grid_kv = (int64_t)a.B * a.Hkv * ((a.Nk + kT - 1) / kT);
  if (grid_kv > 0 && (stages & kStageDkdv)) {
    if (a.D <= 64)
      hipLaunchKernelGGL(f32_bwd_dkdv_kernel<64>, dim3((unsigned)grid_kv), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(f32_bwd_dkdv_kernel<128>, dim3((unsigned)grid_kv), dim3(256), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t grid_q = (int64_t)a.B * a.Hq * ((a.Nq + kT - 1) / kT);
  if (grid_q > 0 && (stages & kStageDq)) {
    if (a.D <= 64)
      hipLaunchKernelGGL(f32_bwd_dq_kernel<64>, dim3((unsigned)grid_q), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(f32_bwd_dq_kernel<128>, dim3((unsigned)grid_q), dim3(256), 0, stream, a);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace fa
