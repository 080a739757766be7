// Global -> register -> LDS staging of 16-bit tiles for the MFMA kernels.
//
// A tile is ROWS x D elements (rows are sequence positions, D contiguous).  With
// NT threads, thread t holds R consecutive rows (R*a .. R*a+R-1, a = t / CPR) of
// one 16-byte column chunk cc = t % CPR (CPR = D / 8 chunks per row), so that
// 16 (D = 128) or 8 (D = 64) consecutive threads read one contiguous row.
//
// The tile is written to LDS either row-major (dst[row][col], pitch P) or
// transposed (dst[col][row], pitch P).  The transposed copy is what a
// 32x32x16 MFMA needs when the sequence axis is its reduction axis: each lane
// then reads 4 consecutive rows of one column with a single 8-byte LDS load.
#pragma once

#include "common.hpp"

namespace fa {

template <int D, int ROWS, int NT>
struct TileRegs {
  static constexpr int CPR = D / 8;
  static constexpr int R = ROWS * CPR / NT;
  static_assert(ROWS * CPR % NT == 0, "tile does not divide over the threads");
  static_assert(R == 2 || R == 4 || R == 8, "unsupported rows per thread");
  u32x4 r[R];

  // Rows row0 .. row0+ROWS-1 of a tensor whose row i starts at base + i*stride;
  // rows at or beyond nrows read as zero.
  __device__ __forceinline__ void load(const uint16_t* base, int64_t stride, int row0, int nrows,
                                       int tid) {
    const int a = tid / CPR, cc = tid % CPR;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int row = row0 + R * a + i;
      if (row < nrows)
        r[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)row * stride + cc * 8);
      else
        r[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  template <int P>
  __device__ __forceinline__ void store_rows(uint16_t* dst, int tid) const {
    static_assert((P * 2) % 16 == 0, "row pitch must keep 16-byte alignment");
    const int a = tid / CPR, cc = tid % CPR;
#pragma unroll
    for (int i = 0; i < R; ++i)
      *reinterpret_cast<u32x4*>(dst + (R * a + i) * P + cc * 8) = r[i];
  }

  template <int P>
  __device__ __forceinline__ void store_cols(uint16_t* dst, int tid) const {
    static_assert((P * 2) % (2 * R) == 0, "column pitch must keep the store aligned");
    const int a = tid / CPR, cc = tid % CPR;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t w[R / 2];
#pragma unroll
      for (int m = 0; m < R / 2; ++m) {
        const uint32_t x = r[2 * m][e >> 1], y = r[2 * m + 1][e >> 1];
        w[m] = (e & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
      }
      uint16_t* p = dst + (cc * 8 + e) * P + R * a;
      if constexpr (R == 2) {
        *reinterpret_cast<uint32_t*>(p) = w[0];
      } else if constexpr (R == 4) {
        *reinterpret_cast<u32x2*>(p) = u32x2{w[0], w[1]};
      } else {
        *reinterpret_cast<u32x4*>(p) = u32x4{w[0], w[1], w[2], w[3]};
      }
    }
  }
};

// Pitches (in elements) of the LDS copies.  Row-major tiles are padded by 16
// bytes per row and transposed tiles by 8 (or 16) bytes, so that the 32 rows
// read by one MFMA operand load fall into different LDS banks.
template <int D>
struct RowPitch {
  static constexpr int value = D + 8;
};
template <int ROWS, int R>
struct ColPitch {
  static constexpr int value = ROWS + (R == 8 ? 8 : 4);
};

// MFMA A/B operand of 8 consecutive elements from a row-major LDS tile.
__device__ __forceinline__ u32x4 lds_row8(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// MFMA operand over the sequence axis from a transposed LDS tile: elements
// 0..3 at p[0..3], elements 4..7 at p[8..11] (the key order of the 32x32
// accumulator rows held by one lane).
__device__ __forceinline__ u32x4 lds_col8(const uint16_t* p) {
  const u32x2 lo = *reinterpret_cast<const u32x2*>(p);
  const u32x2 hi = *reinterpret_cast<const u32x2*>(p + 8);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

}  // namespace fa
