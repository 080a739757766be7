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

// ===========================================================================
// Swizzled row-major tiles (no padding, no transposed copy).
//
// A tile of ROWS x D 16-bit elements is stored row-major with its 16-byte
// chunks permuted inside each row: chunk c of row r sits at chunk position
// c ^ sw(r).  The permutation makes three access patterns free of LDS bank
// conflicts (64 banks x 4 bytes):
//   * 16-byte row-chunk reads by 16 lanes on 16 consecutive rows (the MFMA
//     operand whose lanes run along the rows),
//   * transposing 8-byte reads (ds_read_b64_tr_b16) of 4 consecutive rows x
//     4 consecutive chunks per 32 lanes (the MFMA operand whose reduction axis
//     runs along the rows),
//   * the 16-byte chunk writes of the loader.
// ===========================================================================
template <int D>
struct Swz {
  static_assert(D == 64 || D == 128, "swizzle defined for D = 64, 128");
  __device__ __forceinline__ static int sw(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
  // Byte offset of logical chunk c (8 elements) of row r.
  __device__ __forceinline__ static int off(int r, int c) { return r * (2 * D) + 16 * (c ^ sw(r)); }
};

// Global -> registers -> swizzled LDS.  Thread t holds chunk cc = t % CPR of
// rows a + i * (NT / CPR), a = t / CPR, i < R; for a fixed i consecutive
// threads read consecutive 16-byte chunks of consecutive rows.
template <int D, int ROWS, int NT>
struct SwzTile {
  static constexpr int CPR = D / 8;
  static constexpr int RSTRIDE = NT / CPR;
  static constexpr int R = ROWS / RSTRIDE;
  static_assert(ROWS % RSTRIDE == 0 && R >= 1, "tile does not divide over the threads");
  u32x4 r[R];
  int a, cc;

  __device__ __forceinline__ void init(int tid) {
    a = tid / CPR;
    cc = tid % CPR;
  }
  // Rows row0 .. row0+ROWS-1 of a tensor whose row i starts at base + i*stride.
  // Rows at or beyond nrows (>= 1) re-read row nrows-1: such keys are always
  // masked (or are queries whose results are discarded), and a finite copy
  // keeps 0 * value finite.
  __device__ __forceinline__ void load(const uint16_t* base, int64_t stride, int row0, int nrows) {
    const uint16_t* p = base + (int64_t)row0 * stride + (int64_t)a * stride + cc * 8;
    if (row0 + ROWS <= nrows) {
#pragma unroll
      for (int i = 0; i < R; ++i)
        r[i] = *reinterpret_cast<const u32x4*>(p + (int64_t)(i * RSTRIDE) * stride);
    } else {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int row = min(row0 + a + i * RSTRIDE, nrows - 1);
        r[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)row * stride + cc * 8);
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* tile) const {
    char* t = reinterpret_cast<char*>(tile);
#pragma unroll
    for (int i = 0; i < R; ++i)
      *reinterpret_cast<u32x4*>(t + Swz<D>::off(a + i * RSTRIDE, cc)) = r[i];
  }
};

// 8 consecutive elements (logical chunk c) of row r: an MFMA operand whose
// lanes run along the rows.
template <int D>
__device__ __forceinline__ u32x4 swz_chunk(const uint16_t* tile, int r, int c) {
  return *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(tile) + Swz<D>::off(r, c));
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// MFMA operand whose reduction axis runs along the rows, for rows 16*s .. 16*s+15
// and columns 32*db .. 32*db+31 of a swizzled tile: lane (l32, hf) receives
// columns 32*db + l32 of rows 16*s + {4hf..4hf+3, 8+4hf..8+4hf+3} -- the key
// order of a 32x32 accumulator's registers 0..7 (or 8..15) in that lane.
// ds_read_b64_tr_b16 hands lane i of each 16-lane group element i%4 of the
// 4-element chunks that lanes {i/4, 4+i/4, 8+i/4, 12+i/4} point to; so lane j
// of a group points at row (j/4) of its 4-row block, columns 4*(j%4)..+3 of
// its 16-column half.
template <int D>
__device__ __forceinline__ u32x4 swz_tr_operand(const uint16_t* tile, int s, int db, int lane) {
  const int G = lane >> 4, j = lane & 15;
  const int hf = G >> 1, gsub = G & 1, ep = j >> 2, q = j & 3;
  const int r0 = 16 * s + 4 * hf + ep;
  const int c = 4 * db + 2 * gsub + (q >> 1);
  const char* t = reinterpret_cast<const char*>(tile);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(t + Swz<D>::off(r0, c) + 8 * (q & 1)));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(t + Swz<D>::off(r0 + 8, c) + 8 * (q & 1)));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

}  // namespace fa

namespace fa {

// ===========================================================================
// Direct global -> LDS tile loads (global_load_lds_dwordx4).
//
// One instruction moves 16 bytes per lane into LDS at (wave-uniform base) +
// 16 * lane, i.e. 1 KB of consecutive LDS per wave.  The swizzled layout above
// is produced by choosing each lane's global address: LDS chunk slot `lane` of
// 1 KB block j is row j*RPB + lane / CPR, physical chunk lane % CPR, which
// holds logical chunk (lane % CPR) ^ sw(row).  Each lane's byte offsets
// (relative to the tile's first row) are computed once per kernel; a tile
// load then adds one wave-uniform base pointer.
// ===========================================================================
// 16 bytes per lane from global memory straight into LDS at
// lds_block + 16 * lane (lds_block must be the same for the whole wave).
__device__ __forceinline__ void dma16(const void* g, uint16_t* lds_block) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_block, 16, 0, 0);
}

template <int D, int ROWS, int NW>
struct DmaTile {
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int RPB = 64 / CPR;              // rows per 1 KB block
  static constexpr int NBLK = ROWS / RPB;           // 1 KB blocks per tile
  static constexpr int PER_WAVE = (NBLK + NW - 1) / NW;
  static_assert(ROWS % RPB == 0, "tile rows must fill whole 1 KB blocks");
  uint32_t off[PER_WAVE];  // byte offsets of this lane's chunk in each of its blocks
  int lane_row, lane_pc;

  __device__ __forceinline__ void init(int wave, int lane, int64_t row_stride_elems) {
    lane_row = lane / CPR;
    lane_pc = lane % CPR;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int j = wave + i * NW;
      const int r = j * RPB + lane_row;
      const int c = lane_pc ^ Swz<D>::sw(r);
      off[i] = (uint32_t)(r * row_stride_elems * 2 + c * 16);
    }
  }
  // Rows row0 .. row0+ROWS-1 of a tensor whose rows start every row_stride
  // elements.  Rows at or beyond nrows (>= 1) re-read row nrows-1 (those keys
  // are masked; a finite copy keeps 0 * value finite).
  __device__ __forceinline__ void issue(const uint16_t* base, int64_t row_stride, int row0, int nrows,
                                        uint16_t* lds_tile, int wave) const {
    const char* tb = reinterpret_cast<const char*>(base + (int64_t)row0 * row_stride);
    if (row0 + ROWS <= nrows) {
#pragma unroll
      for (int i = 0; i < PER_WAVE; ++i) {
        const int j = wave + i * NW;
        if (NBLK % NW == 0 || j < NBLK) dma16(tb + off[i], lds_tile + j * 512);
      }
    } else {
#pragma unroll
      for (int i = 0; i < PER_WAVE; ++i) {
        const int j = wave + i * NW;
        if (NBLK % NW == 0 || j < NBLK) {
          const int r = j * RPB + lane_row;
          const int row = min(row0 + r, nrows - 1);
          const int c = lane_pc ^ Swz<D>::sw(r);
          dma16(reinterpret_cast<const char*>(base + (int64_t)row * row_stride) + c * 16, lds_tile + j * 512);
        }
      }
    }
  }
};

// Wait until this wave's direct-to-LDS loads (and every other outstanding
// memory operation of the wave) have completed.
__device__ __forceinline__ void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0); }

}  // namespace fa
