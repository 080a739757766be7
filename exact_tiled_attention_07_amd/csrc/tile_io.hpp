// LDS tile layout and global -> LDS tile loads for the MFMA kernels.
//
// A tile is ROWS x D 16-bit elements (rows are sequence positions, D
// contiguous), stored row-major in LDS with a chunk swizzle and filled by
// direct-to-LDS loads.  MFMA operands are read from it in two ways: 16-byte
// row chunks (operands whose lanes run along the rows) and the transposing
// 8-byte read ds_read_b64_tr_b16 (operands whose reduction axis runs along the
// rows), so no transposed copy of any tile is ever made.
#pragma once

#include "common.hpp"

namespace fa {

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

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Transposing read.  ds_read_b64_tr_b16 hands lane i of each 16-lane group
// element i%4 of the 4-element (8-byte) chunks that lanes {i/4, 4+i/4, 8+i/4,
// 12+i/4} of the group point to.  To build the MFMA operand for rows
// 16*s .. 16*s+15 and columns 32*db .. 32*db+31 -- lane (l32, hf) receiving
// column 32*db + l32 of rows 16*s + {4hf..4hf+3, 8+4hf..8+4hf+3}, the key
// order of a 32x32 accumulator's registers 0..7 (or 8..15) -- lane j of a
// group points at row j/4 of its 4-row block, columns 4*(j%4) .. +3 of its
// 16-column half; two such reads (rows +0 and +8) give the 8 elements.

// Per-lane LDS byte offsets of a swizzled D-wide tile (above):
// row chunks for an operand whose lanes run along the rows (row l32 of each
// 32-row block, chunk 2*st + hf), and the transposing reads for an operand
// whose reduction axis runs along the rows (16-row step 0, column block db,
// lower/upper 8 rows).  Row-block, step and buffer offsets are immediates.
template <int D>
struct SwzOffsets {
  int chunk[D / 16];
  int tr[D / 32][2];
  __device__ __forceinline__ void init(int lane) {
    const int l32 = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) chunk[st] = Swz<D>::off(l32, 2 * st + hf);
    const int G = lane >> 4, j = lane & 15;
    const int vhf = G >> 1, gsub = G & 1, ep = j >> 2, q = j & 3;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int cc = 4 * db + 2 * gsub + (q >> 1);
      tr[db][0] = Swz<D>::off(4 * vhf + ep, cc) + 8 * (q & 1);
      tr[db][1] = Swz<D>::off(8 + 4 * vhf + ep, cc) + 8 * (q & 1);
    }
  }
  // Row chunk operand at row-block rb (32 rows) of the tile at `tile`.
  __device__ __forceinline__ u32x4 row_chunk(const char* tile, int rb, int st) const {
    return *reinterpret_cast<const u32x4*>(tile + rb * 32 * 2 * D + chunk[st]);
  }
  // Transposed operand for 16-row step si and column block db.
  __device__ __forceinline__ u32x4 tr_operand(const char* tile, int si, int db) const {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + si * 16 * 2 * D + tr[db][0]));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + si * 16 * 2 * D + tr[db][1]));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
  }
};

// 16 bytes at element offset col of a row, or zeros where col lies past the
// row's head dim dh (head dims are multiples of 8, so a chunk is all in or all out).
__device__ __forceinline__ u32x4 load_cols(const uint16_t* row, int col, int dh) {
  return col < dh ? *reinterpret_cast<const u32x4*>(row + col) : u32x4{0u, 0u, 0u, 0u};
}

// ===========================================================================
// Direct global -> LDS tile loads (buffer_load_dwordx4 ... lds).
//
// One instruction moves 16 bytes per lane into LDS at (wave-uniform base) +
// 16 * lane, i.e. 1 KB of consecutive LDS per wave.  The swizzled layout above
// is produced by choosing each lane's source offset: LDS chunk slot `lane` of
// 1 KB block j is row j*RPB + lane / CPR, physical chunk lane % CPR, which
// holds logical chunk (lane % CPR) ^ sw(row).  Each lane's byte offsets
// (relative to the tile's first row) are computed once per kernel; a tile
// load then builds one buffer resource from scalars.
//
// The buffer form addresses memory with a scalar resource plus one 32-bit
// lane offset.  On MI355X it issues in about the same time whether or not
// another wave of the SIMD is streaming MFMAs, while global_load_lds with
// 64-bit per-lane addresses measured up to 40x slower to issue in that case.
// Rows past the end of the tensor lie outside the resource's range and read
// as zeros (those keys or queries are masked, and 0 * 0 stays finite).
// ===========================================================================
// Word 3 of a raw buffer resource on this chip family (32-bit data format, no
// swizzle, no stride): loads at or past num_records bytes return zeros.
static constexpr int kRawBufferWord3 = 0x00020000;
// Cache-policy operand of a buffer load: the non-temporal hint.
static constexpr int kNonTemporal = 2;

// The base and size must be the same in every lane; they are read from the
// first lane, so the resource sits in scalar registers (the compiler cannot
// always prove such values uniform and would otherwise loop over lanes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), kRawBufferWord3);
}

// 16 bytes per lane at byte offset voff of resource rs straight into LDS at
// lds_block + 16 * lane (lds_block must be the same for the whole wave).
__device__ __forceinline__ void buffer_dma16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, const void* lds_block) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_block, 16, (int)voff, 0,
                                           0, 0);
}

template <int D, int ROWS, int NW>
struct DmaTile {
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int RPB = 64 / CPR;              // rows per 1 KB block
  static constexpr int NBLK = ROWS / RPB;           // 1 KB blocks per tile
  static constexpr int PER_WAVE = (NBLK + NW - 1) / NW;
  static_assert(ROWS % RPB == 0, "tile rows must fill whole 1 KB blocks");
  uint32_t off[PER_WAVE];  // byte offsets of this lane's chunk in each of its blocks
  uint32_t tail;           // bytes of a row that hold data (16 * dch); wave-uniform
  int wv;                  // this wave's index among the NW loading waves; wave-uniform

  // dch = 16-byte chunks of a row that hold data (head dim / 8, <= D / 8).  A
  // lane whose chunk lies past it loads chunk 0 of the same row instead (valid
  // memory, no per-load test): the kernels pair those LDS columns only with
  // zero register columns or with outputs that are never stored.  Row strides
  // are at most 2^22 elements, so every offset fits 32 bits.  The wave-uniform
  // values are read from the first lane here, so that issue() runs on the
  // scalar unit alone: a vector instruction in it would wait behind the other
  // wave of the SIMD, which is streaming its softmax through the vector unit
  // while this wave finishes its matrix products.
  __device__ __forceinline__ void init(int wave, int lane, int64_t row_stride_elems, int dch = D / 8) {
    const int lane_row = lane / CPR, lane_pc = lane % CPR;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int j = wave + i * NW;
      const int r = j * RPB + lane_row;
      const int c = lane_pc ^ Swz<D>::sw(r);
      off[i] = (uint32_t)(r * row_stride_elems * 2 + (c < dch ? c : 0) * 16);
    }
    tail = __builtin_amdgcn_readfirstlane((uint32_t)dch * 16u);
    wv = __builtin_amdgcn_readfirstlane(wave);
  }
  // Rows row0 .. row0+ROWS-1 of a tensor whose rows start every row_stride
  // elements; rows at or beyond nrows read as zeros.  The resource ends with
  // the data of the last row, so a single row is read whole whatever its
  // stride (a tensor of one row may carry any stride, 0 included).  base,
  // row_stride, row0, nrows and lds_tile must be wave-uniform.
  __device__ __forceinline__ void issue(const uint16_t* base, int64_t row_stride, int row0, int nrows,
                                        uint16_t* lds_tile) const {
    const int rows = min(max(nrows - row0, 0), ROWS);
    const uint32_t bytes = rows > 0 ? (uint32_t)((rows - 1) * row_stride * 2) + tail : 0u;
    dma(raw_rsrc(base + (int64_t)row0 * row_stride, bytes), lds_tile);
  }
  // The same for a tile that holds at least one row (row0 < nrows).  Without
  // the clamp at zero rows the arithmetic stays on the scalar unit; the
  // clamped form above is combined into a vector med3.
  __device__ __forceinline__ void issue_nonempty(const uint16_t* base, int64_t row_stride, int row0, int nrows,
                                                 uint16_t* lds_tile) const {
    const int rows = min(nrows - row0, ROWS);
    const uint32_t bytes = (uint32_t)((rows - 1) * row_stride * 2) + tail;
    dma(raw_rsrc(base + (int64_t)row0 * row_stride, bytes), lds_tile);
  }
  __device__ __forceinline__ void dma(__amdgpu_buffer_rsrc_t rs, uint16_t* lds_tile) const {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int j = wv + i * NW;
      if (NBLK % NW == 0 || j < NBLK) buffer_dma16(rs, off[i], lds_tile + j * 512);
    }
  }
};

// Workgroup barrier that publishes LDS written by ds_write only: this wave's
// LDS accesses are complete when it arrives, while its direct-to-LDS global
// loads may stay in flight (a fence would wait for those too).  The signal
// fences keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left open
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wait until this wave's direct-to-LDS loads (and every other outstanding
// memory operation of the wave) have completed.
__device__ __forceinline__ void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0); }

}  // namespace fa
