// Tile movement between HBM and LDS for the [B][N][H][d] token-major layout.
//
// A tile is ROWS consecutive tokens of one (batch, head), all D dims. It is fetched as
// "items" of 4 rows x 8 dims: each thread issues four 16-byte buffer loads (consecutive
// threads take consecutive 16-byte chunks of a row, so a wave reads whole rows). Rows past
// the end of the sequence read as zeros through the buffer range check.
//
// The registers can be written to LDS in two layouts:
//  * row-major  [row][dim], row pitch D*2 + 16 bytes (the pad spreads a 32-row column read
//    over distinct banks) - the operand layout when the contraction runs over dims;
//  * transposed [dim][pos], pos = swap23(row) within each 32-row block, 16-byte groups
//    XOR-swizzled by dim - the operand layout when the contraction runs over rows, with
//    rows in the order in which a 32x32 MFMA accumulator hands them to the next product.
#pragma once
#include "attn_device.h"

namespace attn {

// Position of rows 4*kg .. 4*kg+3 in the transposed layout: bits 0 and 1 of kg swap, which
// swaps bits 2 and 3 of the row index.
__device__ __forceinline__ int swap01(int x) { return (x & ~3) | ((x & 1) << 1) | ((x >> 1) & 1); }

// XOR swizzle of the 16-byte group index for transposed row `d` (NG groups per row).
template <int NG>
__device__ __forceinline__ int tswz(int d) {
  if constexpr (NG == 4) return (d ^ (d >> 2)) & 3;
  else if constexpr (NG == 8) return (d ^ (d >> 3)) & 7;
  else return (d ^ (d >> 4)) & 15;
}

template <int D>
constexpr int rm_pitch() { return D * 2 + 16; }

template <int D, int ROWS>
struct Tile {
  static constexpr int ITEMS = (ROWS / 4) * (D / 8);
  static constexpr int NIT = (ITEMS + 255) / 256;
  static constexpr int NG = ROWS / 8;          // 16-byte groups per transposed row
  static constexpr int TPITCH = ROWS * 2;      // transposed row pitch (bytes)
  static constexpr int RM_BYTES = ROWS * rm_pitch<D>();
  static constexpr int T_BYTES = D * TPITCH;
  u32x4 r[NIT][4];

  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int row0, uint32_t row_bytes, int tid) {
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int i = tid + 256 * it;
      if (ITEMS % 256 == 0 || i < ITEMS) {
        const int c8 = i % (D / 8), rg = i / (D / 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) r[it][j] = buf_load16(rs, (uint32_t)(row0 + 4 * rg + j) * row_bytes + c8 * 16);
      }
    }
  }
  __device__ __forceinline__ void store_rowmajor(char* dst, int tid) const {
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int i = tid + 256 * it;
      if (ITEMS % 256 == 0 || i < ITEMS) {
        const int c8 = i % (D / 8), rg = i / (D / 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) *(u32x4*)(dst + (4 * rg + j) * rm_pitch<D>() + c8 * 16) = r[it][j];
      }
    }
  }
  __device__ __forceinline__ void store_transposed(char* dst, int tid) const {
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int i = tid + 256 * it;
      if (ITEMS % 256 == 0 || i < ITEMS) {
        const int c8 = i % (D / 8), rg = i / (D / 8);
        const int pg = swap01(rg);
        const int g = pg >> 1, off8 = (pg & 1) * 8;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t a0 = r[it][0][w], a1 = r[it][1][w], a2 = r[it][2][w], a3 = r[it][3][w];
          const int d0 = c8 * 8 + 2 * w;
          const u32x2 lo = {(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
          const u32x2 hi = {(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
          *(u32x2*)(dst + d0 * TPITCH + ((g ^ tswz<NG>(d0)) & (NG - 1)) * 16 + off8) = lo;
          *(u32x2*)(dst + (d0 + 1) * TPITCH + ((g ^ tswz<NG>(d0 + 1)) & (NG - 1)) * 16 + off8) = hi;
        }
      }
    }
  }
};

// Operand reads (lane l: l32 = l % 32, hf = l / 32).
// Row-major tile, A/B operand over dims: row `row`, dims 16*ks + 8*hf .. +7.
template <int D>
__device__ __forceinline__ u32x4 read_rm(const char* base, int row, int ks, int hf) {
  return *(const u32x4*)(base + row * rm_pitch<D>() + (16 * ks + 8 * hf) * 2);
}
// Transposed tile, A operand over rows: dim `d`, positions 16*c + 8*hf .. +7.
template <int ROWS>
__device__ __forceinline__ u32x4 read_t(const char* base, int d, int c, int hf) {
  constexpr int NG = ROWS / 8;
  return *(const u32x4*)(base + d * (ROWS * 2) + (((2 * c + hf) ^ tswz<NG>(d)) & (NG - 1)) * 16);
}

// The score-shaped accumulators of a 32-row block, as a 16-bit B operand over rows:
// chunk c (16 rows) of block `blk` is accumulators 8*(c%2) .. +7 of that block.
template <bool BF16>
__device__ __forceinline__ u32x4 pack_chunk(const f32x16& acc, int half) {
  const int b = half * 8;
  return u32x4{pack2<BF16>(acc[b + 0], acc[b + 1]), pack2<BF16>(acc[b + 2], acc[b + 3]),
               pack2<BF16>(acc[b + 4], acc[b + 5]), pack2<BF16>(acc[b + 6], acc[b + 7])};
}

}  // namespace attn
