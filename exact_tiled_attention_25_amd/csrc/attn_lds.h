// LDS tiles filled by direct HBM->LDS DMA (buffer_load_dwordx4 ... lds) and read as MFMA
// operands, for 16-bit tiles of ROWS tokens x D dims of one (batch, head).
//
// DMA: one wave instruction writes 1 KiB of LDS, lane l's 16 bytes at (M0 base + 16*l); the
// global address of each lane is free. The tile is stored row-major without padding (row
// pitch 2*D bytes); bank conflicts are avoided by XOR-swizzling the 16-byte chunk index of
// each row: LDS chunk c' of row r holds global chunk c = c' ^ swz(r). Rows past the end of
// the sequence arrive as zeros through the buffer range check.
//
// Two read patterns, each with its own swizzle:
//  * row reads (ds_read_b128): lane l reads 16 bytes of row `r` (rows of a 32-row block go
//    to lanes l%32). swz_row(r) = (r ^ (r >> 3)) & 7 for D = 64, r & 15 otherwise, so any 8
//    or 16 consecutive rows hit distinct banks.
//  * transposed reads (ds_read_b64_tr_b16): within each 16-lane group, lane i receives
//    element i%4 of the 8-byte pieces that source lanes 4j + i/4 (j = 0..3) point at.
//    Pointing source lane s at row (base + s/4) and dims (d0 + 4*(s%4)) hands lane i the
//    column d0 + i of four consecutive rows: an MFMA operand whose contraction runs over
//    rows, read from a row-major tile. A 16-lane group reads 2 chunks of each of 4 rows and
//    the two groups of a half-wave read the next 2 chunks of the same rows; swz_tr(r) =
//    (2j ^ 4j) & 15 (j = r & 3) gives the 4 rows disjoint bank sets both within a group
//    (bits 1-2 distinct) and across the half-wave (bits 2-3 distinct); for d = 64 the
//    128-byte rows already alternate bank halves and 2j suffices.
#pragma once
#include "attn_device.h"

namespace attn {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

template <int D>
__device__ __forceinline__ int swz_row(int r) {
  if constexpr (D == 64) return (r ^ (r >> 3)) & 7;
  else return r & 15;
}
template <int D>
__device__ __forceinline__ int swz_tr(int r) {
  const int j = r & 3;
  if constexpr (D == 64) return 2 * j;
  else return ((2 * j) ^ (4 * j)) & 15;
}

// Byte offset of the 16-byte chunk holding dims [8c, 8c+8) of row r.
template <int D, bool TR>
__device__ __forceinline__ int chunk_off(int r, int c) {
  return r * (2 * D) + ((c ^ (TR ? swz_tr<D>(r) : swz_row<D>(r))) << 4);
}

// DMA one ROWS x D tile (rows row0 .. row0+ROWS-1 of the buffer view) into `dst`.
// Each of the NWAVES waves issues ROWS*2*D/1024/NWAVES instructions.
template <int D, int ROWS, bool TR, int NWAVES>
__device__ __forceinline__ void dma_tile(char* dst, __amdgpu_buffer_rsrc_t rs, int row0, uint32_t row_bytes,
                                         int wave, int lane) {
  constexpr int KIB = ROWS * 2 * D / 1024;
  static_assert(KIB % NWAVES == 0, "tile must split evenly over the waves");
  constexpr int PER = KIB / NWAVES;
  constexpr int NCH = D / 8;  // 16-byte chunks per row
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int blk = wave * PER + it;
    const int byte = blk * 1024 + 16 * lane;
    const int r = byte / (2 * D);
    const int cp = (byte % (2 * D)) >> 4;
    const int c = (cp ^ (TR ? swz_tr<D>(r) : swz_row<D>(r))) & (NCH - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + blk * 1024), 16,
                                             (uint32_t)(row0 + r) * row_bytes + c * 16, 0, 0, 0);
  }
}

// Row read: dims 16*ks + 8*hf .. +7 of row r.
template <int D>
__device__ __forceinline__ u32x4 lds_row(const char* base, int r, int ks, int hf) {
  return *(const u32x4*)(base + chunk_off<D, false>(r, 2 * ks + hf));
}

// Transposed read for O^T += X^T P^T style products: lane l gets dim d0 + (l % 32) of the
// 8 rows  rbase + 4*hf + {0,1,2,3}  and  rbase + 8 + 4*hf + {0,1,2,3}  (hf = l / 32), i.e.
// the rows a 32x32 accumulator hands to k-slots 0..7 of lane half hf for the 16-row chunk
// starting at rbase.
template <int D>
__device__ __forceinline__ u32x4 lds_tr(const char* base, int rbase, int d0, int lane) {
  const int i16 = lane & 15, grp = lane >> 4, hf = grp >> 1;
  const int dcol = d0 + 16 * (grp & 1) + 4 * (i16 & 3);
  const int ra = rbase + 4 * hf + (i16 >> 2);
  const int rb = ra + 8;
  const char* pa = base + chunk_off<D, true>(ra, dcol >> 3) + ((dcol & 7) << 1);
  const char* pb = base + chunk_off<D, true>(rb, dcol >> 3) + ((dcol & 7) << 1);
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)pa);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)pb);
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  return u32x4{ua[0], ua[1], ub[0], ub[1]};
}

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace attn
