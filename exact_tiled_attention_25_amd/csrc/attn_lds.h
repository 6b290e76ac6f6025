// LDS tiles filled by direct HBM->LDS DMA (buffer_load_dwordx4 ... lds) and read as MFMA
// operands, for 16-bit tiles of ROWS tokens x D dims of one (batch, head).
//
// Layout: row-major with padded row pitches, so that every operand read is a per-lane base
// address plus a compile-time offset (no per-read address arithmetic):
//  * K tiles, pitch 2D + 16 bytes: a 16-lane group reading 16 bytes of 16 consecutive rows
//    at the same column hits 16 disjoint 4-bank sets (pitch = 4 banks mod 64).
//  * V tiles, pitch 2D + 64 bytes: read with ds_read_b64_tr_b16. Within each 16-lane group,
//    lane i receives element i%4 of the 8-byte pieces that source lanes 4j + i/4 (j = 0..3)
//    point at; pointing source lane s at row (base + s/4), dims (d0 + 4*(s%4)) hands lane i
//    dim d0 + i of four consecutive rows - an MFMA operand whose contraction runs over rows.
//    A 32-lane half-wave then covers 4 rows x 64 bytes, and a pitch of 16 banks mod 64 puts
//    the 4 rows on disjoint bank sets (the LDS has 64 banks of 4 bytes).
//
// DMA: one wave instruction writes 1 KiB of LDS, lane l's 16 bytes at (M0 base + 16*l); the
// global address of each lane is free. With padded rows, lane slots that fall on padding
// are pointed past the buffer's end and receive zeros. Each lane's global offsets relative
// to the tile's first row are computed once per kernel; per tile only the buffer resource's
// base moves (scalar arithmetic). Rows past the end of the sequence arrive as zeros
// through the buffer range check.
#pragma once
#include "attn_device.h"

namespace attn {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

template <int D> __host__ __device__ constexpr int k_pitch() { return 2 * D + 16; }
template <int D> __host__ __device__ constexpr int v_pitch() { return 2 * D + 64; }

// DMA plan of a ROWS x RB-byte tile with a padded row pitch (constants only; the per-lane
// offsets live in a plain uint32_t[NPW] register array, filled by dma_init and used by
// dma_issue).
template <int RB, int ROWS, int PITCH, int NWAVES>
struct DmaPlanBytes {
  static constexpr int CPRP = PITCH / 16;             // 16-byte slots per padded row
  static constexpr int CPR = RB / 16;                 // data chunks per row
  static constexpr int SLOTS = ROWS * CPRP;
  static constexpr int NI = (SLOTS + 63) / 64;        // wave instructions per tile
  static constexpr int NPW = (NI + NWAVES - 1) / NWAVES;
  static constexpr int BYTES = NI * 1024;             // LDS taken (the last instruction may overhang the tile)
  static_assert(PITCH % 16 == 0 && RB % 16 == 0, "pitch and row must be whole 16-byte slots");
};
// 16-bit elements, D per row.
template <int D, int ROWS, int PITCH, int NWAVES>
using DmaPlan = DmaPlanBytes<2 * D, ROWS, PITCH, NWAVES>;

// Chunk swizzle of an unpadded 16-bit tile (pitch 2D bytes): logical 16-byte chunk c of row
// r is stored at chunk c ^ swz<D>(r). It makes both read patterns conflict-free on the
// 64-bank LDS: row reads (a 16-lane pass: 16 consecutive rows, one chunk) and transpose
// reads (a 32-lane pass: 4 consecutive rows from a multiple of 4, 4 chunks from a multiple
// of 4). d = 128 (256-byte rows, every row starts on bank 0): swz = 4*(r%4) + (r/4)%4,
// a bijection on r%16 whose bits 2-3 move with r%4. d = 64 (128-byte rows alternate bank
// halves): swz = 4*((r/2)%2) + (r/4)%4. SWZ = 0 selects no swizzle.
template <int SWZ>
__host__ __device__ constexpr int swz(int r) {
  return SWZ == 0 ? 0 : SWZ == 64 ? ((((r >> 1) & 1) << 2) | ((r >> 2) & 3)) : (((r & 3) << 2) | ((r >> 2) & 3));
}

// SWAP23: LDS row r holds source row r with bits 2 and 3 exchanged (an involution that
// stays inside each 16-row group), so the rows a transpose read gathers can be made to sit
// at consecutive LDS rows.
__host__ __device__ constexpr int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

template <class Plan, int NWAVES, int SWZ = 0, bool SWAP23 = false>
__device__ __forceinline__ void dma_init(uint32_t* voff, uint32_t row_bytes, int wave, int lane) {
#pragma unroll
  for (int t = 0; t < Plan::NPW; ++t) {
    const int blk = wave + NWAVES * t;
    const int g = blk * 64 + lane;
    const int r = g / Plan::CPRP, cp = g % Plan::CPRP;
    const int src = SWAP23 ? swap23(r) : r;
    voff[t] = (blk < Plan::NI && g < Plan::SLOTS && cp < Plan::CPR) ? (uint32_t)src * row_bytes + (cp ^ swz<SWZ>(r)) * 16
                                                                     : 0x80000000u;
  }
}

// DMA of the tile whose first row is `row0` of the (batch, head) view starting at
// `head_base` (`nrec` bytes valid from there). The buffer resource is built here: a
// resource passed into a function template fails substitution in the host compilation
// pass, which silently drops the kernel's launch stub. Every argument must be provably
// wave-uniform (the resource and the LDS base live in scalar registers); otherwise the
// compiler wraps each load in a loop over the lanes' distinct values.
template <class Plan, int NWAVES>
__device__ __forceinline__ void dma_issue(const uint32_t* voff, char* dst, const char* head_base,
                                          int row0, uint32_t row_bytes, uint32_t nrec, int wave) {
  const uint32_t off = (uint32_t)row0 * row_bytes;
  const auto rs = make_rsrc(head_base + off, nrec - off);
#pragma unroll
  for (int t = 0; t < Plan::NPW; ++t) {
    const int blk = wave + NWAVES * t;
    if (Plan::NI % NWAVES == 0 || blk < Plan::NI)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + blk * 1024), 16, voff[t], 0, 0, 0);
  }
}

// Number of DMA instructions dma_issue makes in wave `wave` for one tile.
template <class Plan, int NWAVES>
__device__ __forceinline__ int dma_count(int wave) {
  return Plan::NI % NWAVES == 0 ? Plan::NPW : (Plan::NI - wave + NWAVES - 1) / NWAVES;
}

// Generic forms for a tile of row pitch PITCH bytes.
// Row reads (MFMA operand over dims): lane base l%32 rows, 16-byte chunk l/32; then
// rows blk*32 + l%32, dims 16*ks + 8*(l/32) .. +7 are at base + blk*32*PITCH + ks*32.
template <int PITCH>
__device__ __forceinline__ int row_lane_off(int lane) { return (lane & 31) * PITCH + (lane >> 5) * 16; }
template <int PITCH>
__device__ __forceinline__ u32x4 lds_row(const char* lane_base, int blk, int ks) {
  return *(const u32x4*)(lane_base + blk * 32 * PITCH + ks * 32);
}
// Transposed reads (MFMA operand over rows): lane l gets dim 32*i + l%32 of rows
// 16*c + 4*hf + {0..3} and 16*c + 8 + 4*hf + {0..3} (hf = l/32), i.e. the rows a 32x32
// accumulator hands to k-slots 0..7 of lane half hf for the 16-row chunk c.
template <int PITCH>
__device__ __forceinline__ int tr_lane_off(int lane) {
  const int i16 = lane & 15, grp = lane >> 4, hf = grp >> 1;
  return (4 * hf + (i16 >> 2)) * PITCH + (16 * (grp & 1) + 4 * (i16 & 3)) * 2;
}
template <int PITCH>
__device__ __forceinline__ u32x4 lds_tr(const char* lane_base, int c, int i) {
  const char* pa = lane_base + c * 16 * PITCH + i * 64;
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)pa);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(pa + 8 * PITCH));
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  return u32x4{ua[0], ua[1], ub[0], ub[1]};
}
// Pitch for tiles read both ways: rows conflict-free, transposed reads 2-way.
template <int D> __host__ __device__ constexpr int rt_pitch() { return 2 * D + 48; }

// Reads of a swizzled tile (pitch 2D) through per-lane offsets computed once per kernel.
// Row reads: lane l, 16-dim step ks, row block blk -> rows 32*blk + l%32, dims 16*ks + 8*(l/32)
// at tile + row_off[ks] + blk*32*2D. Transpose reads (the same operand as lds_tr): chunk-row
// block c, output block i -> tile + tr_off[0][i] + c*16*2D and tile + tr_off[1][i] + c*16*2D.
template <int D>
__device__ __forceinline__ void swz_offsets(int lane, int (&row_off)[D / 16], int (&tr_off)[2][D / 32]) {
  constexpr int RB = 2 * D;
  const int hf = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) row_off[ks] = (lane & 31) * RB + 16 * ((2 * ks + hf) ^ swz<D>(lane & 15));
  const int i16 = lane & 15, g1 = (lane >> 4) & 1;
  const int lo = 2 * g1 + ((i16 & 3) >> 1);   // chunk within the 4-chunk (32-dim) group
#pragma unroll
  for (int sec = 0; sec < 2; ++sec) {
    const int r = 4 * hf + (i16 >> 2) + 8 * sec;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) tr_off[sec][i] = r * RB + 16 * ((4 * i + lo) ^ swz<D>(r)) + 8 * (i16 & 1);
  }
}
__device__ __forceinline__ u32x4 lds_read16(const char* p) { return *(const u32x4*)p; }
__device__ __forceinline__ u32x4 lds_tr_pair(const char* p0, const char* p1) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p0);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p1);
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  return u32x4{ua[0], ua[1], ub[0], ub[1]};
}

// Forward-kernel aliases: K tiles are read as rows, V tiles transposed.
template <int D>
__device__ __forceinline__ int k_lane_off(int lane) { return row_lane_off<k_pitch<D>()>(lane); }
template <int D>
__device__ __forceinline__ u32x4 lds_k(const char* lane_base, int kb, int ks) { return lds_row<k_pitch<D>()>(lane_base, kb, ks); }
template <int D>
__device__ __forceinline__ int v_lane_off(int lane) { return tr_lane_off<v_pitch<D>()>(lane); }
template <int D>
__device__ __forceinline__ u32x4 lds_vt(const char* lane_base, int c, int i) { return lds_tr<v_pitch<D>()>(lane_base, c, i); }

// Output tile of one wave (32 rows of RB bytes: the 16-bit rows of O, dQ, dK or dV) written
// through LDS. The MFMA accumulator hands each lane 8-byte pieces of one row, so a store
// straight from it makes every instruction touch 32 rows, 16 bytes of each. Staged in the
// wave's own LDS area (pitch RB + 16: the 32 rows of one piece write fall on 16 bank offsets,
// two rows each, the least a 512-byte write can take) and read back as 16-byte row chunks,
// each store instruction writes RB-byte rows whole (64 x 16 bytes). The stores carry the
// non-temporal hint (cache-policy bit 1 of a buffer instruction): no kernel here reads its
// own output again. Rows past the end of the buffer resource are dropped by its range check.
template <int RB>
struct RowStage {
  static constexpr int PITCH = RB + 16;
  static constexpr int BYTES = 32 * PITCH;
  static constexpr int CPR = RB / 16;   // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;  // rows per store instruction
  static_assert(RB % 16 == 0 && 64 % CPR == 0, "whole rows per store instruction");
  // the piece of `row` at byte `byte` (8 bytes)
  __device__ static __forceinline__ void put(char* st, int row, int byte, u32x2 v) {
    *(u32x2*)(st + row * PITCH + byte) = v;
  }
  // rows 0..31 of the staged tile to bytes col0 .. col0 + RB - 1 of rows row0.. of the
  // buffer (row_bytes apart); a kernel short of LDS stages its rows in column parts
  __device__ static __forceinline__ void store(const char* st, __amdgpu_buffer_rsrc_t r, uint32_t row0,
                                               uint32_t row_bytes, uint32_t col0, int lane) {
#pragma unroll
    for (int k = 0; k < 32 / RPI; ++k) {
      const int row = k * RPI + lane / CPR, c = lane % CPR;
      __builtin_amdgcn_raw_buffer_store_b128(*(const u32x4*)(st + row * PITCH + c * 16), r,
                                             (row0 + row) * row_bytes + col0 + c * 16, 0, 2);
    }
  }
};

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N of this wave's vector-memory operations are outstanding (the N most
// recent ones may stay in flight across the following barrier).
template <int N>
__device__ __forceinline__ void wait_dma_keep() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier between the tiles of a DMA ring. __syncthreads() is s_barrier between a
// release and an acquire fence, and the compiler completes the release by waiting for every
// LDS DMA in flight (vmcnt(0)), the tiles prefetched further ahead included. This barrier
// takes only what a ring needs: each wave has already waited for its own part of the tile
// the next step reads (wait_dma_keep*); its LDS reads are complete (lgkmcnt(0)) before any
// wave passes, so that no later DMA into a stage overtakes a read of it; and the empty asm
// with a memory clobber keeps the compiler from moving LDS accesses across.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The same for a wave-uniform count 0 <= n <= MAX (s_waitcnt takes an immediate; counts
// above MAX wait as for MAX, which only waits longer).
template <int... I>
__device__ __forceinline__ void wait_dma_keep_sel(int n, std::integer_sequence<int, I...>) {
  ((n == I ? wait_dma_keep<I>() : void()), ...);
}
template <int MAX>
__device__ __forceinline__ void wait_dma_keep_rt(int n) {
  wait_dma_keep_sel(n < MAX ? n : MAX, std::make_integer_sequence<int, MAX + 1>{});
}

}  // namespace attn
