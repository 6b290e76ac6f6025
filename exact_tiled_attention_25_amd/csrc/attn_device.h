// Device-side building blocks for the gfx950 attention kernels: vector types, the MFMA
// forms used (32x32x16 bf16/f16, 32x32x64 f8f6f4), buffer resources, packed converts,
// the cross-half lane swap and the XCD-aware block remap.
//
// MFMA register layouts (32x32 output tile, wave64; verified on the hardware):
//   A (32 x K):  lane l holds row  l%32, its K-chunk (l/32); 8 bf16/f16 (or 32 fp8) per lane.
//   B (K x 32):  lane l holds column l%32, the same K-chunk (l/32).
//   C (32 x 32): lane l holds column l%32; accumulator r is row 8*(r/4) + 4*(l/32) + r%4.
// A and B share their per-lane K mapping, so any consistent permutation of the contraction
// index (head dim for Q K^T, keys for P V) is harmless; the kernels rely on that to feed the
// score accumulator straight into the P V product (see attn_fwd.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace attn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// Buffer resource word 3 for raw (untyped) gfx9 buffer accesses: DATA_FORMAT = 32 bit.
// Loads past num_records return zero and stores past it are dropped.
constexpr int kBufWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufWord3);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}

// 32x32x16 MFMA on 16-bit inputs held as 4 dwords per lane.
template <bool BF16>
__device__ __forceinline__ f32x16 mfma32x16(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two floats -> two 16-bit values (round to nearest even) in one dword, first in the low half.
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  f32x2 v = {lo, hi};
  if constexpr (BF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// Combine a lane value with the same lane of the other wave half (lane l ^ 32).
// permlane32_swap(x, x) returns r[0] = (x[0..31], x[0..31]) and r[1] = (x[32..63], x[32..63])
// across the two halves, so r[0] op r[1] is the two-half reduction in every lane.
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A 32-bit value the caller knows to be the same in every lane, made provably wave-uniform
// (scalar): buffer resources and the LDS base of a DMA must live in scalar registers, and
// where the compiler cannot prove uniformity it wraps each such instruction in a loop over
// lanes. (Only for values the compiler cannot see are uniform: forcing an already scalar
// value through readfirstlane can leave a vector copy that other users then pick up.)
__device__ __forceinline__ uint32_t uniform(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// max(max(a, b), c): a running maximum written this way (two new values per step) folds
// into one v_max3_f32 per step; max(a, max(b, c)) pairs the new values first and costs more.
// (Not inline asm: the compiler inserts the wait states that a read or write next to an
// in-flight MFMA needs only for instructions it emits itself.)
__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Workgroups are handed to the 8 XCDs round-robin (block b runs on XCD b % 8). Give each XCD
// a contiguous range of work items so that the query tiles of one head, which read the same
// K and V, share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
  const int q = nblk >> 3, r = nblk & 7;
  const int x = bid & 7, i = bid >> 3;
  return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// Inverse of xcd_remap: the block index that xcd_remap sends to v (0 <= v < n).
__device__ __forceinline__ int xcd_unremap(int v, int n) {
  const int q = n >> 3, r = n & 7;
  const int x = v < r * (q + 1) ? v / (q + 1) : r + (v - r * (q + 1)) / max(q, 1);
  return (v - x * q - min(x, r)) * 8 + x;
}
// (sequence, head) pair of virtual pair index vp. Fixed lengths: vp itself, so the XCD that
// owns a contiguous range of work items runs a few whole heads. Variable lengths: the pairs
// are dealt to the XCDs round-robin (pair p to the XCD range of class p % 8, with the tiles
// of one pair kept together for L2 reuse of its K and V), so that every XCD holds a share of
// every sequence instead of whole sequences of very different lengths.
__device__ __forceinline__ int spread_pair(int vp, int npairs, bool varlen) {
  return varlen ? xcd_unremap(vp, npairs) : vp;
}

// Compile-time loop: f(std::integral_constant<int, I>{}) for I = 0 .. N-1, fully expanded
// (unlike #pragma unroll, which gives up on large bodies and leaves register arrays
// dynamically indexed).
// Ties a value to this point of the instruction stream: the arithmetic that produced it
// cannot be sunk past later scheduling fences (used to keep VALU work under the MFMAs it
// was placed beside).
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(uint32_t& x) { asm volatile("" : "+v"(x)); }
// Makes the compiler wait here for a register loaded from memory. Without it the wait is
// placed at the register's first use; when that use sits inside a loop (the first use
// before the loop being conditional), every iteration executes the wait, and once the loop
// has DMA in flight a vmcnt wait there waits for that DMA as well.
// (The host compilation pass checks asm constraints against x86, where "v" on a 256-bit
// vector is invalid; the statement only matters in the device pass.)
template <class T>
__device__ __forceinline__ void settle(const T& x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::"v"(x));
#else
  (void)x;
#endif
}

// Ties an MFMA accumulator to the accumulation register file (AGPRs). Accumulators that
// live across a whole loop and are only touched by MFMAs belong there; without the hint
// the allocator may park them in VGPRs and copy them over before every MFMA.
__device__ __forceinline__ void pin_acc(f32x16& x) { asm volatile("" : "+a"(x)); }
// ... and an MFMA operand held in registers for a whole loop (MFMAs read AGPR operands).
__device__ __forceinline__ void pin_acc(u32x4& x) { asm volatile("" : "+a"(x)); }

// Sequence b of a batch: its first token row and its length. Fixed-length batches (cu =
// null): b * N and N. Variable-length batches: cu_seqlens[b] and cu_seqlens[b+1] - that.
struct SeqView {
  int start, len;
};
// The offsets are clamped to [0, T] and the length to N (the longest sequence), so that
// malformed offsets give unspecified results but never an access outside the tensors.
__device__ __forceinline__ SeqView seq_view(const int* cu, int b, int N, int T) {
  if (cu == nullptr) return SeqView{b * N, N};
  const int s0 = min(max(cu[b], 0), T);
  const int s1 = min(max(cu[b + 1], s0), T);
  return SeqView{s0, min(s1 - s0, N)};
}
// First element of the per-row statistics (L, D) of sequence b, head h: [B][H][N] for fixed
// lengths, [H][T] for packed variable-length batches.
__device__ __forceinline__ size_t stat_row(const int* cu, int T, int b, int H, int h, const SeqView& sv) {
  return cu == nullptr ? ((size_t)b * H + h) * sv.len : (size_t)h * T + sv.start;
}

template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace attn
